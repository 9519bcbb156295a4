// bf16 matrix-core (MFMA) building blocks of the lm_head path, gfx950.
//
// A workgroup of 4 waves computes a 256 x BN tile of C[m][n] = sum_k A(m, k)
// B(n, k) with v_mfma_f32_32x32x16_bf16: waves 2 x 2, each a 128 x (32 NJ)
// block held as 4 x NJ MFMA accumulators (fp32, 16 per lane each).  K advances
// in slices of 32 that go straight from memory to LDS (buffer loads with the
// LDS-destination bit) through a ring of NS stages: while slice kt is
// multiplied, slices kt + 1 .. kt + NS - 1 are in flight, so a load has NS - 1
// slices of matrix-core time to arrive.
//
// Operand layouts.  A(m, k) = A[m * lda + k] (K-contiguous) or A[k * lda + m]
// (M-contiguous), B likewise.  A K-contiguous operand lands in LDS as rows of
// 64 bytes (the slice's 32 k) whose four 16-byte chunks are XOR-swizzled by
// bits 1-2 and 3 of the row: the 8 (or 16) rows one LDS cycle of a fragment
// read serves then fall on distinct banks whether the LDS serves 128 or 256
// bytes a cycle.  An M/N-contiguous operand (256 rows only) lands as 32 rows of
// 512 bytes, its chunks XOR-swizzled by k, and its fragments are read with the
// gfx950 LDS transpose read (ds_read_b64_tr_b16: in each group of 16 lanes, the
// lane that supplies row j receives element i % 4 of rows 4 s + i / 4, s =
// 0..3), which hands every lane 4 consecutive k of one row or column; two
// reads make the 8 k of an MFMA operand.
//
// MFMA operand and result layout (v_mfma_f32_32x32x16_bf16): for a 32 x 32
// tile at k = ks..ks+15, lane l supplies row (or column) l % 32, k = ks + 8 (l /
// 32) + 0..7 of A (or B); result register r of lane l holds row (r % 4) +
// 4 (l / 32) + 8 (r / 4), column l % 32.
//
// Schedule.  A slice is 2 k-steps of 16; a step is 4 groups, group I being
// the NJ MFMAs of A fragment I.  Every fragment is read from LDS during the
// step before its MFMAs (group I of a step requests A fragment I and B
// fragments 2I, 2I+1 of the next step), so LDS latency hides behind MFMAs.  At the top
// of a slice's last step each wave waits for its share of slice kt + 1 and the
// workgroup meets at a barrier: past it, slice kt + 1 is in LDS and nobody
// reads slice kt's stage any more (its last step's fragments are already in
// registers), so the last step reads the first fragments of slice kt + 1 and
// sends the loads of slice kt + NS into slice kt's stage.  One barrier per
// slice.
//
// Loads past the matrix (ragged M, N, K) get an offset past the buffer
// resource's range and read zeros, with no branch; K and the leading
// dimensions are multiples of 8, so a 16-byte chunk is all in or all out.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ids.hpp"

namespace lx {
namespace mm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kBM = 256;     // tile rows (M)
constexpr int kBK = 32;      // K-slice
constexpr int kSteps = kBK / 16;
constexpr int kThreads = 256;
constexpr int kRsrcFlags = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;  // a load offset past every buffer's range: reads 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const uint16_t* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), (short)0, (int)bytes, kRsrcFlags);
}

// LDS placement of 16-byte chunks (see the header comment).
__device__ __forceinline__ int kc_swizzle(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }
__device__ __forceinline__ int tr_swizzle(int k) { return (k & 3) << 1; }

// One operand's share of a K-slice load: ROWS rows r0.. of the M or N
// dimension, k0..k0+31, into an LDS tile of ROWS * 64 bytes; lane L of wave w
// fills 16 bytes of each of the 1 KB pieces w * kLoads + q.  Everything that
// does not change from slice to slice is computed once per tile; rows past the
// matrix get an out-of-range offset once, and the K bound is checked per
// slice, so slices past the last one load nothing.
template <bool KC, int ROWS>
struct SliceLoader {
  static_assert(KC || ROWS == 256, "M/N-contiguous operands come in 256-row tiles");
  static constexpr int kTileBytes = ROWS * kBK * 2;
  static constexpr int kLoads = kTileBytes / (kThreads * 16);  // 16-byte loads per thread and slice
  static_assert(kLoads >= 1 && kLoads <= 4, "one load per group of a step at most");
  uint32_t off[kLoads];
  int kk[kLoads];
  const uint16_t* P;
  int64_t ld, end;
  int K, r0;

  __device__ __forceinline__ void init(const uint16_t* P_, int64_t ld_, int64_t end_, int rows, int K_, int r0_,
                                       int wave) {
    P = P_;
    ld = ld_;
    end = end_;
    K = K_;
    r0 = r0_;
    const int lane = tid_x() & 63;
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
      const int kb = wave * kLoads + q;
      int r, k;
      if (KC) {
        r = kb * 16 + (lane >> 2);
        const int c = (lane & 3) ^ kc_swizzle(r);
        k = 8 * c;
        off[q] = r0 + r < rows ? (uint32_t)(r * ld + k) * 2u : kOutOfRange;
      } else {
        k = kb * 2 + (lane >> 5);
        const int c = (lane & 31) ^ tr_swizzle(k);
        r = 8 * c;
        off[q] = r0 + r < rows ? (uint32_t)(k * ld + r) * 2u : kOutOfRange;
      }
      kk[q] = k;
    }
  }

  // load q of the slice at k0 into tile T
  __device__ __forceinline__ void issue(int q, uint8_t* T, int k0, int wave) const {
    const int64_t base = KC ? (int64_t)r0 * ld + k0 : (int64_t)k0 * ld + r0;
    const int64_t left = end - 2 * base;
    const uint32_t range = left > 0x7fffffff ? 0x7fffffffu : (uint32_t)(left > 0 ? left : 0);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(P + base, range);
    const uint32_t o = k0 + kk[q] < K ? off[q] : kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(T + (wave * kLoads + q) * 1024), 16, o, 0, 0, 0);
  }
};

// The MFMA fragment of rows rb..rb+31, k = ks..ks+15 of an LDS tile.
template <bool KC>
__device__ __forceinline__ bf16x8_t fragment(const uint8_t* T, int rb, int ks) {
  const int lane = tid_x() & 63;
  if (KC) {
    const int r = rb + (lane & 31);
    const int c = (ks >> 3) + (lane >> 5);
    return *reinterpret_cast<const bf16x8_t*>(T + r * (kBK * 2) + ((c ^ kc_swizzle(r)) << 4));
  } else {
    const int g = lane >> 4, j = lane & 15;
    const int r = rb + 16 * (g & 1) + 4 * (j & 3);
    const int k = ks + 8 * (g >> 1) + (j >> 2);
    typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
    // 4 elements r..r+3 (r % 4 == 0) lie in one chunk; k and k + 4 share k % 4
    const int in_row = (((r >> 3) ^ tr_swizzle(k)) << 4) + (r & 7) * 2;
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(T + k * 512 + in_row));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(T + (k + 4) * 512 + in_row));
    const s16x4_t v8[2] = {lo, hi};
    return __builtin_bit_cast(bf16x8_t, v8);
  }
}

template <int NJ>
struct Frags {
  bf16x8_t a_cur[4], a_nxt[4], b_cur[NJ], b_nxt[NJ];
};

// Wait until at most N of this wave's loads are outstanding and for its LDS
// and scalar reads, then meet the workgroup.  The wait goes through the
// builtin (s_waitcnt fields: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
// 11:8), so the compiler's own wait bookkeeping knows what has retired; the
// empty memory clobbers keep every LDS access on its side of the barrier.
template <int N>
__device__ __forceinline__ void wait_loads_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Group I of k-step S of a slice: request A fragment I and B fragments 2I, 2I+1
// of the next step (in the last step: of the next slice, after the barrier, which
// also sends load I of slice kt + NS to the current stage), then the NJ MFMAs
// of A fragment I.
template <bool AK, bool BK, int NJ, int BROWS, int WAIT, int S, int I>
__device__ __forceinline__ void step(Frags<NJ>& f, f32x16_t (&acc)[4][NJ], const uint8_t* TA, const uint8_t* TB,
                                     const uint8_t* NA, const uint8_t* NB, uint8_t* LA, uint8_t* LB, int wm, int wn,
                                     const SliceLoader<AK, 256>& la, const SliceLoader<BK, BROWS>& lb, int k0n,
                                     int wave) {
  constexpr bool last = S == kSteps - 1;
  if (last && I == 0) wait_loads_barrier<WAIT>();
  // every group needs all B fragments: they come two a group, done by group 1,
  // ahead of the A fragment, so group 0's MFMAs never wait for A fragments 1-3
#pragma unroll
  for (int h = 0; h < 2; ++h)
    if (2 * I + h < NJ) f.b_nxt[2 * I + h] = fragment<BK>(last ? NB : TB, wn + 32 * (2 * I + h), last ? 0 : 16 * (S + 1));
  f.a_nxt[I] = fragment<AK>(last ? NA : TA, wm + 32 * I, last ? 0 : 16 * (S + 1));
  if (last) {
    if (I < SliceLoader<AK, 256>::kLoads) la.issue(I, LA, k0n, wave);
    if (I < SliceLoader<BK, BROWS>::kLoads) lb.issue(I, LB, k0n, wave);
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[I][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a_cur[I], f.b_cur[j], acc[I][j], 0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  if (I == 3) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f.a_cur[i] = f.a_nxt[i];
#pragma unroll
    for (int j = 0; j < NJ; ++j) f.b_cur[j] = f.b_nxt[j];
  }
}

// The whole K loop of one product into acc (4 x NJ accumulators per wave),
// with LDS at `lds`: NS stages of [A tile 16 KB][B tile BROWS * 64 B].
// Leaves LDS free: every load has landed and every wave is past the final
// barrier.
template <bool AK, bool BK, int NJ, int BROWS, int NS>
__device__ __forceinline__ void mainloop(f32x16_t (&acc)[4][NJ], uint8_t* lds, const SliceLoader<AK, 256>& la,
                                         const SliceLoader<BK, BROWS>& lb, int K, int wm, int wn, int wave) {
  static_assert(kSteps == 2, "the schedule below spells out two k-steps per slice");
  constexpr int kAT = SliceLoader<AK, 256>::kTileBytes;
  constexpr int kStage = kAT + SliceLoader<BK, BROWS>::kTileBytes;
  constexpr int kL = SliceLoader<AK, 256>::kLoads + SliceLoader<BK, BROWS>::kLoads;  // loads per slice and thread
  constexpr int kWait = (NS - 2) * kL;  // outstanding past slice kt + 1 at its wait
  static_assert(NS >= 2 && (NS - 1) * kL <= 63, "vmcnt holds 6 bits");
  const int nk = (K + kBK - 1) / kBK;
  // prologue: slices 0 .. NS - 1 into stages 0 .. NS - 1 (those past K load nothing)
#pragma unroll
  for (int s = 0; s < NS; ++s) {
#pragma unroll
    for (int q = 0; q < SliceLoader<AK, 256>::kLoads; ++q) la.issue(q, lds + s * kStage, s * kBK, wave);
#pragma unroll
    for (int q = 0; q < SliceLoader<BK, BROWS>::kLoads; ++q) lb.issue(q, lds + s * kStage + kAT, s * kBK, wave);
  }
  wait_loads_barrier<(NS - 1) * kL>();
  Frags<NJ> f;
  // in the order the first groups use them (B, then A 0..3)
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    f.b_cur[j] = fragment<BK>(lds + kAT, wn + 32 * j, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f.a_cur[i] = fragment<AK>(lds, wm + 32 * i, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  int cur = 0;
  for (int kt = 0; kt < nk; ++kt) {
    const int nxt = cur + 1 == NS ? 0 : cur + 1;
    uint8_t* T = lds + cur * kStage;
    uint8_t* N = lds + nxt * kStage;
    const int k0n = (kt + NS) * kBK;
#define LX_STEP(S, I) \
  step<AK, BK, NJ, BROWS, kWait, S, I>(f, acc, T, T + kAT, N, N + kAT, T, T + kAT, wm, wn, la, lb, k0n, wave)
    LX_STEP(0, 0); LX_STEP(0, 1); LX_STEP(0, 2); LX_STEP(0, 3);
    LX_STEP(1, 0); LX_STEP(1, 1); LX_STEP(1, 2); LX_STEP(1, 3);
#undef LX_STEP
    cur = nxt;
  }
  // the loads of the slices past K (all out of range) and the last step's
  // reads (of a stage nobody filled) are still outstanding
  wait_loads_barrier<0>();
}

// Row (within the 32 x 32 MFMA tile) of result register r of lane `lane`.
__device__ __forceinline__ int acc_row(int r, int lane) { return (r & 3) + 4 * (lane >> 5) + 8 * (r >> 2); }

// XCD-aware tile order: workgroup id i runs on XCD i % 8; tiles are dealt to
// the XCDs in contiguous runs, and within a run they go in groups of
// kGroupM M-tiles sweeping N, so the tiles an XCD runs at once share their A
// and B slices in that XCD's L2.  Returns false for a workgroup past the end.
constexpr int kXcds = 8;
constexpr int kGroupM = 4;
__device__ __forceinline__ bool tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  const int tiles = tiles_m * tiles_n;
  const int per_xcd = (tiles + kXcds - 1) / kXcds;
  const int tile = (int)(bid_x() % kXcds) * per_xcd + (int)(bid_x() / kXcds);
  if (tile >= tiles) return false;
  const int per_group = kGroupM * tiles_n;
  const int group = tile / per_group;
  const int gm = min(kGroupM, tiles_m - group * kGroupM);
  const int in_group = tile - group * per_group;
  tm = group * kGroupM + in_group % gm;
  tn = in_group / gm;
  return true;
}

inline unsigned grid_for(int tiles_m, int tiles_n) {
  const int tiles = tiles_m * tiles_n;
  const int per_xcd = (tiles + kXcds - 1) / kXcds;
  return (unsigned)(per_xcd * kXcds);
}

}  // namespace mm
}  // namespace lx
