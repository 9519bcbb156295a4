// bf16 matrix-core (MFMA) building blocks of the lm_head path, gfx950.
//
// A workgroup of NT / 64 waves (4, or 8 for two waves per SIMD) computes a
// 256 x BN tile of C[m][n] = sum_k A(m, k) B(n, k) with
// v_mfma_f32_32x32x16_bf16: waves 2 x (NT / 128), each a 128 x (32 NJ) block
// held as 4 x NJ MFMA accumulators (fp32, 16 per lane each).  K advances
// in slices of 64.  A slice travels memory -> registers -> LDS: while slice kt
// is multiplied out of one LDS stage, each thread writes its share of slice
// kt + 1 (loaded during slice kt - 1) into the other stage and, piece by
// piece, loads its share of slice kt + 2 into the registers just written out.
// A load thus has a whole slice of matrix-core time to arrive, and the loads
// and LDS writes are spread evenly over the slice, which keeps the memory
// pipeline of the compute unit from stalling the in-order waves.  (Sent
// straight from memory to LDS, the same slices streamed measurably slower on
// MI355X, and slices of 32 k, which fetch half of each 128-byte line per
// request, slower again.)
//
// Operand layouts.  A(m, k) = A[m * lda + k] (K-contiguous) or A[k * lda + m]
// (M-contiguous), B likewise.  A K-contiguous operand lands in LDS as rows of
// 128 bytes (the slice's 64 k) whose eight 16-byte chunks are XOR-swizzled by
// (r ^ r / 8) % 8: the rows one LDS cycle of a fragment read serves fall on
// distinct banks whether the LDS serves 8 or 16 lanes of 16 bytes a cycle
// (measured: no bank conflicts).  An M/N-contiguous operand (256 rows only)
// lands as 64 rows of 512 bytes, its chunks XOR-swizzled by k, and its
// fragments are read with the gfx950 LDS transpose read (ds_read_b64_tr_b16:
// in each group of 16 lanes, the lane that supplies row j receives element
// i % 4 of rows 4 s + i / 4, s = 0..3), which hands every lane 4 consecutive
// k of one row or column; two reads make the 8 k of an MFMA operand.
//
// MFMA operand and result layout (v_mfma_f32_32x32x16_bf16): for a 32 x 32
// tile at k = ks..ks+15, lane l supplies row (or column) l % 32, k = ks + 8 (l /
// 32) + 0..7 of A (or B); result register r of lane l holds row (r % 4) +
// 4 (l / 32) + 8 (r / 4), column l % 32.
//
// Schedule.  A slice is 4 k-steps of 16; a step is 4 groups, group I being
// the NJ MFMAs of A fragment I.  Every fragment is read from LDS during the
// step before its MFMAs (group I of a step requests B fragments 2I, 2I+1 and
// A fragment I of the next step), so LDS latency hides behind MFMAs.  The
// groups of steps 0-2 write the slice-(kt + 1) pieces and load the
// slice-(kt + 2) pieces.  At the top of step 3 every wave waits for its own LDS
// writes and the workgroup meets at a barrier: past it, slice kt + 1 is in LDS
// and nobody reads slice kt's stage any more (its step-3 fragments are already
// in registers), so step 3 reads the first fragments of slice kt + 1.  One
// barrier per slice.
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
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBM = 256;  // tile rows (M)
constexpr int kBK = 64;   // K-slice
constexpr int kThreads = 256;
constexpr int kRsrcFlags = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;  // a load offset past every buffer's range: reads 0
constexpr int kStoreGroups = 12;               // groups (steps 0-2) that carry the slice traffic

// LDS placement of 16-byte chunks (see the header comment).
__device__ __forceinline__ int kc_swizzle(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int tr_swizzle(int k) { return (k & 3) << 1; }

// One operand's share of a K-slice: ROWS rows r0.. of the M or N dimension,
// k0..k0+63, as an LDS tile of ROWS * 128 bytes; lane L of wave w moves 16
// bytes of each of the 1 KB pieces w * kLoads + q.  Everything that does not
// change from slice to slice is computed once per tile; rows past the matrix
// get an out-of-range offset once, and the K bound is checked per slice, so
// slices past the last one load zeros.
template <bool KC, int ROWS, int NT = kThreads>
struct SliceLoader {
  static_assert(KC || ROWS == 256, "M/N-contiguous operands come in 256-row tiles");
  static constexpr int kTileBytes = ROWS * kBK * 2;
  static constexpr int kLoads = kTileBytes / (NT * 16);  // 16-byte pieces per thread and slice
  static_assert(kLoads >= 1 && kLoads * NT * 16 == kTileBytes, "whole 1 KB pieces per wave");
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
        r = kb * 8 + (lane >> 3);
        k = 8 * ((lane & 7) ^ kc_swizzle(r));
        off[q] = r0 + r < rows ? (uint32_t)(r * ld + k) * 2u : kOutOfRange;
      } else {
        k = kb * 2 + (lane >> 5);
        r = 8 * ((lane & 31) ^ tr_swizzle(k));
        off[q] = r0 + r < rows ? (uint32_t)(k * ld + r) * 2u : kOutOfRange;
      }
      kk[q] = k;
    }
  }

  // the buffer resource of the slice at k0 (the offsets are relative to its base)
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(int k0) const {
    const int64_t base = KC ? (int64_t)r0 * ld + k0 : (int64_t)k0 * ld + r0;
    const int64_t left = end - 2 * base;
    const uint32_t range = left > 0x7fffffff ? 0x7fffffffu : (uint32_t)(left > 0 ? left : 0);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(P + base), (short)0, (int)range, kRsrcFlags);
  }
  // piece q of the slice at k0, from memory into registers
  __device__ __forceinline__ u32x4_t load(const __amdgpu_buffer_rsrc_t& rs, int q, int k0) const {
    const uint32_t o = k0 + kk[q] < K ? off[q] : kOutOfRange;
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, 0));
  }
  // piece q from registers into tile T
  __device__ __forceinline__ void store(uint8_t* T, int q, int wave, const u32x4_t& v) const {
    *reinterpret_cast<u32x4_t*>(T + (wave * kLoads + q) * 1024 + (tid_x() & 63) * 16) = v;
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

// A thread's share of one slice in registers.
template <int LA, int LB>
struct Staged {
  u32x4_t a[LA], b[LB];
};

// Wait for this wave's LDS accesses (and scalar loads), then meet the
// workgroup.  The wait goes through the builtin (s_waitcnt fields: vmcnt bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8), so the compiler's own wait
// bookkeeping knows what has retired; the empty memory clobbers keep every LDS
// access on its side of the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt not waited for
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Group I of k-step S of a slice (see the schedule in the header comment).
template <bool AK, bool BK, int NJ, int BROWS, int NT, int MEM, int S, int I>
__device__ __forceinline__ void step(Frags<NJ>& f, f32x16_t (&acc)[4][NJ],
                                     Staged<SliceLoader<AK, 256, NT>::kLoads, SliceLoader<BK, BROWS, NT>::kLoads>& st,
                                     const uint8_t* T, uint8_t* NX, int wm, int wn,
                                     const SliceLoader<AK, 256, NT>& la, const SliceLoader<BK, BROWS, NT>& lb,
                                     const __amdgpu_buffer_rsrc_t& ra, const __amdgpu_buffer_rsrc_t& rb, int k2,
                                     int wave) {
  constexpr int kAT = SliceLoader<AK, 256, NT>::kTileBytes;
  constexpr int kLA = SliceLoader<AK, 256, NT>::kLoads, kLB = SliceLoader<BK, BROWS, NT>::kLoads;
  constexpr int kP = kLA + kLB;  // pieces per thread and slice
  constexpr int G = S * 4 + I;
  if (S == 3 && I == 0) lds_barrier();
  const uint8_t* src = S == 3 ? NX : T;
  const int ks = S == 3 ? 0 : 16 * (S + 1);
  // every group needs all B fragments: they come two a group, done by group 1,
  // ahead of the A fragment, so group 0's MFMAs never wait for A fragments 1-3
#pragma unroll
  for (int h = 0; h < 2; ++h)
    if (2 * I + h < NJ) f.b_nxt[2 * I + h] = fragment<BK>(src + kAT, wn + 32 * (2 * I + h), ks);
  f.a_nxt[I] = fragment<AK>(src, wm + 32 * I, ks);
  if (G < kStoreGroups) {
    // pieces [G kP / 12, (G + 1) kP / 12): A's first, then B's
#pragma unroll
    for (int p = G * kP / kStoreGroups; p < (G + 1) * kP / kStoreGroups; ++p) {
      if (p < kLA) {
        la.store(NX, p, wave, st.a[p]);
        st.a[p] = la.load(ra, p, k2);
      } else {
        lb.store(NX + kAT, p - kLA, wave, st.b[p - kLA]);
        st.b[p - kLA] = lb.load(rb, p - kLA, k2);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[I][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a_cur[I], f.b_cur[j], acc[I][j], 0, 0, 0);
  // issue order inside the group: each MFMA followed by up to two memory
  // instructions (LDS reads and writes, global loads), so the in-order wave
  // never holds several MFMAs back behind a burst of memory instructions
  // (6-7% faster than letting the compiler put the group's memory
  // instructions first)
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100 | 0x200 | 0x020, MEM, 0);  // LDS reads / writes, VMEM reads
  }
  __builtin_amdgcn_sched_group_barrier(0x100 | 0x200 | 0x020, 8, 0);
  __builtin_amdgcn_sched_barrier(0);
  if (I == 3) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f.a_cur[i] = f.a_nxt[i];
#pragma unroll
    for (int j = 0; j < NJ; ++j) f.b_cur[j] = f.b_nxt[j];
  }
}

// The whole K loop of one product into acc (4 x NJ accumulators per wave),
// with LDS at `lds`: 2 stages of [A tile 32 KB][B tile BROWS * 128 B].
// Leaves LDS free: every load and LDS access has retired and every wave is
// past the final barrier.
template <bool AK, bool BK, int NJ, int BROWS, int NT = kThreads, int MEM = 2>
__device__ __forceinline__ void mainloop(f32x16_t (&acc)[4][NJ], uint8_t* lds, const SliceLoader<AK, 256, NT>& la,
                                         const SliceLoader<BK, BROWS, NT>& lb, int K, int wm, int wn, int wave) {
  constexpr int kAT = SliceLoader<AK, 256, NT>::kTileBytes;
  constexpr int kStage = kAT + SliceLoader<BK, BROWS, NT>::kTileBytes;
  constexpr int kLA = SliceLoader<AK, 256, NT>::kLoads, kLB = SliceLoader<BK, BROWS, NT>::kLoads;
  const int nk = (K + kBK - 1) / kBK;
  Staged<kLA, kLB> st;
  {
    // slice 0 into stage 0, slice 1 into registers
    const __amdgpu_buffer_rsrc_t ra = la.rsrc(0), rb = lb.rsrc(0);
#pragma unroll
    for (int q = 0; q < kLA; ++q) st.a[q] = la.load(ra, q, 0);
#pragma unroll
    for (int q = 0; q < kLB; ++q) st.b[q] = lb.load(rb, q, 0);
#pragma unroll
    for (int q = 0; q < kLA; ++q) la.store(lds, q, wave, st.a[q]);
#pragma unroll
    for (int q = 0; q < kLB; ++q) lb.store(lds + kAT, q, wave, st.b[q]);
    const __amdgpu_buffer_rsrc_t ra1 = la.rsrc(kBK), rb1 = lb.rsrc(kBK);
#pragma unroll
    for (int q = 0; q < kLA; ++q) st.a[q] = la.load(ra1, q, kBK);
#pragma unroll
    for (int q = 0; q < kLB; ++q) st.b[q] = lb.load(rb1, q, kBK);
  }
  lds_barrier();
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
  for (int kt = 0; kt < nk; ++kt) {
    const uint8_t* T = lds + (kt & 1) * kStage;
    uint8_t* NX = lds + ((kt & 1) ^ 1) * kStage;
    const int k2 = (kt + 2) * kBK;
    const __amdgpu_buffer_rsrc_t ra = la.rsrc(k2), rb = lb.rsrc(k2);
#define LX_STEP(S, I) step<AK, BK, NJ, BROWS, NT, MEM, S, I>(f, acc, st, T, NX, wm, wn, la, lb, ra, rb, k2, wave)
    LX_STEP(0, 0); LX_STEP(0, 1); LX_STEP(0, 2); LX_STEP(0, 3);
    LX_STEP(1, 0); LX_STEP(1, 1); LX_STEP(1, 2); LX_STEP(1, 3);
    LX_STEP(2, 0); LX_STEP(2, 1); LX_STEP(2, 2); LX_STEP(2, 3);
    LX_STEP(3, 0); LX_STEP(3, 1); LX_STEP(3, 2); LX_STEP(3, 3);
#undef LX_STEP
  }
  // the last loads (past K, unused), writes and reads retire before LDS is reused
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Makes a kernel argument live in scalar registers from this point on.  An
// argument that only the epilogue reads would otherwise be fetched by a
// scalar load the compiler may sink into the main loop's preheader, and a
// scalar load still in flight at the loop's head (scalar loads may return out
// of order) makes the first MFMA of every slice wait for all LDS reads.
template <class T>
__device__ __forceinline__ void pin_scalar(const T& v) {
  asm volatile("" ::"s"(v));
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
