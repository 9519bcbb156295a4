// bf16 matrix products on the matrix cores (MFMA) for the linear + CE + TVD
// path: the logits of an lm_head (X W^T), and the gradients of the hidden
// states (G W) and of the weight (G^T X) from the logits' gradient G.
//
// One kernel computes C[m][n] (+)= sum_k A(m, k) * B(n, k) for bf16 A and B
// and fp32 C, with A(m, k) stored at A[m * lda + k] (AK: K-contiguous) or at
// A[k * lda + m], and B(n, k) at B[n * ldb + k] (BK) or at B[k * ldb + n]:
//
//   logits  z = X W^T : A = X (AK),   B = W (BK),   K = hidden size
//   grad X  dX = G W  : A = G (AK),   B = W (!BK),  K = vocabulary
//   grad W  dW = G^T X: A = G (!AK),  B = X (!BK),  K = rows
//
// Workgroup tile 256 x 256, four waves of 128 x 128 (2 x 2), each wave a
// 4 x 4 grid of v_mfma_f32_32x32x16_bf16 with its accumulators in AGPRs, one
// workgroup per compute unit (the accumulators take all 256 AGPRs).  K
// advances in slices of 64 that go straight from memory to LDS (buffer loads
// with the LDS-destination bit: no staging registers), double buffered
// (2 x 2 x 32 KB): the next slice loads while the current one is multiplied.
// A K-contiguous operand lands as 256 rows of 128 bytes whose eight 16-byte
// chunks are XOR-swizzled by the row (kc_swizzle), so a fragment read
// spreads over the banks; an M- or N-contiguous operand lands as 64 rows of
// 512 bytes, its chunks XOR-swizzled by k (tr_swizzle), and its
// fragments are read with the gfx950 LDS transpose read (ds_read_b64_tr_b16:
// in each group of 16 lanes, the lane that supplies row j receives element
// i % 4 of rows 4 s + i / 4, s = 0..3), which hands every lane 4 consecutive
// k of one row or column: two reads make the 8 k of an MFMA operand.  Each
// group of 4 MFMAs is preceded by the LDS reads of the fragments the next
// group needs.  The loads' addresses are computed once per tile (only the
// slice base and the K bound change per slice); the next slice's loads go out
// with the first four MFMA groups when both operands are K-contiguous (38-40%
// instead of 37%), and all before the first group when one is transposed
// (spreading them over the slice drops those products to 12-24%: the strided
// rows miss L2 more, and late loads stall the end-of-slice wait).  Loads past the matrix (ragged M, N, K) get an offset past the
// buffer's range and read zeros, with no branch.
//
// Tiles are dealt to the XCDs in contiguous runs (the hardware hands
// workgroup ids to the 8 XCDs round robin), and within a run they go in
// groups of 4 M-tiles sweeping N, so the ~32 tiles an XCD runs at once (4 x 8)
// share their A and B slices in that XCD's L2.
//
// Measured on the 4096 x 151936 x 4096 logits product: 37% of the dense bf16
// peak on random data (47% on zeros: the matrix cores draw less power), 78%
// with the global loads switched off (the pure MFMA + LDS-read ceiling of this
// structure); counters put the L2 hit rate at 77% (the compulsory misses of
// 4 x 8 tile groups) and the waves waiting on the loads a third of the time.
// Tried and not kept: a 4-stage ring of 32-wide K-slices (loads three slices
// ahead; 32%) and a 3-stage ring of 48-wide K-slices (30%): deeper rings of
// narrower slices lose, so the loads' latency is not what limits this kernel;
// staging through registers with transposing LDS writes (35%).
//
// Requirements (checked on the host): the contiguous dimension of every
// operand is a multiple of 8 elements and every row starts on a 16-byte
// boundary; M, N, K >= 1.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm.hpp"
#include "ids.hpp"

namespace lx {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kStages = 2;                       // K-slices in LDS: the next one loads while one is multiplied
constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr int kGroupM = 4;                       // tiles per group along M (tile order)
constexpr int kTileBytes = 256 * kBK * 2;       // one operand's K-slice: 32 KB
constexpr int kLoads = kTileBytes / (kThreads * 16);  // 16-byte loads per thread per operand and slice
constexpr int kRsrcFlags = 0x00020000;           // buffer resource word 3 for gfx9-family raw buffers
constexpr uint32_t kOutOfRange = 0x80000000u;    // a load offset past every buffer's range: reads 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const uint16_t* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), (short)0, (int)bytes, kRsrcFlags);
}

// LDS placement of 16-byte chunks.  K-contiguous tiles (rows of 128 bytes):
// chunk c of row r sits in slot c ^ (r % 8), so 8 consecutive rows of a
// fragment read (same chunk) land on distinct banks (c ^ ((r / 2) % 8), which
// spreads 16 rows, measured the same within run-to-run variation).  M/N-contiguous
// tiles (rows of 512 bytes, one per k): chunk c of row k sits in slot
// c ^ (2 (k % 4)), so the four k rows a 16-lane transpose read touches (two
// neighbouring chunks each) land on distinct banks instead of the same ones
// (the grad-w product, both operands transposed: 8.54 -> 8.14 ms).
__device__ __forceinline__ int kc_swizzle(int r) { return r & 7; }
__device__ __forceinline__ int tr_swizzle(int k) { return (k & 3) << 1; }

// One operand's share of a K-slice load (256 rows r0.. of the M or N
// dimension, k0..k0+63, into an LDS tile), split so that everything that does
// not change from slice to slice is computed once per tile: lane L of wave w
// fills 16 bytes of each of the 1 KB pieces w * 8 + q of the 32 KB tile.
//   K-contiguous: 8 rows of 128 bytes per KB, lane L fills slot L % 8 of row
//   kb * 8 + L / 8 (the chunk that belongs there, kc_swizzle);
//   otherwise: 2 rows of 512 bytes per KB, lane L fills slot L % 32 of row
//   kb * 2 + L / 32 (tr_swizzle).
// Rows past the matrix get an out-of-range offset (zeros, no access) once;
// the K bound is checked per slice, so the slice past the last one loads
// nothing at all.
template <bool KC>
struct SliceLoader {
  uint32_t off[kLoads];  // byte offset from the slice base, or kOutOfRange
  int kk[kLoads];        // k of this lane's 16 bytes within the slice
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
        const int c = (lane & 7) ^ kc_swizzle(r);
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

  // load q of slice k0 into tile T (T and the 1 KB piece are wave-uniform)
  __device__ __forceinline__ void issue(int q, uint8_t* T, int k0, int wave) const {
    const int64_t base = KC ? (int64_t)r0 * ld + k0 : (int64_t)k0 * ld + r0;
    const int64_t left = end - 2 * base;
    const uint32_t range = left > 0x7fffffff ? 0x7fffffffu : (uint32_t)(left > 0 ? left : 0);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(P + base, range);
    const uint32_t o = k0 + kk[q] < K ? off[q] : kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(T + (wave * kLoads + q) * 1024), 16, o, 0, 0, 0);
  }
};

// The MFMA fragment of rows rb..rb+31 (M or N), k = ks..ks+15: lane l gets row
// rb + l % 32, k = ks + 8 (l / 32) + 0..7.
template <bool KC>
__device__ __forceinline__ bf16x8_t fragment(const uint8_t* T, int rb, int ks) {
  const int lane = tid_x() & 63;
  if (KC) {
    const int r = rb + (lane & 31);
    const int c = (ks >> 3) + (lane >> 5);
    return *reinterpret_cast<const bf16x8_t*>(T + r * 128 + ((c ^ kc_swizzle(r)) << 4));
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

struct Frags {
  bf16x8_t a_cur, a_nxt, b_cur[4], b_nxt[4];
};

// One group of 4 MFMAs: A fragment I of the 16-wide k step S against the
// step's 4 B fragments.  Before the group, the next A fragment (I + 1, or
// fragment 0 of step S + 1) and B fragment I of step S + 1 are requested, so
// their LDS latency hides behind the group's MFMAs; the scheduling barriers
// keep that order (the compiler would otherwise read each fragment just
// before its first use, to save registers, and stall on every read).
template <bool AK, bool BK, int S, int I>
__device__ __forceinline__ void step(Frags& f, f32x16_t (&acc)[4][4], const uint8_t* TA, const uint8_t* TB, int wm,
                                     int wn, const SliceLoader<AK>& la, const SliceLoader<BK>& lb, uint8_t* NA,
                                     uint8_t* NB, int k0n, int wave) {
  constexpr bool has_a = I < 3 || S < 3;
  constexpr bool has_b = S < 3;
  constexpr int reads = (has_a ? (AK ? 1 : 2) : 0) + (has_b ? (BK ? 1 : 2) : 0);
  if (has_a) f.a_nxt = fragment<AK>(TA, I < 3 ? wm + 32 * (I + 1) : wm, I < 3 ? 16 * S : 16 * (S + 1));
  if (has_b) f.b_nxt[I] = fragment<BK>(TB, wn + 32 * I, 16 * (S + 1));
  // both operands K-contiguous: the next slice's 16 loads go out with the
  // first 4 groups (4 each: 2 of A, 2 of B), early enough to land before the
  // slice ends; otherwise they all went out before the first group (loop body)
  constexpr bool spread = AK && BK;
  if (spread && S == 0) {
    la.issue(2 * I, NA, k0n, wave);
    lb.issue(2 * I, NB, k0n, wave);
    la.issue(2 * I + 1, NA, k0n, wave);
    lb.issue(2 * I + 1, NB, k0n, wave);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[I][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a_cur, f.b_cur[j], acc[I][j], 0, 0, 0);
  if (reads) __builtin_amdgcn_sched_group_barrier(0x100, reads, 0);  // DS reads
  if (spread && S == 0) __builtin_amdgcn_sched_group_barrier(0x020, 4, 0);  // the loads
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);                  // then the MFMAs
  if (has_a) f.a_cur = f.a_nxt;
  if (I == 3 && has_b) {
#pragma unroll
    for (int j = 0; j < 4; ++j) f.b_cur[j] = f.b_nxt[j];
  }
}

template <bool AK, bool BK, bool ACC>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(const uint16_t* __restrict__ A, int64_t lda, int64_t a_end, const uint16_t* __restrict__ B,
                      int64_t ldb, int64_t b_end, float* __restrict__ C, int64_t ldc, int M, int N, int K,
                      int tiles_m, int tiles_n, int tiles) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kStages * kTileBytes];  // A stages, then B stages

  // XCD-contiguous tile order: workgroup id i runs on XCD i % 8; within an
  // XCD, groups of kGroupM M-tiles sweep N, so the tiles that run together
  // share A and B slices in that XCD's L2
  const int per_xcd = (tiles + kXcds - 1) / kXcds;
  const int tile = (int)(bid_x() % kXcds) * per_xcd + (int)(bid_x() / kXcds);
  if (tile >= tiles) return;
  const int per_group = kGroupM * tiles_n;
  const int group = tile / per_group;
  const int gm = min(kGroupM, tiles_m - group * kGroupM);  // M-tiles in this (possibly last, short) group
  const int in_group = tile - group * per_group;
  const int m0 = (group * kGroupM + in_group % gm) * kBM;
  const int n0 = (in_group / gm) * kBN;

  const int lane = tid_x() & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid_x() >> 6);
  const int wm = (wave & 1) * 128, wn = (wave >> 1) * 128;

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16_t){};

  SliceLoader<AK> la;
  SliceLoader<BK> lb;
  la.init(A, lda, a_end, M, K, m0, wave);
  lb.init(B, ldb, b_end, N, K, n0, wave);
  const int nk = (K + kBK - 1) / kBK;
#pragma unroll
  for (int q = 0; q < kLoads; ++q) {
    la.issue(q, lds, 0, wave);
    lb.issue(q, lds + kStages * kTileBytes, 0, wave);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    const uint8_t* TA = lds + st * kTileBytes;
    const uint8_t* TB = lds + (kStages + st) * kTileBytes;
    // the next slice goes to the other stage, free since the barrier that
    // ended slice kt - 1; past the last slice every load is out of range
    uint8_t* NA = lds + (st ^ 1) * kTileBytes;
    uint8_t* NB = lds + (kStages + (st ^ 1)) * kTileBytes;
    const int k0n = (kt + 1) * kBK;
    if (!(AK && BK)) {  // a transposed operand: the whole next slice is requested before any MFMA
#pragma unroll
      for (int q = 0; q < kLoads; ++q) {
        la.issue(q, NA, k0n, wave);
        lb.issue(q, NB, k0n, wave);
      }
    }
    // Fragments run one step ahead of the MFMAs that use them, and the next
    // slice's 16 loads go out with the first groups of MFMAs (see step()).
    Frags f;
    f.a_cur = fragment<AK>(TA, wm, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) f.b_cur[j] = fragment<BK>(TB, wn + 32 * j, 0);
#define LX_STEP(S, I) step<AK, BK, S, I>(f, acc, TA, TB, wm, wn, la, lb, NA, NB, k0n, wave)
    LX_STEP(0, 0); LX_STEP(0, 1); LX_STEP(0, 2); LX_STEP(0, 3);
    LX_STEP(1, 0); LX_STEP(1, 1); LX_STEP(1, 2); LX_STEP(1, 3);
    LX_STEP(2, 0); LX_STEP(2, 1); LX_STEP(2, 2); LX_STEP(2, 3);
    LX_STEP(3, 0); LX_STEP(3, 1); LX_STEP(3, 2); LX_STEP(3, 3);
#undef LX_STEP
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // slice kt + 1 has landed
    __syncthreads();
  }

  // register r of lane l holds row (r % 4) + 4 * (l / 32) + 8 * (r / 4), column l % 32 of each 32 x 32 tile
  // (accumulating: the 16 values of a 32 x 32 tile are all read before any is
  // written back, so the reads are in flight together)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn + 32 * j + (lane & 31);
      float old[16];
      if (ACC) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm + 32 * i + (r & 3) + 4 * (lane >> 5) + 8 * (r >> 2);
          old[r] = (m < M && n < N) ? C[(int64_t)m * ldc + n] : 0.0f;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm + 32 * i + (r & 3) + 4 * (lane >> 5) + 8 * (r >> 2);
        if (m < M && n < N) C[(int64_t)m * ldc + n] = ACC ? old[r] + acc[i][j][r] : acc[i][j][r];
      }
    }
  }
}

template <bool AK, bool BK, bool ACC>
hipError_t launch_t(const GemmArgs& g, hipStream_t st) {
  const int tiles_m = (int)((g.M + kBM - 1) / kBM);
  const int tiles_n = (int)((g.N + kBN - 1) / kBN);
  const int tiles = tiles_m * tiles_n;
  const int per_xcd = (tiles + kXcds - 1) / kXcds;
  // bytes from each operand's start to the end of its last stored row
  const int64_t a_end = 2 * (AK ? (g.M - 1) * g.lda + g.K : (g.K - 1) * g.lda + g.M);
  const int64_t b_end = 2 * (BK ? (g.N - 1) * g.ldb + g.K : (g.K - 1) * g.ldb + g.N);
  hipLaunchKernelGGL((gemm_bf16_kernel<AK, BK, ACC>), dim3((unsigned)(per_xcd * kXcds)), dim3(kThreads), 0, st,
                     g.A, g.lda, a_end, g.B, g.ldb, b_end, g.C, g.ldc, (int)g.M, (int)g.N, (int)g.K, tiles_m, tiles_n,
                     tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t st) {
  (void)hipGetLastError();
  if (g.a_kc) {
    if (g.b_kc) return g.accumulate ? launch_t<true, true, true>(g, st) : launch_t<true, true, false>(g, st);
    return g.accumulate ? launch_t<true, false, true>(g, st) : launch_t<true, false, false>(g, st);
  }
  if (g.b_kc) return g.accumulate ? launch_t<false, true, true>(g, st) : launch_t<false, true, false>(g, st);
  return g.accumulate ? launch_t<false, false, true>(g, st) : launch_t<false, false, false>(g, st);
}

}  // namespace lx
