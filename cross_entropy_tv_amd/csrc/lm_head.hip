// The lm_head product and the CE + TVD loss together, on the matrix cores,
// with the logits kept on chip.
//
// The aibars.net Liger-Kernel project page lists a fused linear
// cross-entropy among its kernels (the lm_head projection and the loss in one
// operation, so the full logits are never kept); the Liger-Kernel PR #1384
// analysis page describes the CE + TVD loss ("Forward Pass", "Backward Pass").
// For student hidden states X_s (BT, H_s), student weight W_s (V, H_s) and
// teacher X_t, W_t, with logits z = X_s W_s^T and u = X_t W_t^T:
//
//   pass 1 (stats)  every 256 x 256 tile of z (then of u) is computed on the
//                   matrix cores and reduced in registers to per-row (max,
//                   sum-exp) partials; the target logit z_t = x . w_t comes
//                   from a per-row dot product; the tiles' partials are merged
//                   like column shards of the vocabulary (in a fixed order:
//                   eight contiguous tile ranges, then the ranges) -> lse_s,
//                   lse_t, ce;
//   pass 2 (TV)     256 x 128 tiles of z and u together are computed again and
//                   reduced to per-row
//                   (sum |p - q|, sum p * sign(p - q)) partials, merged the same
//                   way -> tvd, sigma; when gradients are wanted the pass also
//                   writes 2^15 p as binary16 with the sign of p - q in its sign
//                   bit, and a bit per logit marking exact ties (sign 0);
//   G               from those, the per-row sigma and the target logit:
//                   G = k (g_ce (p - [v == t]) + g_tvd / 2 * p (s - sigma)), bf16
//                   (rounded to nearest even), written over the binary16 p;
//   grad_x = G W_s  and  grad_w = G^T X_s on the matrix cores, reading G, W_s
//                   and X_s as they lie (W_s in grad_x, and G and X_s in
//                   grad_w, down their columns: the main loop's transposing
//                   LDS reads), so nothing is transposed in memory.
//
// z and u never reach memory: each pass recomputes its tiles from X and W
// (every element is accumulated over k in the same order by the same main
// loop, whatever the tile shape, so both passes see bit-identical logits).
// Rows go in chunks for pass 2 and the gradients; what a chunk keeps in the
// workspace is 2 bytes of binary16 p and 1 bit per logit (becoming G) and
// O(rows x V / 128) partials.
#include "launch.hpp"
#include "linear.hpp"
#include "gemm.hpp"
#include "mm.hpp"
#include "common.hpp"

namespace lx {

namespace {

using mm::f32x16_t;

// LDS of the main loop: 2 stages of a 64-k slice, 64 KB each for 256 x 256
// tiles and 48 KB for the dual 256 x 128 tiles.
constexpr int kLds = 2 * 65536;
constexpr int kLdsDual = 2 * (32768 + 16384);
// The 256 x 256 kernels (the gradient products and pass 1) run 8 waves, two per
// SIMD, each 128 x 64 of the tile (4 x 2 accumulators, 128 registers): while one
// wave of a SIMD waits for its slice data the other issues its MFMAs (6-7%
// faster than 4 waves of 128 x 128 on the same main loop); each MFMA is then
// followed by up to three of the slice's memory instructions.
constexpr int kWideThreads = 512;
constexpr int kWideMem = 3;
// pass 2's epilogue in the same LDS: row bases, (S, Q) partials, the tile's
// binary16 p (rows padded to 272 bytes: the two half-waves' rows, 4 apart, fall
// on different banks) and its tie words
constexpr int kTilePStride = 136;  // halves per staged row
constexpr int kTileP = 8192;
constexpr int kTileT = kTileP + 256 * kTilePStride * 2;
static_assert(kTileT + 256 * 4 * 4 <= kLdsDual, "pass 2 epilogue exceeds the main loops' LDS");

// ---------------------------------------------------------------- plain products (fp32 C)

// C[m][n] (+)= sum_k A(m, k) B(n, k): 256 x 256 tiles, one workgroup of 4 waves
// per compute unit (the accumulators take all 256 AGPRs).
//
// Split-K (splits > 1): the N sweep runs over tiles_n * splits virtual tiles, the
// splits of one output tile next to each other; split s takes k in [s kslice,
// min(K, (s + 1) kslice)) (kslice a multiple of the 64-k slice) by moving the
// operands' bases to its first k, and writes its product (ACC = false) to
// C + s * split_stride.
template <bool AK, bool BK, bool ACC>
__global__ __attribute__((amdgpu_flat_work_group_size(kWideThreads, kWideThreads), amdgpu_waves_per_eu(2, 2)))
void gemm_bf16_kernel(const uint16_t* __restrict__ A, int64_t lda, int64_t a_end, const uint16_t* __restrict__ B,
                      int64_t ldb, int64_t b_end, float* __restrict__ C, int64_t ldc, int M, int N, int K,
                      int tiles_m, int tiles_n, int splits, int kslice, int64_t split_stride) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLds];
  int tm, tn;
  if (!mm::tile_coords(tiles_m, tiles_n * splits, tm, tn)) return;
  if (splits > 1) {
    const int s = tn % splits;
    tn /= splits;
    const int k0 = s * kslice;
    A += AK ? (int64_t)k0 : (int64_t)k0 * lda;
    B += BK ? (int64_t)k0 : (int64_t)k0 * ldb;
    a_end -= 2 * (AK ? (int64_t)k0 : (int64_t)k0 * lda);
    b_end -= 2 * (BK ? (int64_t)k0 : (int64_t)k0 * ldb);
    K = min(K - k0, kslice);
    C += s * split_stride;
  }
  const int m0 = tm * mm::kBM, n0 = tn * 256;
  const int lane = tid_x() & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid_x() >> 6);
  const int wm = (wave & 1) * 128, wn = (wave >> 1) * 64;
  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (f32x16_t){};
  mm::pin_scalar(C);
  mm::pin_scalar(ldc);
  mm::SliceLoader<AK, 256, kWideThreads> la;
  mm::SliceLoader<BK, 256, kWideThreads> lb;
  la.init(A, lda, a_end, M, K, m0, wave);
  lb.init(B, ldb, b_end, N, K, n0, wave);
  mm::mainloop<AK, BK, 2, 256, kWideThreads, kWideMem>(acc, lds, la, lb, K, wm, wn, wave);
  // (accumulating: the 16 values of a 32 x 32 tile are all read before any is
  // written back, so the reads are in flight together)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn + 32 * j + (lane & 31);
      float old[16];
      if (ACC) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm + 32 * i + mm::acc_row(r, lane);
          old[r] = (m < M && n < N) ? C[(int64_t)m * ldc + n] : 0.0f;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm + 32 * i + mm::acc_row(r, lane);
        if (m < M && n < N) C[(int64_t)m * ldc + n] = ACC ? old[r] + acc[i][j][r] : acc[i][j][r];
      }
    }
  }
}

template <bool AK, bool BK, bool ACC>
hipError_t launch_gemm_t(const GemmArgs& g, hipStream_t st) {
  const int tiles_m = (int)((g.M + mm::kBM - 1) / mm::kBM);
  const int tiles_n = (int)((g.N + 255) / 256);
  // bytes from each operand's start to the end of its last stored row
  const int64_t a_end = 2 * (AK ? (g.M - 1) * g.lda + g.K : (g.K - 1) * g.lda + g.M);
  const int64_t b_end = 2 * (BK ? (g.N - 1) * g.ldb + g.K : (g.K - 1) * g.ldb + g.N);
  hipLaunchKernelGGL((gemm_bf16_kernel<AK, BK, ACC>), dim3(mm::grid_for(tiles_m, tiles_n)), dim3(kWideThreads), 0, st,
                     g.A, g.lda, a_end, g.B, g.ldb, b_end, g.C, g.ldc, (int)g.M, (int)g.N, (int)g.K, tiles_m,
                     tiles_n, 1, (int)g.K, (int64_t)0);
  return hipGetLastError();
}

// C (+)= sum over s in order of partials[s] (M x N, row stride N).
template <bool ACC>
__global__ __launch_bounds__(256) void split_sum_kernel(const float* __restrict__ P, int splits, int64_t M, int64_t N,
                                                        float* __restrict__ C, int64_t ldc) {
  const int64_t total = M * N;
  const int64_t plane = M * N;
  for (int64_t i = (int64_t)bid_x() * 256 + tid_x(); i < total; i += (int64_t)nblocks_x() * 256) {
    const int64_t m = i / N, n = i - m * N;
    float v = ACC ? C[m * ldc + n] : 0.0f;
    for (int s = 0; s < splits; ++s) v += P[s * plane + i];
    C[m * ldc + n] = v;
  }
}

template <bool AK, bool BK>
hipError_t launch_gemm_split(const GemmArgs& g, hipStream_t st) {
  const int tiles_m = (int)((g.M + mm::kBM - 1) / mm::kBM);
  const int tiles_n = (int)((g.N + 255) / 256);
  const int64_t a_end = 2 * (AK ? (g.M - 1) * g.lda + g.K : (g.K - 1) * g.lda + g.M);
  const int64_t b_end = 2 * (BK ? (g.N - 1) * g.ldb + g.K : (g.K - 1) * g.ldb + g.N);
  const int64_t per = (g.K + g.splits - 1) / g.splits;
  const int kslice = (int)((per + mm::kBK - 1) / mm::kBK * mm::kBK);
  const int splits = (int)((g.K + kslice - 1) / kslice);  // no empty split
  hipLaunchKernelGGL((gemm_bf16_kernel<AK, BK, false>), dim3(mm::grid_for(tiles_m, tiles_n * splits)),
                     dim3(kWideThreads), 0, st, g.A, g.lda, a_end, g.B, g.ldb, b_end, g.partials, g.N, (int)g.M,
                     (int)g.N, (int)g.K, tiles_m, tiles_n, splits, kslice, g.M * g.N);
  if (hipError_t e = hipGetLastError()) return e;
  const int64_t total = g.M * g.N;
  const unsigned blocks = (unsigned)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
  if (g.accumulate)
    hipLaunchKernelGGL(split_sum_kernel<true>, dim3(blocks), dim3(256), 0, st, g.partials, splits, g.M, g.N, g.C, g.ldc);
  else
    hipLaunchKernelGGL(split_sum_kernel<false>, dim3(blocks), dim3(256), 0, st, g.partials, splits, g.M, g.N, g.C,
                       g.ldc);
  return hipGetLastError();
}

// ---------------------------------------------------------------- the loss passes over logit tiles

constexpr int kDualBN = 128;  // logit columns per tile (each of z and u)
// 32-bit words of tie bits per row
__host__ __device__ __forceinline__ int64_t tie_words(int64_t V) { return (V + 31) >> 5; }
constexpr float kInvPqBiasG = 0x1p-15f;  // 2^-kPqBias

struct DualArgs {
  const uint16_t *xs, *ws, *xt, *wt;  // bf16 X_s (rows, H_s), W_s (V, H_s), X_t, W_t (nullptr: CE-only)
  int64_t Hs, Ht;
  int rows, V;                        // this launch's rows (from row 0 of xs / xt) and the vocabulary
  const int64_t* target;              // target of row 0 of this launch
  int64_t ignore_index;
  float* partials;                    // [tiles_n][rows][2]: (S - Q, S) per tile
  const float *lse_s, *lse_t;         // TV: per row
  uint16_t* p16;                      // TV with gradients: binary16 2^15 p, (rows, V), or nullptr
  uint32_t* ties;                     // TV with gradients and a teacher: (rows, tie_words(V)) tie bits
  int tiles_m, tiles_n;
};

// Reductions over the 32 lanes of each half-wave (the 32 columns of one
// accumulator row), on the vector ALU: two quad permutations and two rotations
// inside each row of 16 lanes (DPP), then the gfx950 swap of rows 0 <-> 1 and
// 2 <-> 3.  Every lane ends with the reduction of its half; the sum's
// association order is fixed, so the half's first lane always sees the same
// value for the same data.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float swap16(float v, float* other) {
  const unsigned u = __float_as_uint(v);
  const auto pr = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  // the elements go through scalars: this compiler's __builtin_bit_cast of an
  // element of the returned pair reads element 0 whatever the index
  const unsigned lo = pr[0], hi = pr[1];
  *other = __uint_as_float(hi);
  return __uint_as_float(lo);
}
__device__ __forceinline__ float half_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));   // quad_perm [1, 0, 3, 2]
  v = fmaxf(v, dpp_mov<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  v = fmaxf(v, dpp_mov<0x124>(v));  // row_ror 4
  v = fmaxf(v, dpp_mov<0x128>(v));  // row_ror 8
  float hi;
  const float lo = swap16(v, &hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float half_sum(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x124>(v);
  v += dpp_mov<0x128>(v);
  float hi;
  const float lo = swap16(v, &hi);
  return lo + hi;
}

// Row sums of a 32 x 32 accumulator block (one column per lane of each
// half-wave, v[r] the lane's value in row r of its half, r = 0..15), all rows at
// once: at the level of lane bit b every lane keeps half of its rows (those
// its bit b selects), sends the other half to its partner (the lane differing
// only in bit b) and adds what it receives.  Bit 4: the row-pair swap, two rows
// an instruction; bit 3: row_ror 8; bits 0 and 1: quad permutations; then one
// row per lane is left, and bit 2 (a swizzle) completes its sum.  Lane L of a
// half ends with the total of row xsum_row(L) = b1 + 2 b0 + 4 b3 + 8 b4 (lanes
// L and L ^ 4 the same row).  The association order is fixed.
__device__ __forceinline__ int xsum_row(int lane) {
  return ((lane >> 1) & 1) | ((lane & 1) << 1) | (((lane >> 3) & 1) << 2) | (((lane >> 4) & 1) << 3);
}
template <int CTRL>
__device__ __forceinline__ float xsum_level(float lo, float hi, bool bit) {
  const float keep = bit ? hi : lo, send = bit ? lo : hi;
  return keep + dpp_mov<CTRL>(send);
}
__device__ __forceinline__ float xsum16(const float (&v)[16], int lane) {
  float w[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    // rows 0 and 2 of v[k] stay, rows 1 and 3 receive v[k + 8] of rows 0 and 2,
    // and the reverse in the second result: a lane of row 0 gets v[k] of both
    // partners, a lane of row 1 v[k + 8] of both
    const auto pr = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[k]), __float_as_uint(v[k + 8]), false, false);
    const unsigned a = pr[0], b = pr[1];  // copied out: see swap16
    w[k] = __uint_as_float(a) + __uint_as_float(b);
  }
  const bool b3 = (lane >> 3) & 1, b0 = lane & 1, b1 = (lane >> 1) & 1;
  float u[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) u[k] = xsum_level<0x128>(w[k], w[k + 4], b3);  // row_ror 8
  float t[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) t[k] = xsum_level<0xB1>(u[k], u[k + 2], b0);    // quad_perm [1, 0, 3, 2]
  const float x = xsum_level<0x4E>(t[0], t[1], b1);                           // quad_perm [2, 3, 0, 1]
  // lane ^ 4 within each 32 lanes: and-mask 31, or-mask 0, xor-mask 4
  return x + __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x101F));
}

// Per-row (max, sum-exp) of one tensor's tile values for the wave's 128 rows x
// 32 NJ columns (the maxima reduced row by row, the sums 16 rows at a time),
// merged with the other waves of the same rows through LDS: the
// wave's result for tile row `lr` lands in red[wn / (32 NJ) * 256 + lr]
// (workgroup-visible after the caller's barrier).  Columns n >= V do not count.
template <int NJ>
__device__ __forceinline__ void tile_lse(const f32x16_t (&acc)[4][NJ], int wm, int wn, int n0, int V, int lane,
                                         Lse* red /* [256 / (32 NJ)][256] */) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float sr[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v[NJ];
      float m = kMFloor;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const bool ok = n0 + wn + 32 * j + (lane & 31) < V;
        v[j] = acc[i][j][r];
        m = ok ? fmaxf(m, v[j]) : m;
      }
      m = half_max(m);
      const float nb = -(m * kLog2e);
      float s = 0.0f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const bool ok = n0 + wn + 32 * j + (lane & 31) < V;
        s += ok ? exp2_hw(__builtin_fmaf(v[j], kLog2e, nb)) : 0.0f;
      }
      sr[r] = s;
      if ((lane & 31) == 0) red[wn / (32 * NJ) * 256 + wm + 32 * i + mm::acc_row(r, lane)].m = m;
    }
    // the row sums, all 16 rows of the block at once (xsum16)
    const float s = xsum16(sr, lane);
    red[wn / (32 * NJ) * 256 + wm + 32 * i + mm::acc_row(xsum_row(lane & 31), lane)].s = s;
  }
}

// Pass 1 for one tensor: a 256 x 256 tile of its logits (the plain product's
// main loop and tile), reduced to per-row (max, sum-exp) over the tile's
// columns, written to slots `slot`, `slot + 1` of the row's record in
// partials [tiles_n][rows][P]; the student's launch (slot 0) also writes +0
// to slot P - 1 (the target logit's, filled for the target's tile by
// target_logit_kernel).  The teacher's launch fills slots 2, 3 of the same
// records.
struct StatsArgs {
  const uint16_t *x, *w;
  int64_t H;
  int rows, V;
  float* partials;
  int P, slot;
  int tiles_m, tiles_n;
};

__global__ __attribute__((amdgpu_flat_work_group_size(kWideThreads, kWideThreads), amdgpu_waves_per_eu(2, 2)))
void lm_stats_kernel(StatsArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLds];
  int tm, tn;
  if (!mm::tile_coords(a.tiles_m, a.tiles_n, tm, tn)) return;
  const int m0 = tm * mm::kBM, n0 = tn * 256;
  const int lane = tid_x() & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid_x() >> 6);
  const int wm = (wave & 1) * 128, wn = (wave >> 1) * 64;
  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (f32x16_t){};
  {
    mm::SliceLoader<true, 256, kWideThreads> la;
    mm::SliceLoader<true, 256, kWideThreads> lb;
    la.init(a.x, a.H, 2 * ((int64_t)(a.rows - 1) * a.H + a.H), a.rows, (int)a.H, m0, wave);
    lb.init(a.w, a.H, 2 * ((int64_t)(a.V - 1) * a.H + a.H), a.V, (int)a.H, n0, wave);
    mm::pin_scalar(a.partials);
    mm::pin_scalar(a.P);
    mm::pin_scalar(a.slot);
    mm::mainloop<true, true, 2, 256, kWideThreads, kWideMem>(acc, lds, la, lb, (int)a.H, wm, wn, wave);
  }
  const int tid = tid_x();
  Lse* red = reinterpret_cast<Lse*>(lds);  // [4][256]: the four waves of each row block
  tile_lse<2>(acc, wm, wn, n0, a.V, lane, red);
  __syncthreads();
  const int m = m0 + tid;
  if (tid < 256 && m < a.rows) {
    float* o = a.partials + ((int64_t)tn * a.rows + m) * a.P;
    Lse f = red[tid];
    lse_merge(f, red[256 + tid]);
    lse_merge(f, red[512 + tid]);
    lse_merge(f, red[768 + tid]);
    o[a.slot] = f.m;
    o[a.slot + 1] = f.s;
    if (a.slot == 0) o[a.P - 1] = 0.0f;  // the target-logit kernel fills the target tile's slot
  }
}

// The target logit z_t = x_m . w_t of every row with a target in [0, V),
// one wave per row: products of bf16 pairs are exact in fp32 and summed in
// fp32 (lanes take 16-byte pieces of the row in turn, then a fixed-order
// reduction across the wave).  It goes into the last slot of the record of
// the 256-column tile that holds column t, where the stats launches left +0.
__global__ __launch_bounds__(256) void target_logit_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ w, int64_t H, int rows,
                                                           int64_t V, const int64_t* __restrict__ target,
                                                           int64_t ignore_index, float* __restrict__ partials, int P) {
  const int lane = tid_x() & 63;
  const int64_t m = (int64_t)bid_x() * 4 + (tid_x() >> 6);
  if (m >= rows) return;
  const int64_t t = target[m];
  if (t == ignore_index || t < 0 || t >= V) return;
  const uint4* xr = reinterpret_cast<const uint4*>(x + m * H);
  const uint4* wr = reinterpret_cast<const uint4*>(w + t * H);
  float acc = 0.0f;
  for (int64_t c = lane; c < H / 8; c += 64) {
    const uint4 a = xr[c], b = wr[c];
    const unsigned av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = __builtin_fmaf(__uint_as_float(av[e] << 16), __uint_as_float(bv[e] << 16), acc);
      acc = __builtin_fmaf(__uint_as_float(av[e] & 0xffff0000u), __uint_as_float(bv[e] & 0xffff0000u), acc);
    }
  }
  acc += __shfl_xor(acc, 32, 64);
  acc = half_sum(acc);
  if (lane == 0) partials[((t >> 8) * rows + m) * P + (P - 1)] = acc;
}

// Pass 2 over the logit tiles: the products of a 256 x 128 tile of z (and u),
// then the total-variation epilogue.  Four waves, 2 x 2, each 128 x 64 of each
// tensor (4 x 2 MFMA accumulators per tensor: 128 + 128 AGPRs).
template <bool TEACHER, bool WRITE_P>
__global__ __attribute__((amdgpu_flat_work_group_size(mm::kThreads, mm::kThreads), amdgpu_waves_per_eu(1, 1)))
void lm_tile_kernel(DualArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsDual];
  int tm, tn;
  if (!mm::tile_coords(a.tiles_m, a.tiles_n, tm, tn)) return;
  const int m0 = tm * mm::kBM, n0 = tn * kDualBN;
  const int lane = tid_x() & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid_x() >> 6);
  const int wm = (wave & 1) * 128, wn = (wave >> 1) * 64;

  f32x16_t az[4][2], au[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      az[i][j] = (f32x16_t){};
      au[i][j] = (f32x16_t){};
    }
  {
    mm::SliceLoader<true, 256> la;
    mm::SliceLoader<true, 128> lb;
    la.init(a.xs, a.Hs, 2 * ((int64_t)(a.rows - 1) * a.Hs + a.Hs), a.rows, (int)a.Hs, m0, wave);
    lb.init(a.ws, a.Hs, 2 * ((int64_t)(a.V - 1) * a.Hs + a.Hs), a.V, (int)a.Hs, n0, wave);
    mm::mainloop<true, true, 2, 128>(az, lds, la, lb, (int)a.Hs, wm, wn, wave);
  }
  if (TEACHER) {
    mm::SliceLoader<true, 256> la;
    mm::SliceLoader<true, 128> lb;
    la.init(a.xt, a.Ht, 2 * ((int64_t)(a.rows - 1) * a.Ht + a.Ht), a.rows, (int)a.Ht, m0, wave);
    lb.init(a.wt, a.Ht, 2 * ((int64_t)(a.V - 1) * a.Ht + a.Ht), a.V, (int)a.Ht, n0, wave);
    mm::mainloop<true, true, 2, 128>(au, lds, la, lb, (int)a.Ht, wm, wn, wave);
  }
  // LDS is free again (every wave is past the main loops' final barrier)
  const int tid = tid_x();

  {
    // TV: p' = 2^15 p, q' = 2^15 q and s' = 2^-24 sign(p - q) from the arguments
    // a = x log2(e) - lse log2(e) + 15, exactly as the other TV kernels form them.
    // With gradients the tile's binary16 p and its tie words are staged in LDS and
    // written afterwards with whole 16-byte (p) and 4-byte (tie word) stores.
    float* nbs = reinterpret_cast<float*>(lds);         // [256]
    float* nbt = reinterpret_cast<float*>(lds + 1024);  // [256]
    float* red = reinterpret_cast<float*>(lds + 2048);  // [2][256][2] (S, Q) per wave column
    uint16_t* ps = reinterpret_cast<uint16_t*>(lds + kTileP);  // [256][kTilePStride]
    uint32_t* ts = reinterpret_cast<uint32_t*>(lds + kTileT);  // [256][4] tie words
    {
      const int m = m0 + tid;
      float bs = kMFloor, bt = kMFloor;  // ignored and absent rows: p = q = 0
      if (m < a.rows && a.target[m] != a.ignore_index) {
        bs = pq_bias(a.lse_s[m]);
        if (TEACHER) bt = pq_bias(a.lse_t[m]);
      }
      nbs[tid] = bs;
      nbt[tid] = bt;
    }
    __syncthreads();
    // tie words of this wave: lane 4 r + 2 j + h of tw[i] holds the word of
    // accumulator row r of block i, column block j, half-wave h (row + 4 h)
    uint32_t tw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float Sr[16], Qr[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lr = wm + 32 * i + mm::acc_row(r, lane);
        const float bs = nbs[lr], bt = nbt[lr];
        float S = 0.0f, Q = 0.0f;
        uint64_t tie[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int lc = wn + 32 * j + (lane & 31);
          const bool ok = n0 + lc < a.V;
          const float ap = exparg(az[i][j][r], bs);
          const float pp = exp2_hw(ap);
          float sg = 0.0f;
          if (TEACHER) {
            const float aq = exparg(au[i][j][r], bt);
            sg = sign_eps(ap, aq);
            S = __builtin_fmaf(ok ? pp : 0.0f, sg, S);
            Q = __builtin_fmaf(ok ? exp2_hw(aq) : 0.0f, sg, Q);
          }
          if (WRITE_P) {
            uint16_t h = __builtin_bit_cast(uint16_t, (_Float16)pp);
            if (TEACHER && sg < 0.0f) h |= 0x8000u;
            ps[lr * kTilePStride + lc] = h;
            // one bit per logit: sign(p - q) = 0 exactly (the lanes of a half
            // hold 32 consecutive columns of one row)
            if (TEACHER) tie[j] = __ballot(ok && sg == 0.0f);
          }
        }
        if (WRITE_P && TEACHER) {
          // lane 4 r + 2 j + h of tw[i] takes half h of ballot j
          const uint32_t x0 = (lane & 1) ? (uint32_t)(tie[0] >> 32) : (uint32_t)tie[0];
          const uint32_t x1 = (lane & 1) ? (uint32_t)(tie[1] >> 32) : (uint32_t)tie[1];
          const uint32_t y = (lane & 2) ? x1 : x0;
          if ((lane >> 2) == r) tw[i] = y;
        }
        Sr[r] = S;
        Qr[r] = Q;
      }
      if (TEACHER) {
        const float S = xsum16(Sr, lane), Q = xsum16(Qr, lane);
        const int lr = wm + 32 * i + mm::acc_row(xsum_row(lane & 31), lane);
        red[((wn != 0) * 256 + lr) * 2] = S;
        red[((wn != 0) * 256 + lr) * 2 + 1] = Q;
      }
    }
    if (WRITE_P && TEACHER) {
      const int h = lane & 1, j = (lane >> 1) & 1, r = lane >> 2;
#pragma unroll
      for (int i = 0; i < 4; ++i) ts[(wm + 32 * i + (r & 3) + 8 * (r >> 2) + 4 * h) * 4 + (wn >> 5) + j] = tw[i];
    }
    __syncthreads();
    if (TEACHER) {
      const int m = m0 + tid;
      if (m < a.rows) {
        const float S = red[tid * 2] + red[(256 + tid) * 2];
        const float Q = red[tid * 2 + 1] + red[(256 + tid) * 2 + 1];
        float* o = a.partials + ((int64_t)tn * a.rows + m) * 2;
        o[0] = (S - Q) * kTvScale;  // sum |p - q| over the tile's columns
        o[1] = S * kTvScale;        // sum p * sign(p - q)
      }
    }
    if (WRITE_P) {
      // 256 rows x 128 columns of binary16: 16 threads a row, 16 bytes each
      const int c = (tid & 15) * 8;
#pragma unroll 4
      for (int k = 0; k < 16; ++k) {
        const int row = (tid >> 4) + 16 * k;
        const int m = m0 + row;
        if (m < a.rows && n0 + c < a.V)
          *reinterpret_cast<uint4*>(a.p16 + (int64_t)m * a.V + n0 + c) =
              *reinterpret_cast<const uint4*>(ps + row * kTilePStride + c);
      }
      if (TEACHER) {
        const int64_t words = tie_words(a.V);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int row = (tid >> 2) + 64 * k, w = tid & 3;
          const int m = m0 + row;
          if (m < a.rows && tn * 4 + w < words) a.ties[(int64_t)m * words + tn * 4 + w] = ts[row * 4 + w];
        }
      }
    }
  }
}

template <bool TEACHER, bool WRITE_P>
hipError_t launch_tiles(const DualArgs& a, hipStream_t st) {
  (void)hipGetLastError();
  hipLaunchKernelGGL((lm_tile_kernel<TEACHER, WRITE_P>), dim3(mm::grid_for(a.tiles_m, a.tiles_n)),
                     dim3(mm::kThreads), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- G from binary16 p

constexpr int kGRows = 64;   // rows per tile
constexpr int kGCols = 256;  // columns per tile

struct GformArgs {
  const int64_t* target;
  int rows, V;
  int64_t ignore_index;
  const float *lse_s, *sigma, *zt;   // per row (sigma nullptr: CE-only)
  const uint32_t* ties;              // (rows, tie_words(V)) or nullptr (CE-only)
  uint16_t* g;                       // (rows, V): binary16 p in, bf16 G out (in place)
  float g_ce, g_tvd;
  const float* g_scale;
};

// G = p (alpha + beta s) - k g_ce [v == t] with alpha = k g_ce - beta sigma,
// beta = k g_tvd / 2 (the one-pass kernels' step 3: p' (a1 + b1 s'), p' =
// 2^15 p from the binary16 copy, a1 = alpha 2^-15, b1 = beta 2^9, s' = 2^-24
// sign), the target element from its logit in fp32.  A tile of 64 rows x 256
// columns per workgroup: each thread converts 8 groups of 8 consecutive
// values (16 bytes in, 16 bytes out in place).  The gradient products read G
// as it lies: grad_x along its rows, grad_w down its columns.
__global__ __launch_bounds__(256) void gform_kernel(GformArgs a) {
  const int tid = tid_x();
  const unsigned tiles_c = (unsigned)(a.V + kGCols - 1) / kGCols;
  const unsigned b = bid_x();
  const unsigned tr = b / tiles_c;
  const int r0 = (int)tr * kGRows, c0 = (int)(b - tr * tiles_c) * kGCols;
  const int lc = (tid & 7) * 8;
  const float k = a.g_scale ? *a.g_scale : 1.0f;
  const float kce = k * a.g_ce;
  const float beta = a.sigma ? 0.5f * k * a.g_tvd : 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {  // (row half, 64-column block)
    const int lr = (tid >> 3) + 32 * (i & 1), cc = lc + 64 * (i >> 1);
    const int r = r0 + lr, c = c0 + cc;
    if (r >= a.rows || c >= a.V) continue;
    const int64_t t = a.target[r];
    uint16_t* gp = a.g + (int64_t)r * a.V + c;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (t != a.ignore_index) {
      const bool t_ok = t >= 0 && t < a.V;
      const float alpha = kce - beta * (a.sigma ? a.sigma[r] : 0.0f);
      const float a1 = alpha * kInvPqBiasG, b1 = beta * kTvScale;
      const uint4 in = *reinterpret_cast<const uint4*>(gp);
      const uint32_t tb = a.ties ? a.ties[(int64_t)r * tie_words(a.V) + (c >> 5)] >> (c & 31) : 0u;
      // the target element from its logit in fp32 (p may be close to 1 there)
      const float pt = t_ok ? exp2_hw(exparg(a.zt[r], pq_bias(a.lse_s[r]))) : 0.0f;
      const uint32_t iw[4] = {in.x, in.y, in.z, in.w};
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t h = (uint16_t)(iw[e >> 1] >> (16 * (e & 1)));
        const float pp = (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0x7fffu));
        const float sg = ((tb >> e) & 1u) ? 0.0f : ((h & 0x8000u) ? -kSignEps : kSignEps);
        const float f = __builtin_fmaf(sg, b1, a1);
        o[e] = (c + e == t) ? pt * f - kce : pp * f;
      }
      w[0] = pack_bf16x2(o[0], o[1]);
      w[1] = pack_bf16x2(o[2], o[3]);
      w[2] = pack_bf16x2(o[4], o[5]);
      w[3] = pack_bf16x2(o[6], o[7]);
      if (!t_ok) w[0] = w[1] = w[2] = w[3] = (uint32_t)kQNaN16 * 0x10001u;
    }
    *reinterpret_cast<uint4*>(gp) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// ---------------------------------------------------------------- merges of the per-tile partials

// A row's partials from its ~600 (pass 1) or ~1200 (pass 2) tiles: kMergeRows
// rows per workgroup and kMergeParts threads per row, thread j merging, in tile
// order, the j-th of kMergeParts contiguous ranges of tiles; the ranges are then
// merged in order.  A fixed order, so the result does not depend on timing.
// (One thread per row, as in the vocabulary-parallel merges of a few shards,
// would leave most of the GPU idle here.)
constexpr int kMergeRows = 32;
constexpr int kMergeParts = 8;

// partials [N][BT][P]: (m_s, s_s[, m_t, s_t], target logit or +0) per tile -> ce,
// lse_s, lse_t and the target logit
template <bool TEACHER>
__global__ __launch_bounds__(kMergeRows * kMergeParts) void lm_merge_stats_kernel(
    const float* __restrict__ stats, int N, int64_t BT, const int64_t* __restrict__ target, int64_t V,
    int64_t ignore_index, float* __restrict__ ce, float* __restrict__ lse_s, float* __restrict__ lse_t,
    float* __restrict__ zt_out) {
  constexpr int P = TEACHER ? 5 : 3;
  __shared__ float red[kMergeParts][kMergeRows][5];
  const int lr = tid_x() % kMergeRows, part = tid_x() / kMergeRows;
  const int64_t r = (int64_t)bid_x() * kMergeRows + lr;
  const int per = (N + kMergeParts - 1) / kMergeParts;
  const int n0 = min(N, part * per), n1 = min(N, n0 + per);
  Lse fs = lse_init(), ft = lse_init();
  float zt = 0.0f;
  if (r < BT) {
    for (int n = n0; n < n1; ++n) {
      const float* w = stats + ((int64_t)n * BT + r) * P;
      lse_merge(fs, Lse{w[0], w[1]});
      if (TEACHER) lse_merge(ft, Lse{w[2], w[3]});
      zt += w[P - 1];  // the target's tile holds its logit, every other tile +0
    }
  }
  red[part][lr][0] = fs.m;
  red[part][lr][1] = fs.s;
  red[part][lr][2] = ft.m;
  red[part][lr][3] = ft.s;
  red[part][lr][4] = zt;
  __syncthreads();
  if (part != 0 || r >= BT) return;
  for (int j = 1; j < kMergeParts; ++j) {
    lse_merge(fs, Lse{red[j][lr][0], red[j][lr][1]});
    if (TEACHER) lse_merge(ft, Lse{red[j][lr][2], red[j][lr][3]});
    zt += red[j][lr][4];
  }
  const int64_t t = target[r];
  if (t == ignore_index) {
    ce[r] = 0.0f;
    lse_s[r] = 0.0f;
    if (TEACHER) lse_t[r] = 0.0f;
    zt_out[r] = 0.0f;
    return;
  }
  const float ls = lse_value(fs);
  if (t >= 0 && t < V) ce[r] = ls - zt; else store_nan(ce + r);
  lse_s[r] = ls;
  if (TEACHER) lse_t[r] = lse_value(ft);
  zt_out[r] = zt;
}

// partials [N][BT][2]: (sum |p - q|, sum p sign) per tile -> tvd, sigma
__global__ __launch_bounds__(kMergeRows * kMergeParts) void lm_merge_tv_kernel(
    const float* __restrict__ tv, int N, int64_t BT, const int64_t* __restrict__ target, int64_t ignore_index,
    float* __restrict__ tvd, float* __restrict__ sigma) {
  __shared__ float red[kMergeParts][kMergeRows][2];
  const int lr = tid_x() % kMergeRows, part = tid_x() / kMergeRows;
  const int64_t r = (int64_t)bid_x() * kMergeRows + lr;
  const int per = (N + kMergeParts - 1) / kMergeParts;
  const int n0 = min(N, part * per), n1 = min(N, n0 + per);
  float A = 0.0f, S = 0.0f;
  if (r < BT) {
    for (int n = n0; n < n1; ++n) {
      const float2 w = *reinterpret_cast<const float2*>(tv + ((int64_t)n * BT + r) * 2);
      A += w.x;
      S += w.y;
    }
  }
  red[part][lr][0] = A;
  red[part][lr][1] = S;
  __syncthreads();
  if (part != 0 || r >= BT) return;
  for (int j = 1; j < kMergeParts; ++j) {
    A += red[j][lr][0];
    S += red[j][lr][1];
  }
  const bool ign = target[r] == ignore_index;
  tvd[r] = ign ? 0.0f : 0.5f * A;
  sigma[r] = ign ? 0.0f : S;
}

hipError_t launch_lm_merge_stats(const float* stats, int N, const int64_t* target, int64_t BT, int64_t V,
                                 int64_t ignore_index, bool teacher, float* ce, float* lse_s, float* lse_t, float* zt,
                                 hipStream_t st) {
  (void)hipGetLastError();
  const dim3 grid((unsigned)((BT + kMergeRows - 1) / kMergeRows)), block(kMergeRows * kMergeParts);
  if (teacher)
    lm_merge_stats_kernel<true><<<grid, block, 0, st>>>(stats, N, BT, target, V, ignore_index, ce, lse_s, lse_t, zt);
  else
    lm_merge_stats_kernel<false><<<grid, block, 0, st>>>(stats, N, BT, target, V, ignore_index, ce, lse_s, lse_t, zt);
  return hipGetLastError();
}

hipError_t launch_lm_merge_tv(const float* tv, int N, const int64_t* target, int64_t BT, int64_t ignore_index,
                              float* tvd, float* sigma, hipStream_t st) {
  (void)hipGetLastError();
  lm_merge_tv_kernel<<<dim3((unsigned)((BT + kMergeRows - 1) / kMergeRows)), dim3(kMergeRows * kMergeParts), 0, st>>>(
      tv, N, BT, target, ignore_index, tvd, sigma);
  return hipGetLastError();
}

// ---------------------------------------------------------------- workspace

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

struct LinearWs {
  float* stats;      // [V / 256 tiles][BT][P]
  float* zt;         // [BT]
  float* tv;         // [tiles_n][chunk][2]
  uint16_t* p16;     // (chunk, V): binary16 p, then bf16 G
  uint32_t* ties;    // (chunk, tie_words(V))
  float* gxp;        // [gx_splits][chunk][H_s]: split-K partials of grad_x (gx_splits > 1)
  int gx_splits;
  size_t bytes;
};

// Splits of grad_x = G W_s over the vocabulary for a chunk of `rows` rows: a chunk
// whose product has fewer than two 256 x 256 tiles per compute unit would leave
// compute units idle through its whole (V-long) K loop, so K is cut into up to 8
// ranges of at least 2048 (whole 64-k slices each), the partials summed in order.
int gx_splits(int64_t rows, int64_t Hs, int64_t V) {
  const int64_t tiles = ((rows + 255) / 256) * ((Hs + 255) / 256);
  constexpr int64_t kWanted = 512;
  if (tiles >= kWanted) return 1;
  int64_t s = (kWanted + tiles - 1) / tiles;
  if (s > 8) s = 8;
  if (s > V / 2048) s = V / 2048;
  return s < 1 ? 1 : (int)s;
}

LinearWs linear_ws(void* base, int64_t BT, int64_t chunk, int64_t V, int64_t Hs, bool teacher, bool gx, bool gw) {
  LinearWs w{};
  const int64_t tiles_n = (V + kDualBN - 1) / kDualBN;
  const int P = teacher ? 5 : 3;
  const bool grads = gx || gw;
  size_t off = 0;
  char* p = static_cast<char*>(base);
  auto take = [&](size_t bytes) {
    char* q = p ? p + off : nullptr;
    off += align256(bytes);
    return q;
  };
  w.stats = reinterpret_cast<float*>(take((size_t)((V + 255) / 256) * BT * P * 4));
  w.zt = reinterpret_cast<float*>(take((size_t)BT * 4));
  w.tv = teacher ? reinterpret_cast<float*>(take((size_t)tiles_n * chunk * 2 * 4)) : nullptr;
  w.p16 = grads ? reinterpret_cast<uint16_t*>(take((size_t)chunk * V * 2)) : nullptr;
  w.ties = (grads && teacher) ? reinterpret_cast<uint32_t*>(take((size_t)chunk * tie_words(V) * 4)) : nullptr;
  w.gx_splits = gx ? gx_splits(chunk, Hs, V) : 1;
  w.gxp = w.gx_splits > 1 ? reinterpret_cast<float*>(take((size_t)w.gx_splits * chunk * Hs * 4)) : nullptr;
  w.bytes = off;
  return w;
}

}  // namespace

// ---------------------------------------------------------------- entry points

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t st) {
  (void)hipGetLastError();
  if (g.splits > 1) {
    if (!g.partials || !g.a_kc) return hipErrorInvalidValue;  // the lm_head path's layouts only
    return g.b_kc ? launch_gemm_split<true, true>(g, st) : launch_gemm_split<true, false>(g, st);
  }
  if (g.a_kc) {
    if (g.b_kc) return g.accumulate ? launch_gemm_t<true, true, true>(g, st) : launch_gemm_t<true, true, false>(g, st);
    return g.accumulate ? launch_gemm_t<true, false, true>(g, st) : launch_gemm_t<true, false, false>(g, st);
  }
  if (g.b_kc) return g.accumulate ? launch_gemm_t<false, true, true>(g, st) : launch_gemm_t<false, true, false>(g, st);
  return g.accumulate ? launch_gemm_t<false, false, true>(g, st) : launch_gemm_t<false, false, false>(g, st);
}

size_t linear_workspace_bytes(int64_t BT, int64_t chunk_rows, int64_t V, int64_t Hs, bool teacher) {
  if (BT <= 0) return 0;
  const int64_t chunk = chunk_rows < BT ? chunk_rows : BT;
  return linear_ws(nullptr, BT, chunk, V, Hs, teacher, true, true).bytes;
}

hipError_t run_linear(const LinearArgs& a, hipStream_t st) {
  const bool teacher = a.x_t != nullptr;
  const int64_t V = a.V;
  const int64_t chunk = a.chunk_rows < a.BT ? a.chunk_rows : a.BT;
  const bool gx = a.grad_x_s != nullptr, gw = a.grad_w_s != nullptr, grads = gx || gw;
  const LinearWs w = linear_ws(a.workspace, a.BT, chunk, V, a.H_s, teacher, true, true);
  const int tiles_n = (int)((V + kDualBN - 1) / kDualBN);

  // pass 1 over all rows: per-tile (max, sum-exp) of z and of u (256 x 256 tiles,
  // one launch per tensor) and the target logit
  {
    const int stiles_n = (int)((V + 255) / 256);
    StatsArgs sa{};
    sa.x = a.x_s; sa.w = a.w_s; sa.H = a.H_s; sa.rows = (int)a.BT; sa.V = (int)V;
    sa.partials = w.stats; sa.P = teacher ? 5 : 3; sa.slot = 0;
    sa.tiles_m = (int)((a.BT + mm::kBM - 1) / mm::kBM);
    sa.tiles_n = stiles_n;
    (void)hipGetLastError();
    const unsigned grid = mm::grid_for(sa.tiles_m, sa.tiles_n);
    lm_stats_kernel<<<dim3(grid), dim3(kWideThreads), 0, st>>>(sa);
    hipError_t e = hipGetLastError();
    if (e) return e;
    if (teacher) {
      sa.x = a.x_t; sa.w = a.w_t; sa.H = a.H_t; sa.slot = 2;
      lm_stats_kernel<<<dim3(grid), dim3(kWideThreads), 0, st>>>(sa);
      if ((e = hipGetLastError())) return e;
    }
    target_logit_kernel<<<dim3((unsigned)((a.BT + 3) / 4)), dim3(256), 0, st>>>(
        a.x_s, a.w_s, a.H_s, (int)a.BT, V, a.target, a.ignore_index, w.stats, sa.P);
    if ((e = hipGetLastError())) return e;
    if ((e = launch_lm_merge_stats(w.stats, stiles_n, a.target, a.BT, V, a.ignore_index, teacher, a.ce, a.lse_s,
                                   teacher ? a.lse_t : nullptr, w.zt, st)))
      return e;
  }
  if (!teacher && !grads) return hipSuccess;
  for (int64_t r0 = 0; r0 < a.BT; r0 += chunk) {
    const int64_t rows = a.BT - r0 < chunk ? a.BT - r0 : chunk;
    // pass 2 over the chunk: (sum |p - q|, sum p s) per tile, and binary16 p + tie bits for G
    DualArgs d{};
    d.xs = a.x_s + r0 * a.H_s; d.ws = a.w_s; d.xt = teacher ? a.x_t + r0 * a.H_t : nullptr; d.wt = a.w_t;
    d.Hs = a.H_s; d.Ht = a.H_t; d.rows = (int)rows; d.V = (int)V; d.target = a.target + r0;
    d.ignore_index = a.ignore_index; d.partials = w.tv; d.lse_s = a.lse_s + r0;
    d.lse_t = teacher ? a.lse_t + r0 : nullptr; d.p16 = w.p16; d.ties = w.ties;
    d.tiles_m = (int)((rows + mm::kBM - 1) / mm::kBM);
    d.tiles_n = tiles_n;
    hipError_t e;
    if (teacher) {
      e = grads ? launch_tiles<true, true>(d, st) : launch_tiles<true, false>(d, st);
      if (e) return e;
      if ((e = launch_lm_merge_tv(w.tv, tiles_n, a.target + r0, rows, a.ignore_index, a.tvd + r0, a.sigma + r0, st)))
        return e;
    } else {
      if ((e = launch_tiles<false, true>(d, st))) return e;  // binary16 p only
    }
    if (!grads) continue;
    // G (bf16, over the binary16 p, in place)
    GformArgs g{};
    g.target = a.target + r0; g.rows = (int)rows; g.V = (int)V; g.ignore_index = a.ignore_index;
    g.lse_s = a.lse_s + r0; g.sigma = teacher ? a.sigma + r0 : nullptr; g.zt = w.zt + r0;
    g.ties = w.ties; g.g = w.p16;
    g.g_ce = a.g_ce; g.g_tvd = a.g_tvd; g.g_scale = a.g_scale;
    const int64_t gtiles = ((rows + kGRows - 1) / kGRows) * ((V + kGCols - 1) / kGCols);
    (void)hipGetLastError();
    gform_kernel<<<dim3((unsigned)gtiles), dim3(256), 0, st>>>(g);
    if ((e = hipGetLastError())) return e;
    if (gx) {  // grad_x[chunk] = G W_s: M = rows, N = H_s, K = V; W_s read down its columns
      GemmArgs p{w.p16, V, a.w_s, a.H_s, a.grad_x_s + r0 * a.H_s, a.H_s, rows, a.H_s, V, true, false, false};
      p.splits = w.gx_splits;  // sized for a full chunk; a shorter last chunk uses as many
      p.partials = w.gxp;
      if ((e = launch_gemm_bf16(p, st))) return e;
    }
    if (gw) {  // grad_w (+)= G^T X_s[chunk]: M = V, N = H_s, K = rows; G and X_s read down their columns
      GemmArgs p{w.p16, V, a.x_s + r0 * a.H_s, a.H_s, a.grad_w_s, a.H_s, V, a.H_s, rows, false, false, r0 > 0};
      if ((e = launch_gemm_bf16(p, st))) return e;
    }
  }
  return hipSuccess;
}

}  // namespace lx
