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
// Workgroup tile 256 x 256 x 64, four waves of 128 x 128 (2 x 2), each wave
// a 4 x 4 grid of v_mfma_f32_32x32x16_bf16.  The K-slices of A and B go
// through LDS, double buffered (2 x 2 x 256 x 72 bf16 = 144 KB, so one
// workgroup per compute unit), always stored K-contiguous with 16 bytes of
// padding per row: an operand that is K-contiguous in memory is copied with
// 16-byte writes, one that is M- or N-contiguous is transposed on the way in
// (16-byte global loads along M or N, one k per lane, eight 2-byte LDS
// writes that fill 64 consecutive columns of a row per instruction).  The next
// K-slice is loaded into registers while the current one is multiplied.
//
// Tiles are ordered M-fastest and dealt to the XCDs in contiguous runs (the
// hardware hands workgroup ids to the 8 XCDs round robin), so the workgroups
// that share a B tile run on one XCD and share its L2.
//
// Requirements (checked on the host): the contiguous dimension of every
// operand is a multiple of 8 elements and every row starts on a 16-byte
// boundary; M, N, K >= 1.  Tails of M, N and K are handled by predication
// (zeros are loaded past the ends; stores are masked).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm.hpp"

namespace lx {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kLdsRow = kBK + 8;  // bf16 per LDS row (16 bytes of padding)
constexpr int kThreads = 256;
constexpr int kXcds = 8;

// 16-byte global loads of one K-slice into registers: 2048 vectors of 8 bf16
// per operand, 8 per thread.
struct Slice {
  uint4 v[8];
};

// Operand tile rows r0.. (m or n) over k0..k0+kBK.  KC: K-contiguous storage.
template <bool KC>
__device__ __forceinline__ void load_slice(Slice& s, const uint16_t* P, int64_t ld, int rows, int K, int r0, int k0) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int v = t + kThreads * i;
    int r, k;
    if (KC) {  // 256 rows x 8 vectors along k
      r = v >> 3;
      k = (v & 7) * 8;
    } else {  // 64 k-rows x 32 vectors along r; the 64 lanes of a wave take 64 different k
      k = v & 63;
      r = (v >> 6) * 8;
    }
    const int gr = r0 + r, gk = k0 + k;
    const bool ok = KC ? (gr < rows && gk < K) : (gk < K && gr < rows);
    s.v[i] = ok ? *reinterpret_cast<const uint4*>(KC ? P + (int64_t)gr * ld + gk : P + (int64_t)gk * ld + gr)
                : make_uint4(0u, 0u, 0u, 0u);
  }
}

template <bool KC>
__device__ __forceinline__ void store_slice(const Slice& s, uint16_t (*L)[kLdsRow]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int v = t + kThreads * i;
    if (KC) {
      *reinterpret_cast<uint4*>(&L[v >> 3][(v & 7) * 8]) = s.v[i];
    } else {  // lane k writes column k of rows r..r+7: each row's 64 columns in one instruction
      const int k = v & 63, r = (v >> 6) * 8;
      const uint32_t w[4] = {s.v[i].x, s.v[i].y, s.v[i].z, s.v[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        L[r + 2 * e][k] = (uint16_t)(w[e] & 0xffffu);
        L[r + 2 * e + 1][k] = (uint16_t)(w[e] >> 16);
      }
    }
  }
}

template <bool AK, bool BK, bool ACC>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B, int64_t ldb,
                      float* __restrict__ C, int64_t ldc, int M, int N, int K, int tiles_m, int tiles) {
  __shared__ uint16_t As[2][kBM][kLdsRow];
  __shared__ uint16_t Bs[2][kBN][kLdsRow];

  // XCD-contiguous tile order: workgroup id i runs on XCD i % 8
  const int per_xcd = (tiles + kXcds - 1) / kXcds;
  const int tile = (int)(blockIdx.x % kXcds) * per_xcd + (int)(blockIdx.x / kXcds);
  if (tile >= tiles) return;
  const int m0 = (tile % tiles_m) * kBM;
  const int n0 = (tile / tiles_m) * kBN;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = (wave & 1) * 128, wn = (wave >> 1) * 128;
  const int lr = lane & 31;        // row of the A fragment / column of the B fragment
  const int lk = (lane >> 5) * 8;  // first k of the lane's 8

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16_t){};

  const int nk = (K + kBK - 1) / kBK;
  Slice sa, sb;
  load_slice<AK>(sa, A, lda, M, K, m0, 0);
  load_slice<BK>(sb, B, ldb, N, K, n0, 0);
  store_slice<AK>(sa, As[0]);
  store_slice<BK>(sb, Bs[0]);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      load_slice<AK>(sa, A, lda, M, K, m0, (kt + 1) * kBK);
      load_slice<BK>(sb, B, ldb, N, K, n0, (kt + 1) * kBK);
    }
#pragma unroll
    for (int ks = 0; ks < kBK; ks += 16) {
      bf16x8_t a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const bf16x8_t*>(&As[buf][wm + 32 * i + lr][ks + lk]);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const bf16x8_t*>(&Bs[buf][wn + 32 * j + lr][ks + lk]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      store_slice<AK>(sa, As[buf ^ 1]);
      store_slice<BK>(sb, Bs[buf ^ 1]);
    }
    __syncthreads();
  }

  // register r of lane l holds row (r % 4) + 4 * (l / 32) + 8 * (r / 4), column l % 32 of each 32 x 32 tile
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn + 32 * j + lr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm + 32 * i + (r & 3) + 4 * (lane >> 5) + 8 * (r >> 2);
        if (m < M && n < N) {
          float* c = C + (int64_t)m * ldc + n;
          *c = ACC ? *c + acc[i][j][r] : acc[i][j][r];
        }
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
  hipLaunchKernelGGL((gemm_bf16_kernel<AK, BK, ACC>), dim3((unsigned)(per_xcd * kXcds)), dim3(kThreads), 0, st,
                     g.A, g.lda, g.B, g.ldb, g.C, g.ldc, (int)g.M, (int)g.N, (int)g.K, tiles_m, tiles);
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
