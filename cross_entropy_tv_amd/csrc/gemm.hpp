// Host interface of the bf16 matrix product (gemm.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lx {

// C[m][n] (+)= sum_k A(m, k) * B(n, k), bf16 A and B, fp32 C (row stride ldc).
// A(m, k) = A[m * lda + k] when a_kc, else A[k * lda + m]; likewise B(n, k).
// Preconditions (checked by the caller): 1 <= M, N, K < 2^31; the contiguous
// dimension of A and B a multiple of 8; A, B 16-byte aligned, lda and ldb
// multiples of 8 no larger than kGemmMaxLd; C 4-byte aligned.
// Largest operand row stride (elements) the entry points accept.
constexpr int64_t kGemmMaxLd = 1 << 22;

struct GemmArgs {
  const uint16_t* A;
  int64_t lda;
  const uint16_t* B;
  int64_t ldb;
  float* C;
  int64_t ldc;
  int64_t M, N, K;
  bool a_kc, b_kc, accumulate;
  // split-K: splits > 1 cuts K into `splits` ranges of whole 64-k slices; each
  // range's product goes to partials[s] (M x N, row stride N, fp32) and a second
  // kernel adds them to C in split order (deterministic).  partials: splits * M * N
  // floats of scratch.
  int splits = 1;
  float* partials = nullptr;
};

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t stream);

}  // namespace lx
