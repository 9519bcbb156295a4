// bf16 matrix products for the lm_head path: the logits X W^T, and the
// gradients G W (hidden states) and G^T X (weight) from the logits' gradient
// G.  They are plain products, so they run through hipBLASLt on the matrix
// cores (bf16 operands, fp32 accumulation and output).
//
// C[m][n] (+)= sum_k A(m, k) * B(n, k) with C row-major is, read column-major,
// the N x M product D = op(B) op(A) with D[n, m] = C[m * ldc + n]:
//
//   B(n, k) = B[n * ldb + k] (K-contiguous): B is stored as the K x N
//             column-major matrix B^T (ld = ldb), used transposed;
//   B(n, k) = B[k * ldb + n]: the N x K column-major matrix itself;
//   A(m, k) = A[m * lda + k]: the K x M column-major matrix A^T, as is;
//   A(m, k) = A[k * lda + m]: the M x K column-major matrix, transposed.
//
// so hipBLASLt's first operand is the B buffer, its second the A buffer, and
// its (m, n, k) are (N, M, K).  Accumulation is beta = 1 with C as both the
// input and the output matrix.
//
// Measured on the 8192 x 151936 lm_head of hidden size 4096 (one chunk of
// 4096 rows), these products ran at 39% (logits), 33% (grad_x) and 26%
// (grad_w) of the dense bf16 peak with the library's own MFMA kernel (256 x
// 256 tiles, LDS-direct loads, transposing LDS reads) and run at 48%, 72% and
// 46% through hipBLASLt.
//
// One handle, one workspace (kLtWorkspace bytes of device memory, kept until
// the process ends) and a cache of the chosen algorithm per problem shape are
// kept per device; a mutex serialises their use.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <tuple>

#include "gemm.hpp"

namespace lx {

namespace {

constexpr size_t kLtWorkspace = (size_t)64 << 20;
constexpr int kMaxDevices = 64;

using ShapeKey = std::tuple<int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, bool, bool, bool>;

struct Algo {
  hipblasLtMatmulAlgo_t algo;
  size_t workspace;
};

struct LtDevice {
  std::mutex mu;
  hipblasLtHandle_t handle = nullptr;
  void* ws = nullptr;
  std::map<ShapeKey, Algo> algos;
};

LtDevice g_lt[kMaxDevices];

hipError_t lt_error(hipblasStatus_t s) {
  if (s == HIPBLAS_STATUS_SUCCESS) return hipSuccess;
  if (s == HIPBLAS_STATUS_NOT_SUPPORTED || s == HIPBLAS_STATUS_ARCH_MISMATCH) return hipErrorNotSupported;
  if (s == HIPBLAS_STATUS_ALLOC_FAILED) return hipErrorOutOfMemory;
  if (s == HIPBLAS_STATUS_INVALID_VALUE) return hipErrorInvalidValue;
  return hipErrorUnknown;
}

// descriptors destroyed on every path out of launch_gemm_bf16
struct Desc {
  hipblasLtMatmulDesc_t d = nullptr;
  ~Desc() { if (d) hipblasLtMatmulDescDestroy(d); }
};
struct Layout {
  hipblasLtMatrixLayout_t l = nullptr;
  ~Layout() { if (l) hipblasLtMatrixLayoutDestroy(l); }
};
struct Pref {
  hipblasLtMatmulPreference_t p = nullptr;
  ~Pref() { if (p) hipblasLtMatmulPreferenceDestroy(p); }
};

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t st) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  LtDevice& s = g_lt[dev];
  std::lock_guard<std::mutex> lock(s.mu);
  if (!s.handle) {
    if (hipError_t e = lt_error(hipblasLtCreate(&s.handle))) {
      s.handle = nullptr;
      return e;
    }
  }
  if (!s.ws) {
    if (hipError_t e = hipMalloc(&s.ws, kLtWorkspace)) {
      s.ws = nullptr;
      return e;
    }
  }

  Desc desc;
  if (hipError_t e = lt_error(hipblasLtMatmulDescCreate(&desc.d, HIPBLAS_COMPUTE_32F, HIP_R_32F))) return e;
  const int32_t op_first = g.b_kc ? HIPBLAS_OP_T : HIPBLAS_OP_N;   // the B buffer
  const int32_t op_second = g.a_kc ? HIPBLAS_OP_N : HIPBLAS_OP_T;  // the A buffer
  if (hipError_t e = lt_error(hipblasLtMatmulDescSetAttribute(desc.d, HIPBLASLT_MATMUL_DESC_TRANSA, &op_first,
                                                              sizeof(op_first))))
    return e;
  if (hipError_t e = lt_error(hipblasLtMatmulDescSetAttribute(desc.d, HIPBLASLT_MATMUL_DESC_TRANSB, &op_second,
                                                              sizeof(op_second))))
    return e;
  Layout lf, ls, lc;
  if (hipError_t e = lt_error(hipblasLtMatrixLayoutCreate(&lf.l, HIP_R_16BF, g.b_kc ? g.K : g.N,
                                                          g.b_kc ? g.N : g.K, g.ldb)))
    return e;
  if (hipError_t e = lt_error(hipblasLtMatrixLayoutCreate(&ls.l, HIP_R_16BF, g.a_kc ? g.K : g.M,
                                                          g.a_kc ? g.M : g.K, g.lda)))
    return e;
  if (hipError_t e = lt_error(hipblasLtMatrixLayoutCreate(&lc.l, HIP_R_32F, g.N, g.M, g.ldc))) return e;

  const ShapeKey key{g.M, g.N, g.K, g.lda, g.ldb, g.ldc, g.a_kc, g.b_kc, g.accumulate};
  auto it = s.algos.find(key);
  if (it == s.algos.end()) {
    Pref pref;
    if (hipError_t e = lt_error(hipblasLtMatmulPreferenceCreate(&pref.p))) return e;
    const uint64_t max_ws = kLtWorkspace;
    if (hipError_t e = lt_error(hipblasLtMatmulPreferenceSetAttribute(
            pref.p, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &max_ws, sizeof(max_ws))))
      return e;
    hipblasLtMatmulHeuristicResult_t res[1];
    int found = 0;
    if (hipError_t e = lt_error(hipblasLtMatmulAlgoGetHeuristic(s.handle, desc.d, lf.l, ls.l, lc.l, lc.l, pref.p,
                                                                1, res, &found)))
      return e;
    if (found < 1 || res[0].state != HIPBLAS_STATUS_SUCCESS || res[0].workspaceSize > kLtWorkspace)
      return hipErrorNotSupported;
    it = s.algos.emplace(key, Algo{res[0].algo, res[0].workspaceSize}).first;
  }
  const float alpha = 1.0f, beta = g.accumulate ? 1.0f : 0.0f;
  return lt_error(hipblasLtMatmul(s.handle, desc.d, &alpha, g.B, lf.l, g.A, ls.l, &beta, g.C, lc.l, g.C, lc.l,
                                  &it->second.algo, s.ws, it->second.workspace, st));
}

}  // namespace lx
