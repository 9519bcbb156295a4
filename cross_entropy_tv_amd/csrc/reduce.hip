// Mean of the per-row losses over the rows whose target is not the ignore
// index (a mean-reduced loss, the usual reduction for token-level CE), plus
// 1 / n_valid, the factor such a loss hands to the backward.  With no losses
// given (ce == NULL) the kernel only counts the valid rows, which is all a
// fused forward + backward needs before it runs.
//
// One workgroup; each lane sums a strided subset of rows in float64, then a
// fixed-shape tree in LDS combines the lanes: the result does not depend on
// timing, so it is deterministic.
#include "common.hpp"
#include "launch.hpp"

namespace lx {

constexpr int kRedThreads = 1024;

__global__ __launch_bounds__(kRedThreads) void reduce_mean_kernel(
    const float* __restrict__ ce, const float* __restrict__ tvd, const int64_t* __restrict__ target,
    int64_t BT, int64_t ignore_index, float* __restrict__ mean_out, int64_t* __restrict__ n_valid,
    float* __restrict__ inv_n_valid) {
  __shared__ double sc[kRedThreads];
  __shared__ double st[kRedThreads];
  __shared__ long long sn[kRedThreads];
  const int tid = tid_x();
  double a = 0.0, b = 0.0;
  long long n = 0;
  for (int64_t i = tid; i < BT; i += kRedThreads) {
    if (target[i] != ignore_index) {
      if (ce) a += (double)ce[i];
      if (tvd) b += (double)tvd[i];
      ++n;
    }
  }
  sc[tid] = a;
  st[tid] = b;
  sn[tid] = n;
  __syncthreads();
  for (int w = kRedThreads / 2; w > 0; w >>= 1) {
    if (tid < w) {
      sc[tid] += sc[tid + w];
      st[tid] += st[tid + w];
      sn[tid] += sn[tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) {
    const long long nv = sn[0];
    const double dn = (double)nv;
    if (!mean_out) {
      // counting only (no losses given)
    } else if (nv > 0) {
      mean_out[0] = (float)(sc[0] / dn);
      if (tvd) mean_out[1] = (float)(st[0] / dn);
    } else {  // 0 / 0: NaN, written as bits
      store_nan(mean_out);
      if (tvd) store_nan(mean_out + 1);
    }
    if (n_valid) *n_valid = (int64_t)nv;
    if (inv_n_valid) *inv_n_valid = nv > 0 ? (float)(1.0 / dn) : 0.0f;
  }
}

hipError_t launch_reduce_mean(const float* ce, const float* tvd, const int64_t* target, int64_t BT,
                              int64_t ignore_index, float* mean_out, int64_t* n_valid, float* inv_n_valid,
                              hipStream_t stream) {
  (void)hipGetLastError();  // drop an error left by an earlier, unrelated call
  hipLaunchKernelGGL(reduce_mean_kernel, dim3(1), dim3(kRedThreads), 0, stream, ce, tvd, target, BT,
                     ignore_index, mean_out, n_valid, inv_n_valid);
  return hipGetLastError();
}

}  // namespace lx
