// The lm_head matrix product and the CE + TVD loss in one call (host-side
// orchestration of the kernels).
//
// The aibars.net Liger-Kernel project page lists a fused linear cross-entropy
// among the kernels ("FusedLinearCrossEntropy": the lm_head projection and the
// loss together, so the full logits are not kept), and the Liger-Kernel PR
// #1384 analysis page describes the CE + TVD loss over those logits.  Here,
// for student hidden states X_s (BT, H_s), student weight W_s (V, H_s) and
// optionally teacher X_t, W_t:
//
//   z = X_s W_s^T, u = X_t W_t^T                  (bf16 MFMA products, fp32 logits)
//   ce, tvd, lse_s, lse_t, sigma, G = dL/dz       (the loss kernels; G in bf16;
//                                                  with a teacher one pass over
//                                                  the logits, cluster_f32_kernel)
//   dX_s = G W_s,  dW_s = G^T X_s                 (bf16 MFMA products, fp32)
//
// dW_s is formed from transposed copies of G and of the chunk of X_s, written
// over the chunk's logits once the loss no longer needs them: with both
// operands contiguous along the summed (row) dimension the product takes
// 7.8 ms instead of 9.7 ms at 151936 x 4096 x 8192, and the two transposes
// cost well under the difference.
//
// The rows run in chunks of `chunk_rows`: the chunk's logits (fp32) and G
// (bf16) live in the workspace only while the chunk is processed, so the
// workspace holds chunk_rows x V logits, not BT x V.  The weight gradient
// is the sum over the chunks (the first chunk writes it, the others add).
// Logits are kept in fp32: rounding them to bf16 would move ce by up to half
// a bf16 ulp of the target logit, far outside the loss's 1e-4 tolerance.
#include "gemm.hpp"
#include "ids.hpp"
#include "launch.hpp"
#include "linear.hpp"

namespace lx {

namespace {

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

constexpr int kTrRows = 64;   // input rows per tile
constexpr int kTrCols = 256;  // input columns per tile

// out (cols x ld_out, row stride ld_out) = the transpose of in (rows x cols,
// row stride ld_in), bf16 bit patterns, through a 64 x 256 LDS tile per
// workgroup: 16-byte loads along the input rows (eight per thread, all issued
// before the first is used), 16-byte stores along the output rows.  Output
// columns rows..ld_out-1 are written as zeros.  Needs ld_out % 8 == 0 and out
// 16-byte aligned; vec_in says whether ld_in % 8 == 0 and in is 16-byte
// aligned (else the loads go element by element).  The grid is
// ceil(rows / 64) x ceil(cols / 256) workgroups of 256, tile column fastest.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ in, int64_t ld_in,
                                                             int rows, int cols, uint16_t* __restrict__ out,
                                                             int64_t ld_out, int vec_in) {
  constexpr int kStride = kTrCols + 2;  // halves per LDS row: 2-way bank reuse at most
  __shared__ uint32_t tile32[kTrRows * kStride / 2];
  const uint16_t* tile = reinterpret_cast<const uint16_t*>(tile32);
  const int tid = tid_x();
  const unsigned tiles_c = (unsigned)(cols + kTrCols - 1) / kTrCols;
  const unsigned b = bid_x();
  const unsigned tr = b / tiles_c;
  const int r0 = (int)tr * kTrRows, c0 = (int)(b - tr * tiles_c) * kTrCols;
  const int lc = (tid & 7) * 8;  // 8 consecutive columns of one input row
  uint32_t w[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i) {  // (row half, 64-column block)
    const int lr = (tid >> 3) + 32 * (i & 1), c = c0 + lc + 64 * (i >> 1), r = r0 + lr;
    w[i][0] = w[i][1] = w[i][2] = w[i][3] = 0u;
    if (r < rows) {
      const uint16_t* src = in + (int64_t)r * ld_in + c;
      if (vec_in && c + 8 <= cols) {
        const uint4 v = *reinterpret_cast<const uint4*>(src);
        w[i][0] = v.x; w[i][1] = v.y; w[i][2] = v.z; w[i][3] = v.w;
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (c + k < cols) w[i][k >> 1] |= (uint32_t)src[k] << (16 * (k & 1));
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int lr = (tid >> 3) + 32 * (i & 1), cc = lc + 64 * (i >> 1);
#pragma unroll
    for (int k = 0; k < 4; ++k) tile32[(lr * kStride + cc) / 2 + k] = w[i][k];
  }
  __syncthreads();
  const int lr = (tid & 7) * 8;  // 8 consecutive input rows = output columns
  const int r = r0 + lr;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int oc = (tid >> 3) + 32 * i;  // input column = output row
    const int c = c0 + oc;
    if (c < cols && r < ld_out) {  // r % 8 == 0 and ld_out % 8 == 0: all 8 in the row
      uint32_t o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        o[k] = (uint32_t)tile[(lr + 2 * k) * kStride + oc] | ((uint32_t)tile[(lr + 2 * k + 1) * kStride + oc] << 16);
      *reinterpret_cast<uint4*>(out + (int64_t)c * ld_out + r) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

hipError_t launch_transpose_bf16(const uint16_t* in, int64_t ld_in, int64_t rows, int64_t cols, uint16_t* out,
                                 int64_t ld_out, hipStream_t st) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  if (ld_out % 8 || ld_out < rows || reinterpret_cast<uintptr_t>(out) % 16 || ld_in < cols) return hipErrorInvalidValue;
  const int64_t tiles = ((rows + kTrRows - 1) / kTrRows) * ((cols + kTrCols - 1) / kTrCols);
  if (rows > INT32_MAX || cols > INT32_MAX || tiles > UINT32_MAX) return hipErrorInvalidValue;
  const int vec_in = (ld_in % 8 == 0 && reinterpret_cast<uintptr_t>(in) % 16 == 0) ? 1 : 0;
  transpose_bf16_kernel<<<dim3((unsigned)tiles), dim3(256), 0, st>>>(in, ld_in, (int)rows, (int)cols, out, ld_out,
                                                                     vec_in);
  return hipGetLastError();
}

struct LinearWs {
  float *z, *u;
  uint16_t* g;
  void* fwd;
  size_t bytes;
  size_t logits_bytes;  // z and u, contiguous
};

// Layout for chunks of at most `rows` rows out of BT: z | u | G | the forward's
// workspace (enough for a full chunk and for the last, shorter one).
LinearWs linear_ws(void* base, int64_t BT, int64_t rows, int64_t V, bool teacher) {
  LinearWs w{};
  const size_t zl = align256((size_t)rows * (size_t)V * 4);
  const size_t gl = align256((size_t)rows * (size_t)V * 2);
  // the loss's workspace: the forward's, or the one pass's (with a teacher)
  auto loss_ws = [&](int64_t n) {
    const size_t f = plan_forward(n, V, 4, teacher).workspace_bytes;
    const size_t o = teacher ? plan_linear_onepass(n, V).workspace_bytes : 0;
    return f > o ? f : o;
  };
  size_t fl = loss_ws(rows);
  const int64_t tail = BT % rows;
  if (tail) {
    const size_t ft = loss_ws(tail);
    fl = ft > fl ? ft : fl;
  }
  fl = align256(fl);
  char* p = static_cast<char*>(base);
  w.z = reinterpret_cast<float*>(p);
  w.u = teacher ? reinterpret_cast<float*>(p + zl) : nullptr;
  w.g = reinterpret_cast<uint16_t*>(p + zl * (teacher ? 2 : 1));
  w.fwd = p + zl * (teacher ? 2 : 1) + gl;
  w.bytes = zl * (teacher ? 2 : 1) + gl + fl;
  w.logits_bytes = zl * (teacher ? 2 : 1);
  return w;
}

}  // namespace

size_t linear_workspace_bytes(int64_t BT, int64_t chunk_rows, int64_t V, bool teacher) {
  if (BT <= 0) return 0;
  return linear_ws(nullptr, BT, chunk_rows < BT ? chunk_rows : BT, V, teacher).bytes;
}

hipError_t run_linear(const LinearArgs& a, hipStream_t st) {
  const bool teacher = a.x_t != nullptr;
  const int64_t V = a.V;
  const int64_t max_rows = a.chunk_rows < a.BT ? a.chunk_rows : a.BT;
  const LinearWs w = linear_ws(a.workspace, a.BT, max_rows, V, teacher);
  for (int64_t r0 = 0; r0 < a.BT; r0 += max_rows) {
    const int64_t rows = a.BT - r0 < max_rows ? a.BT - r0 : max_rows;
    // logits of the chunk
    GemmArgs gz{a.x_s + r0 * a.H_s, a.H_s, a.w_s, a.H_s, w.z, V, rows, V, a.H_s, true, true, false};
    if (hipError_t e = launch_gemm_bf16(gz, st)) return e;
    if (teacher) {
      GemmArgs gu{a.x_t + r0 * a.H_t, a.H_t, a.w_t, a.H_t, w.u, V, rows, V, a.H_t, true, true, false};
      if (hipError_t e = launch_gemm_bf16(gu, st)) return e;
    }
    // the loss over the chunk's fp32 logits (and G = dL/dz in bf16)
    FwdArgs f{};
    f.student = w.z;
    f.teacher = w.u;
    f.target = a.target + r0;
    f.BT = rows;
    f.V = V;
    f.ignore_index = a.ignore_index;
    f.lds = V;
    f.ldt = V;
    f.ce = a.ce + r0;
    f.tvd = teacher ? a.tvd + r0 : nullptr;
    f.lse_s = a.lse_s + r0;
    f.lse_t = teacher ? a.lse_t + r0 : nullptr;
    f.sigma = teacher ? a.sigma + r0 : nullptr;
    f.vec = 1;
    f.rows16 = 1;
    f.workspace = w.fwd;
    const bool grads = a.grad_x_s || a.grad_w_s;
    const ClusterPlan op = (teacher && grads) ? plan_linear_onepass(rows, V) : ClusterPlan{0, 0, 0};
    if (op.K > 0) {
      // forward and G in one pass over the logits
      const FusedGrad fg{w.g, V, a.g_ce, a.g_tvd, nullptr, nullptr, a.g_scale};
      if (hipError_t e = launch_linear_onepass(f, fg, op, st)) return e;
    } else {
      if (hipError_t e = launch_forward(f, plan_forward(rows, V, 4, teacher), Dt::F32, st)) return e;
    }
    if (!grads) continue;
    // G = dL/dz in bf16 (when the one pass has not formed it)
    if (op.K == 0) {
      BwdArgs b{};
      b.grad = w.g;
      b.student = w.z;
      b.teacher = w.u;
      b.target = a.target + r0;
      b.BT = rows;
      b.V = V;
      b.ignore_index = a.ignore_index;
      b.ldg = V;
      b.lds = V;
      b.ldt = V;
      b.lse_s = f.lse_s;
      b.lse_t = f.lse_t;
      b.sigma = f.sigma;
      b.g_ce = a.g_ce;
      b.g_tvd = a.g_tvd;
      b.g_scale = a.g_scale;
      b.vec = 1;  // V % 8 == 0 and 256-byte aligned chunks: every fp32 and bf16 row on a 16-byte boundary
      b.v0 = 0;
      b.V_total = V;
      if (hipError_t e = launch_backward_f32_to_bf16(b, st)) return e;
    }
    if (a.grad_x_s) {  // dX_s[chunk] = G W_s
      GemmArgs gx{w.g, V, a.w_s, a.H_s, a.grad_x_s + r0 * a.H_s, a.H_s, rows, a.H_s, V, true, false, false};
      if (hipError_t e = launch_gemm_bf16(gx, st)) return e;
    }
    if (a.grad_w_s) {  // dW_s (+)= G^T X_s[chunk]
      const uint16_t* xc = a.x_s + r0 * a.H_s;
      // G^T (V x ldr) and X_s[chunk]^T (H_s x ldr) over the dead logits, when they fit
      const int64_t ldr = (rows + 7) & ~(int64_t)7;
      const size_t gtl = align256((size_t)V * (size_t)ldr * 2);
      const size_t need = gtl + (size_t)a.H_s * (size_t)ldr * 2;
      if (need <= w.logits_bytes) {
        uint16_t* gt = reinterpret_cast<uint16_t*>(w.z);
        uint16_t* xt = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(w.z) + gtl);
        if (hipError_t e = launch_transpose_bf16(w.g, V, rows, V, gt, ldr, st)) return e;
        if (hipError_t e = launch_transpose_bf16(xc, a.H_s, rows, a.H_s, xt, ldr, st)) return e;
        GemmArgs gw{gt, ldr, xt, ldr, a.grad_w_s, a.H_s, V, a.H_s, rows, true, true, r0 > 0};
        if (hipError_t e = launch_gemm_bf16(gw, st)) return e;
      } else {
        GemmArgs gw{w.g, V, xc, a.H_s, a.grad_w_s, a.H_s, V, a.H_s, rows, false, false, r0 > 0};
        if (hipError_t e = launch_gemm_bf16(gw, st)) return e;
      }
    }
  }
  return hipSuccess;
}

}  // namespace lx
