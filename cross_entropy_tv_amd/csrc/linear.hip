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
// The rows run in chunks of `chunk_rows`: the chunk's logits (fp32) and G
// (bf16) live in the workspace only while the chunk is processed, so the
// workspace holds chunk_rows x V logits, not BT x V.  The weight gradient
// is the sum over the chunks (the first chunk writes it, the others add).
// Logits are kept in fp32: rounding them to bf16 would move ce by up to half
// a bf16 ulp of the target logit, far outside the loss's 1e-4 tolerance.
#include "gemm.hpp"
#include "launch.hpp"
#include "linear.hpp"

namespace lx {

namespace {

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

struct LinearWs {
  float *z, *u;
  uint16_t* g;
  void* fwd;
  size_t bytes;
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
      GemmArgs gw{w.g, V, a.x_s + r0 * a.H_s, a.H_s, a.grad_w_s, a.H_s, V, a.H_s, rows, false, false, r0 > 0};
      if (hipError_t e = launch_gemm_bf16(gw, st)) return e;
    }
  }
  return hipSuccess;
}

}  // namespace lx
