// C ABI entry points (include/lx_ce_tvd.h): host-side validation, path
// selection and kernel launches.  Validation runs entirely on the host and
// before any HIP call, so a rejected call enqueues nothing.
#include <limits.h>
#include <stdint.h>

#include "gemm.hpp"
#include "launch.hpp"
#include "linear.hpp"
#include "lx_ce_tvd.h"

namespace {

thread_local int g_last_hip_error = 0;

lx_status from_hip(hipError_t e) {
  if (e == hipSuccess) return LX_OK;
  g_last_hip_error = (int)e;
  return LX_ERR_HIP;
}

int esize_of(lx_dtype dt) {
  switch (dt) {
    case LX_F32: return 4;
    case LX_BF16: return 2;
    case LX_F16: return 2;
    default: return 0;
  }
}

lx::Dt dt_of(lx_dtype dt) {
  return dt == LX_BF16 ? lx::Dt::BF16 : dt == LX_F16 ? lx::Dt::F16 : lx::Dt::F32;
}

// byte range [lo, hi) of an array; empty when p is NULL
struct Span {
  uintptr_t lo, hi;
};
Span span(const void* p, int64_t bytes) {
  const uintptr_t a = (uintptr_t)p;
  return p ? Span{a, a + (uintptr_t)bytes} : Span{0, 0};
}
bool overlaps(Span a, Span b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }
bool any_overlap(const Span* s, int n) {
  for (int i = 0; i < n; ++i)
    for (int j = i + 1; j < n; ++j)
      if (overlaps(s[i], s[j])) return true;
  return false;
}
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

lx_status check_shape(int64_t BT, int64_t V, int es) {
  if (BT < 0 || V < 1 || V > (int64_t)INT_MAX) return LX_ERR_INVALID_ARG;
  if (BT > 0 && BT > INT64_MAX / V / es) return LX_ERR_INVALID_ARG;
  return LX_OK;
}

// A row stride ld >= V with the last row's end, (BT - 1) * ld + V elements,
// addressable in bytes.
bool stride_ok(int64_t BT, int64_t V, int64_t ld, int es) {
  if (ld < V) return false;
  if (BT <= 1) return true;
  return BT - 1 <= (INT64_MAX / es - V) / ld;
}
// bytes from the first row's start to the last row's end
int64_t strided_bytes(int64_t BT, int64_t V, int64_t ld, int es) { return ((BT - 1) * ld + V) * es; }

// Row r of a tensor starts at base + r * ld * es bytes.  Two tensors' rows
// share their address modulo 16 on every row when their bases do and, with
// more than one row, their strides in bytes agree modulo 16.
bool same_mod16(const void* a, int64_t lda, const void* b, int64_t ldb, int64_t BT, int es) {
  if ((((uintptr_t)a - (uintptr_t)b) & 15u) != 0) return false;
  return BT <= 1 || (((lda - ldb) * es) & 15) == 0;
}
// every row starts on a 16-byte boundary
bool rows16(const void* a, int64_t ld, int64_t BT, int es) {
  return ((uintptr_t)a & 15u) == 0 && (BT <= 1 || ((ld * es) & 15) == 0);
}

struct Tensor {
  const void* p;
  int64_t ld;
};

lx_status forward_impl(Tensor zs, Tensor us, const int64_t* target, int64_t BT, int64_t V, int64_t ignore_index,
                       float* ce, float* tvd, float* lse_s, float* lse_t, float* sigma, lx_dtype dt,
                       void* workspace, size_t workspace_bytes, void* stream) {
  const int es = esize_of(dt);
  if (!es) return LX_ERR_UNSUPPORTED_DTYPE;
  if (lx_status s = check_shape(BT, V, es)) return s;
  if (BT == 0) return LX_OK;
  const bool has_t = us.p != nullptr;
  if (!stride_ok(BT, V, zs.ld, es) || (has_t && !stride_ok(BT, V, us.ld, es))) return LX_ERR_INVALID_ARG;
  if (!zs.p || !target || !ce || !lse_s) return LX_ERR_INVALID_ARG;
  if (has_t && (!tvd || !lse_t || !sigma)) return LX_ERR_INVALID_ARG;
  if (!aligned(zs.p, es) || (has_t && !aligned(us.p, es)) || !aligned(target, 8) || !aligned(ce, 4) ||
      !aligned(lse_s, 4))
    return LX_ERR_INVALID_ARG;
  if (has_t && (!aligned(tvd, 4) || !aligned(lse_t, 4) || !aligned(sigma, 4))) return LX_ERR_INVALID_ARG;

  const int64_t fb = BT * 4;
  const lx::FwdPlan plan = lx::plan_forward(BT, V, es, has_t);
  Span sp[9] = {span(zs.p, strided_bytes(BT, V, zs.ld, es)),
                span(us.p, has_t ? strided_bytes(BT, V, us.ld, es) : 0),
                span(target, BT * 8), span(ce, fb), span(lse_s, fb),
                span(has_t ? tvd : nullptr, fb), span(has_t ? lse_t : nullptr, fb),
                span(has_t ? sigma : nullptr, fb), span(plan.workspace_bytes ? workspace : nullptr,
                                                         (int64_t)plan.workspace_bytes)};
  // inputs may overlap each other (e.g. teacher == student); outputs and the
  // workspace may overlap nothing
  for (int o = 3; o < 9; ++o)
    for (int i = 0; i < 9; ++i)
      if (i != o && overlaps(sp[o], sp[i])) return LX_ERR_ALIAS;
  if (plan.workspace_bytes) {
    if (!workspace || workspace_bytes < plan.workspace_bytes || !aligned(workspace, 256)) return LX_ERR_WORKSPACE;
  }

  lx::FwdArgs a;
  a.student = zs.p;
  a.teacher = us.p;
  a.target = target;
  a.BT = BT;
  a.V = V;
  a.ignore_index = ignore_index;
  a.lds = zs.ld;
  a.ldt = has_t ? us.ld : zs.ld;
  a.ce = ce;
  a.tvd = tvd;
  a.lse_s = lse_s;
  a.lse_t = lse_t;
  a.sigma = sigma;
  a.vec = (!has_t || same_mod16(zs.p, zs.ld, us.p, us.ld, BT, es)) ? 1 : 0;
  a.rows16 = (rows16(zs.p, zs.ld, BT, es) && (!has_t || rows16(us.p, us.ld, BT, es))) ? 1 : 0;
  a.workspace = workspace;
  return from_hip(lx::launch_forward(a, plan, dt_of(dt), static_cast<hipStream_t>(stream)));
}

// The backward over rows of V columns that are columns [v0, v0 + V) of rows of
// V_total (v0 = 0, V_total = V for whole rows).
lx_status backward_impl(void* grad, int64_t ldg, Tensor zs, Tensor us, const int64_t* target, int64_t BT,
                        int64_t V, int64_t v0, int64_t V_total, int64_t ignore_index, const float* lse_s,
                        const float* lse_t, const float* sigma, float g_ce, float g_tvd, const float* gce_rows,
                        const float* gtvd_rows, const float* g_scale, lx_dtype dt, void* stream) {
  const int es = esize_of(dt);
  if (!es) return LX_ERR_UNSUPPORTED_DTYPE;
  if (lx_status s = check_shape(BT, V, es)) return s;
  if (BT == 0) return LX_OK;
  const bool has_t = us.p != nullptr;
  if (!stride_ok(BT, V, ldg, es) || !stride_ok(BT, V, zs.ld, es) || (has_t && !stride_ok(BT, V, us.ld, es)))
    return LX_ERR_INVALID_ARG;
  if (!grad || !zs.p || !target || !lse_s) return LX_ERR_INVALID_ARG;
  if (has_t && (!lse_t || !sigma)) return LX_ERR_INVALID_ARG;
  if (!aligned(grad, es) || !aligned(zs.p, es) || (has_t && !aligned(us.p, es)) || !aligned(target, 8) ||
      !aligned(lse_s, 4) || (has_t && (!aligned(lse_t, 4) || !aligned(sigma, 4))) ||
      (g_scale && !aligned(g_scale, 4)) || !aligned(gce_rows, 4) || !aligned(gtvd_rows, 4))
    return LX_ERR_INVALID_ARG;

  const int64_t fb = BT * 4;
  const Span g = span(grad, strided_bytes(BT, V, ldg, es));
  const Span ins[9] = {span(zs.p, strided_bytes(BT, V, zs.ld, es)),
                       span(us.p, has_t ? strided_bytes(BT, V, us.ld, es) : 0),
                       span(target, BT * 8), span(lse_s, fb),
                       span(has_t ? lse_t : nullptr, fb), span(has_t ? sigma : nullptr, fb), span(g_scale, 4),
                       span(gce_rows, fb), span(has_t ? gtvd_rows : nullptr, fb)};
  // in place (grad == student with the same row stride) is allowed; any other overlap is not
  const bool in_place = grad == zs.p && ldg == zs.ld;
  if (!in_place && overlaps(g, ins[0])) return LX_ERR_ALIAS;
  for (int i = 1; i < 9; ++i)
    if (overlaps(g, ins[i])) return LX_ERR_ALIAS;

  lx::BwdArgs a;
  a.grad = grad;
  a.student = zs.p;
  a.teacher = us.p;
  a.target = target;
  a.BT = BT;
  a.V = V;
  a.ignore_index = ignore_index;
  a.ldg = ldg;
  a.lds = zs.ld;
  a.ldt = has_t ? us.ld : zs.ld;
  a.lse_s = lse_s;
  a.lse_t = lse_t;
  a.sigma = sigma;
  a.g_ce = g_ce;
  a.g_tvd = g_tvd;
  a.gce_rows = gce_rows;
  a.gtvd_rows = has_t ? gtvd_rows : nullptr;
  a.g_scale = g_scale;
  a.v0 = v0;
  a.V_total = V_total;
  a.vec = (same_mod16(grad, ldg, zs.p, zs.ld, BT, es) && (!has_t || same_mod16(us.p, us.ld, zs.p, zs.ld, BT, es)))
              ? 1 : 0;
  return from_hip(lx::launch_backward(a, dt_of(dt), static_cast<hipStream_t>(stream)));
}

lx_status forward_backward_impl(Tensor zs, Tensor us, const int64_t* target, int64_t BT, int64_t V,
                                int64_t ignore_index, float* ce, float* tvd, float* lse_s, float* lse_t,
                                float* sigma, void* grad, int64_t ldg, float g_ce, float g_tvd,
                                const float* gce_rows, const float* gtvd_rows, const float* g_scale, lx_dtype dt,
                                void* workspace, size_t workspace_bytes, void* stream,
                                lx::ScratchProvider scratch = nullptr) {
  const int es = esize_of(dt);
  if (!es) return LX_ERR_UNSUPPORTED_DTYPE;
  if (lx_status s = check_shape(BT, V, es)) return s;
  if (BT == 0) return LX_OK;
  const bool has_t = us.p != nullptr;
  if (!stride_ok(BT, V, ldg, es) || !stride_ok(BT, V, zs.ld, es) || (has_t && !stride_ok(BT, V, us.ld, es)))
    return LX_ERR_INVALID_ARG;
  if (!zs.p || !target || !ce || !lse_s || !grad) return LX_ERR_INVALID_ARG;
  if (has_t && (!tvd || !lse_t || !sigma)) return LX_ERR_INVALID_ARG;
  if (!aligned(zs.p, es) || (has_t && !aligned(us.p, es)) || !aligned(grad, es) || !aligned(target, 8) ||
      !aligned(ce, 4) || !aligned(lse_s, 4) || (g_scale && !aligned(g_scale, 4)) || !aligned(gce_rows, 4) ||
      !aligned(gtvd_rows, 4))
    return LX_ERR_INVALID_ARG;
  if (has_t && (!aligned(tvd, 4) || !aligned(lse_t, 4) || !aligned(sigma, 4))) return LX_ERR_INVALID_ARG;

  const int64_t fb = BT * 4;
  const lx::FwdPlan plan = lx::plan_forward(BT, V, es, has_t);
  const lx::ClusterPlan fused = lx::plan_fused(BT, V, es, has_t);
  const size_t need = plan.workspace_bytes > fused.workspace_bytes ? plan.workspace_bytes : fused.workspace_bytes;
  // 0..2 inputs (may overlap each other), 3..8 outputs and workspace, 9..11 inputs
  Span sp[12] = {span(zs.p, strided_bytes(BT, V, zs.ld, es)),
                 span(us.p, has_t ? strided_bytes(BT, V, us.ld, es) : 0),
                 span(target, BT * 8), span(ce, fb), span(lse_s, fb),
                 span(has_t ? tvd : nullptr, fb), span(has_t ? lse_t : nullptr, fb),
                 span(has_t ? sigma : nullptr, fb), span(need ? workspace : nullptr, (int64_t)need),
                 span(g_scale, 4), span(gce_rows, fb), span(has_t ? gtvd_rows : nullptr, fb)};
  for (int o = 3; o < 9; ++o)
    for (int i = 0; i < 12; ++i)
      if (i != o && overlaps(sp[o], sp[i])) return LX_ERR_ALIAS;
  // the gradient may be the student logits themselves (in place, same row
  // stride); any other overlap is an error
  const Span g = span(grad, strided_bytes(BT, V, ldg, es));
  const bool in_place = grad == zs.p && ldg == zs.ld;
  if (!in_place && overlaps(g, sp[0])) return LX_ERR_ALIAS;
  for (int i = 1; i < 12; ++i)
    if (overlaps(g, sp[i])) return LX_ERR_ALIAS;
  if (need && scratch) {
    // the library's own scratch (after validation: nothing is looked up for a rejected call)
    if (lx_status s = scratch(need, &workspace, &workspace_bytes)) return s;
  }
  if (need) {
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return LX_ERR_WORKSPACE;
  }

  lx::FwdArgs a;
  a.student = zs.p;
  a.teacher = us.p;
  a.target = target;
  a.BT = BT;
  a.V = V;
  a.ignore_index = ignore_index;
  a.lds = zs.ld;
  a.ldt = has_t ? us.ld : zs.ld;
  a.ce = ce;
  a.tvd = tvd;
  a.lse_s = lse_s;
  a.lse_t = lse_t;
  a.sigma = sigma;
  a.vec = (!has_t || same_mod16(zs.p, zs.ld, us.p, us.ld, BT, es)) ? 1 : 0;
  a.rows16 = (rows16(zs.p, zs.ld, BT, es) && (!has_t || rows16(us.p, us.ld, BT, es))) ? 1 : 0;
  a.workspace = workspace;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (fused.K > 0 && a.rows16 && rows16(grad, ldg, BT, es)) {
    const lx::FusedGrad fg{grad, ldg, g_ce, g_tvd, gce_rows, has_t ? gtvd_rows : nullptr, g_scale};
    return from_hip(lx::launch_fused_cluster(a, fg, fused, dt_of(dt), st));
  }
  // no fused kernel for this shape or layout: the forward, then the backward, on the same stream
  if (lx_status s = from_hip(lx::launch_forward(a, plan, dt_of(dt), st))) return s;
  lx::BwdArgs b;
  b.grad = grad;
  b.student = zs.p;
  b.teacher = us.p;
  b.target = target;
  b.BT = BT;
  b.V = V;
  b.ignore_index = ignore_index;
  b.ldg = ldg;
  b.lds = a.lds;
  b.ldt = a.ldt;
  b.lse_s = lse_s;
  b.lse_t = lse_t;
  b.sigma = sigma;
  b.g_ce = g_ce;
  b.g_tvd = g_tvd;
  b.gce_rows = gce_rows;
  b.gtvd_rows = has_t ? gtvd_rows : nullptr;
  b.g_scale = g_scale;
  b.v0 = 0;
  b.V_total = V;
  b.vec = (same_mod16(grad, ldg, zs.p, zs.ld, BT, es) && (!has_t || same_mod16(us.p, us.ld, zs.p, zs.ld, BT, es)))
              ? 1 : 0;
  return from_hip(lx::launch_backward(b, dt_of(dt), st));
}

}  // namespace

namespace lx {
void record_hip_error(hipError_t e) { g_last_hip_error = (int)e; }

lx_status forward_backward_scratch(const void* student, const void* teacher, const int64_t* target, int64_t BT,
                                   int64_t V, int64_t ignore_index, float* ce, float* tvd, float* lse_s,
                                   float* lse_t, float* sigma, void* grad, float g_ce, float g_tvd,
                                   const float* g_scale, lx_dtype dt, void* stream, ScratchProvider scratch) {
  return forward_backward_impl(Tensor{student, V}, Tensor{teacher, V}, target, BT, V, ignore_index, ce, tvd, lse_s,
                               lse_t, sigma, grad, V, g_ce, g_tvd, nullptr, nullptr, g_scale, dt, nullptr, 0,
                               stream, scratch);
}
}  // namespace lx

extern "C" {

const char* lx_status_string(lx_status s) {
  switch (s) {
    case LX_OK: return "LX_OK";
    case LX_ERR_INVALID_ARG: return "LX_ERR_INVALID_ARG";
    case LX_ERR_UNSUPPORTED_DTYPE: return "LX_ERR_UNSUPPORTED_DTYPE";
    case LX_ERR_ALIAS: return "LX_ERR_ALIAS";
    case LX_ERR_WORKSPACE: return "LX_ERR_WORKSPACE";
    case LX_ERR_HIP: return "LX_ERR_HIP";
    case LX_ERR_TOO_LARGE: return "LX_ERR_TOO_LARGE";
  }
  return "LX_ERR_UNKNOWN";
}

int lx_abi_version(void) { return LX_CE_TVD_ABI_VERSION; }

int lx_last_hip_error(void) { return g_last_hip_error; }

lx_status lx_stream_read(const void* src, int64_t bytes, unsigned* sink, void* stream) {
  if (bytes < 0 || bytes % 16 || bytes > ((int64_t)1 << 40)) return LX_ERR_INVALID_ARG;
  if (bytes == 0) return LX_OK;
  if (!src || !sink || !aligned(src, 16) || !aligned(sink, 4)) return LX_ERR_INVALID_ARG;
  if (overlaps(span(src, bytes), span(sink, 4))) return LX_ERR_ALIAS;
  return from_hip(lx::launch_stream_read(src, bytes, sink, static_cast<hipStream_t>(stream)));
}

lx_status lx_stream_read2_write(const void* a, const void* b, void* out, int64_t bytes, void* stream) {
  if (bytes < 0 || bytes % 16 || bytes > ((int64_t)1 << 40)) return LX_ERR_INVALID_ARG;
  if (bytes == 0) return LX_OK;
  if (!a || !b || !out || !aligned(a, 16) || !aligned(b, 16) || !aligned(out, 16)) return LX_ERR_INVALID_ARG;
  if (overlaps(span(out, bytes), span(a, bytes)) || overlaps(span(out, bytes), span(b, bytes))) return LX_ERR_ALIAS;
  return from_hip(lx::launch_stream_read2_write(a, b, out, bytes, static_cast<hipStream_t>(stream)));
}

size_t lx_ce_tvd_workspace_bytes(int64_t BT, int64_t V, lx_dtype dt, int has_teacher) {
  const int es = esize_of(dt);
  if (!es || check_shape(BT, V, es) != LX_OK) return 0;
  return lx::plan_forward(BT, V, es, has_teacher != 0).workspace_bytes;
}

lx_status lx_ce_tvd_forward(const void* student, const void* teacher, const int64_t* target, int64_t BT,
                            int64_t V, int64_t ignore_index, float* ce, float* tvd, float* lse_s, float* lse_t,
                            float* sigma, lx_dtype dt, void* workspace, size_t workspace_bytes, void* stream) {
  return forward_impl(Tensor{student, V}, Tensor{teacher, V}, target, BT, V, ignore_index, ce, tvd, lse_s, lse_t,
                      sigma, dt, workspace, workspace_bytes, stream);
}

lx_status lx_ce_tvd_forward_ex(const void* student, int64_t ld_student, const void* teacher, int64_t ld_teacher,
                               const int64_t* target, int64_t BT, int64_t V, int64_t ignore_index, float* ce,
                               float* tvd, float* lse_s, float* lse_t, float* sigma, lx_dtype dt, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return forward_impl(Tensor{student, ld_student}, Tensor{teacher, ld_teacher}, target, BT, V, ignore_index, ce,
                      tvd, lse_s, lse_t, sigma, dt, workspace, workspace_bytes, stream);
}

lx_status lx_ce_tvd_backward(void* grad, const void* student, const void* teacher, const int64_t* target,
                             int64_t BT, int64_t V, int64_t ignore_index, const float* lse_s, const float* lse_t,
                             const float* sigma, float g_ce, float g_tvd, const float* g_scale, lx_dtype dt,
                             void* stream) {
  return backward_impl(grad, V, Tensor{student, V}, Tensor{teacher, V}, target, BT, V, 0, V, ignore_index, lse_s,
                       lse_t, sigma, g_ce, g_tvd, nullptr, nullptr, g_scale, dt, stream);
}

lx_status lx_ce_tvd_backward_ex(void* grad, int64_t ld_grad, const void* student, int64_t ld_student,
                                const void* teacher, int64_t ld_teacher, const int64_t* target, int64_t BT,
                                int64_t V, int64_t ignore_index, const float* lse_s, const float* lse_t,
                                const float* sigma, float g_ce, float g_tvd, const float* grad_ce_rows,
                                const float* grad_tvd_rows, const float* g_scale, lx_dtype dt, void* stream) {
  return backward_impl(grad, ld_grad, Tensor{student, ld_student}, Tensor{teacher, ld_teacher}, target, BT, V, 0, V,
                       ignore_index, lse_s, lse_t, sigma, g_ce, g_tvd, grad_ce_rows, grad_tvd_rows, g_scale, dt,
                       stream);
}

lx_status lx_ce_tvd_backward_shard(void* grad, const void* student, const void* teacher, const int64_t* target,
                                   int64_t BT, int64_t V_shard, int64_t v0, int64_t V, int64_t ignore_index,
                                   const float* lse_s, const float* lse_t, const float* sigma, float g_ce,
                                   float g_tvd, const float* g_scale, lx_dtype dt, void* stream) {
  if (v0 < 0 || V_shard < 1 || V < 1 || v0 > V - V_shard) return LX_ERR_INVALID_ARG;
  return backward_impl(grad, V_shard, Tensor{student, V_shard}, Tensor{teacher, V_shard}, target, BT, V_shard, v0, V,
                       ignore_index, lse_s, lse_t, sigma, g_ce, g_tvd, nullptr, nullptr, g_scale, dt, stream);
}

size_t lx_ce_tvd_forward_backward_workspace_bytes(int64_t BT, int64_t V, lx_dtype dt, int has_teacher) {
  const int es = esize_of(dt);
  if (!es || check_shape(BT, V, es) != LX_OK) return 0;
  const size_t f = lx::plan_forward(BT, V, es, has_teacher != 0).workspace_bytes;
  const size_t u = lx::plan_fused(BT, V, es, has_teacher != 0).workspace_bytes;
  return f > u ? f : u;
}

lx_status lx_ce_tvd_forward_backward(const void* student, const void* teacher, const int64_t* target, int64_t BT,
                                     int64_t V, int64_t ignore_index, float* ce, float* tvd, float* lse_s,
                                     float* lse_t, float* sigma, void* grad, float g_ce, float g_tvd,
                                     const float* g_scale, lx_dtype dt, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  return forward_backward_impl(Tensor{student, V}, Tensor{teacher, V}, target, BT, V, ignore_index, ce, tvd, lse_s,
                               lse_t, sigma, grad, V, g_ce, g_tvd, nullptr, nullptr, g_scale, dt, workspace,
                               workspace_bytes, stream);
}

lx_status lx_ce_tvd_forward_backward_ex(const void* student, int64_t ld_student, const void* teacher,
                                        int64_t ld_teacher, const int64_t* target, int64_t BT, int64_t V,
                                        int64_t ignore_index, float* ce, float* tvd, float* lse_s, float* lse_t,
                                        float* sigma, void* grad, int64_t ld_grad, float g_ce, float g_tvd,
                                        const float* grad_ce_rows, const float* grad_tvd_rows, const float* g_scale,
                                        lx_dtype dt, void* workspace, size_t workspace_bytes, void* stream) {
  return forward_backward_impl(Tensor{student, ld_student}, Tensor{teacher, ld_teacher}, target, BT, V,
                               ignore_index, ce, tvd, lse_s, lse_t, sigma, grad, ld_grad, g_ce, g_tvd, grad_ce_rows,
                               grad_tvd_rows, g_scale, dt, workspace, workspace_bytes, stream);
}

lx_status lx_ce_tvd_count_valid(const int64_t* target, int64_t BT, int64_t ignore_index, int64_t* n_valid,
                                float* inv_n_valid, void* stream) {
  if (BT < 0 || (BT > 0 && !target) || (!n_valid && !inv_n_valid)) return LX_ERR_INVALID_ARG;
  if (!aligned(target, 8) || !aligned(n_valid, 8) || !aligned(inv_n_valid, 4)) return LX_ERR_INVALID_ARG;
  const Span sp[3] = {span(target, BT * 8), span(n_valid, 8), span(inv_n_valid, 4)};
  if (any_overlap(sp, 3)) return LX_ERR_ALIAS;
  return from_hip(lx::launch_reduce_mean(nullptr, nullptr, target, BT, ignore_index, nullptr, n_valid, inv_n_valid,
                                         static_cast<hipStream_t>(stream)));
}

lx_status lx_ce_tvd_reduce_mean(const float* ce, const float* tvd, const int64_t* target, int64_t BT,
                                int64_t ignore_index, float* mean_out, int64_t* n_valid, float* inv_n_valid,
                                void* stream) {
  if (BT < 0) return LX_ERR_INVALID_ARG;
  if (!mean_out || (BT > 0 && (!ce || !target))) return LX_ERR_INVALID_ARG;
  if (!aligned(ce, 4) || !aligned(tvd, 4) || !aligned(target, 8) || !aligned(mean_out, 4) ||
      !aligned(n_valid, 8) || !aligned(inv_n_valid, 4))
    return LX_ERR_INVALID_ARG;
  const int64_t fb = BT * 4;
  const Span sp[6] = {span(ce, fb), span(tvd, fb), span(target, BT * 8), span(mean_out, tvd ? 8 : 4),
                      span(n_valid, 8), span(inv_n_valid, 4)};
  for (int o = 3; o < 6; ++o)
    for (int i = 0; i < 6; ++i)
      if (i != o && overlaps(sp[o], sp[i])) return LX_ERR_ALIAS;
  return from_hip(lx::launch_reduce_mean(ce, tvd, target, BT, ignore_index, mean_out, n_valid, inv_n_valid,
                                         static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------------ vocabulary-parallel pieces

lx_status lx_ce_tvd_vp_stats(const void* student, const void* teacher, const int64_t* target, int64_t BT,
                             int64_t V_shard, int64_t v0, int64_t ignore_index, lx_dtype dt, float* stats,
                             void* stream) {
  const int es = esize_of(dt);
  if (!es) return LX_ERR_UNSUPPORTED_DTYPE;
  if (lx_status s = check_shape(BT, V_shard, es)) return s;
  if (v0 < 0) return LX_ERR_INVALID_ARG;
  if (BT == 0) return LX_OK;
  const bool has_t = teacher != nullptr;
  if (!student || !target || !stats) return LX_ERR_INVALID_ARG;
  if (!aligned(student, es) || (has_t && !aligned(teacher, es)) || !aligned(target, 8) || !aligned(stats, 4))
    return LX_ERR_INVALID_ARG;
  const int64_t lb = BT * V_shard * es;
  const Span out = span(stats, BT * (has_t ? 5 : 3) * 4);
  const Span ins[3] = {span(student, lb), span(teacher, lb), span(target, BT * 8)};
  for (int i = 0; i < 3; ++i)
    if (overlaps(out, ins[i])) return LX_ERR_ALIAS;
  lx::VpArgs a{student, teacher, target, BT, V_shard, v0, ignore_index, nullptr, nullptr, stats,
               (!has_t || ((uintptr_t)student & 15u) == ((uintptr_t)teacher & 15u)) ? 1 : 0};
  return from_hip(lx::launch_vp_stats(a, dt_of(dt), static_cast<hipStream_t>(stream)));
}

lx_status lx_ce_tvd_vp_merge_stats(const float* stats, int64_t n_shards, const int64_t* target, int64_t BT,
                                   int64_t V, int64_t ignore_index, int has_teacher, float* ce, float* lse_s,
                                   float* lse_t, void* stream) {
  const int P = has_teacher ? 5 : 3;
  if (BT < 0 || V < 1 || n_shards < 1 || n_shards > (int64_t)INT_MAX) return LX_ERR_INVALID_ARG;
  if (BT > 0 && BT > INT64_MAX / n_shards / P / 4) return LX_ERR_INVALID_ARG;
  if (BT == 0) return LX_OK;
  if (!stats || !target || !ce || !lse_s || (has_teacher && !lse_t)) return LX_ERR_INVALID_ARG;
  if (!aligned(stats, 4) || !aligned(target, 8) || !aligned(ce, 4) || !aligned(lse_s, 4) ||
      (has_teacher && !aligned(lse_t, 4)))
    return LX_ERR_INVALID_ARG;
  const int64_t fb = BT * 4;
  const Span sp[5] = {span(stats, n_shards * BT * P * 4), span(target, BT * 8), span(ce, fb), span(lse_s, fb),
                      span(has_teacher ? lse_t : nullptr, fb)};
  for (int o = 2; o < 5; ++o)
    for (int i = 0; i < 5; ++i)
      if (i != o && overlaps(sp[o], sp[i])) return LX_ERR_ALIAS;
  return from_hip(lx::launch_vp_merge_stats(stats, n_shards, target, BT, V, ignore_index, has_teacher != 0, ce,
                                            lse_s, has_teacher ? lse_t : nullptr, static_cast<hipStream_t>(stream)));
}

lx_status lx_ce_tvd_vp_tv(const void* student, const void* teacher, const int64_t* target, int64_t BT,
                          int64_t V_shard, int64_t ignore_index, const float* lse_s, const float* lse_t, lx_dtype dt,
                          float* tv, void* stream) {
  const int es = esize_of(dt);
  if (!es) return LX_ERR_UNSUPPORTED_DTYPE;
  if (lx_status s = check_shape(BT, V_shard, es)) return s;
  if (BT == 0) return LX_OK;
  if (!student || !teacher || !target || !lse_s || !lse_t || !tv) return LX_ERR_INVALID_ARG;
  if (!aligned(student, es) || !aligned(teacher, es) || !aligned(target, 8) || !aligned(lse_s, 4) ||
      !aligned(lse_t, 4) || !aligned(tv, 4))
    return LX_ERR_INVALID_ARG;
  const int64_t lb = BT * V_shard * es, fb = BT * 4;
  const Span out = span(tv, BT * 2 * 4);
  const Span ins[5] = {span(student, lb), span(teacher, lb), span(target, BT * 8), span(lse_s, fb), span(lse_t, fb)};
  for (int i = 0; i < 5; ++i)
    if (overlaps(out, ins[i])) return LX_ERR_ALIAS;
  lx::VpArgs a{student, teacher, target, BT, V_shard, 0, ignore_index, lse_s, lse_t, tv,
               ((uintptr_t)student & 15u) == ((uintptr_t)teacher & 15u) ? 1 : 0};
  return from_hip(lx::launch_vp_tv(a, dt_of(dt), static_cast<hipStream_t>(stream)));
}

lx_status lx_ce_tvd_vp_merge_tv(const float* tv, int64_t n_shards, const int64_t* target, int64_t BT,
                                int64_t ignore_index, float* tvd, float* sigma, void* stream) {
  if (BT < 0 || n_shards < 1 || n_shards > (int64_t)INT_MAX) return LX_ERR_INVALID_ARG;
  if (BT > 0 && BT > INT64_MAX / n_shards / 8) return LX_ERR_INVALID_ARG;
  if (BT == 0) return LX_OK;
  if (!tv || !target || !tvd || !sigma) return LX_ERR_INVALID_ARG;
  if (!aligned(tv, 4) || !aligned(target, 8) || !aligned(tvd, 4) || !aligned(sigma, 4)) return LX_ERR_INVALID_ARG;
  const int64_t fb = BT * 4;
  const Span sp[4] = {span(tv, n_shards * BT * 8), span(target, BT * 8), span(tvd, fb), span(sigma, fb)};
  for (int o = 2; o < 4; ++o)
    for (int i = 0; i < 4; ++i)
      if (i != o && overlaps(sp[o], sp[i])) return LX_ERR_ALIAS;
  return from_hip(lx::launch_vp_merge_tv(tv, n_shards, target, BT, ignore_index, tvd, sigma,
                                         static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------------ lm_head product + loss

lx_status lx_gemm_bf16(const void* A, int64_t lda, int a_k_contiguous, const void* B, int64_t ldb,
                       int b_k_contiguous, float* C, int64_t ldc, int64_t M, int64_t N, int64_t K, int accumulate,
                       void* stream) {
  if (M < 1 || N < 1 || K < 1 || M > INT_MAX || N > INT_MAX || K > INT_MAX) return LX_ERR_INVALID_ARG;
  if (!A || !B || !C) return LX_ERR_INVALID_ARG;
  const int64_t ca = a_k_contiguous ? K : M, cb = b_k_contiguous ? K : N;  // contiguous dimensions
  const int64_t ra = a_k_contiguous ? M : K, rb = b_k_contiguous ? N : K;  // rows of the stored arrays
  if (ca % 8 || cb % 8 || lda < ca || ldb < cb || lda % 8 || ldb % 8 || ldc < N) return LX_ERR_INVALID_ARG;
  if (lda > lx::kGemmMaxLd || ldb > lx::kGemmMaxLd) return LX_ERR_INVALID_ARG;  // in-slice offsets stay 32-bit
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 4)) return LX_ERR_INVALID_ARG;
  if (ra - 1 > (INT64_MAX / 2 - ca) / lda || rb - 1 > (INT64_MAX / 2 - cb) / ldb ||
      M - 1 > (INT64_MAX / 4 - N) / ldc)
    return LX_ERR_INVALID_ARG;
  if ((M + 255) / 256 * ((N + 255) / 256) > INT_MAX / 8) return LX_ERR_INVALID_ARG;
  const Span sa = span(A, ((ra - 1) * lda + ca) * 2), sb = span(B, ((rb - 1) * ldb + cb) * 2);
  const Span sc = span(C, ((M - 1) * ldc + N) * 4);
  if (overlaps(sc, sa) || overlaps(sc, sb)) return LX_ERR_ALIAS;
  lx::GemmArgs g{static_cast<const uint16_t*>(A), lda, static_cast<const uint16_t*>(B), ldb, C, ldc, M, N, K,
                 a_k_contiguous != 0, b_k_contiguous != 0, accumulate != 0};
  return from_hip(lx::launch_gemm_bf16(g, static_cast<hipStream_t>(stream)));
}

size_t lx_ce_tvd_linear_workspace_bytes(int64_t BT, int64_t V, int64_t H_s, int has_teacher, int64_t chunk_rows) {
  if (BT < 1 || V < 1 || V > (int64_t)INT_MAX || chunk_rows < 1 || H_s < 1 || H_s > lx::kGemmMaxLd) return 0;
  const int64_t rows = chunk_rows < BT ? chunk_rows : BT;
  if (rows > INT64_MAX / V / 16 || BT > INT64_MAX / V / 16) return 0;
  return lx::linear_workspace_bytes(BT, chunk_rows, V, H_s, has_teacher != 0);
}

lx_status lx_ce_tvd_linear_forward_backward(const void* x_s, const void* w_s, int64_t H_s, const void* x_t,
                                            const void* w_t, int64_t H_t, const int64_t* target, int64_t BT,
                                            int64_t V, int64_t ignore_index, float* ce, float* tvd, float* lse_s,
                                            float* lse_t, float* sigma, float* grad_x_s, float* grad_w_s,
                                            float g_ce, float g_tvd, const float* g_scale, int64_t chunk_rows,
                                            void* workspace, size_t workspace_bytes, void* stream) {
  if (BT < 0 || V < 8 || V > lx::kGemmMaxLd || V % 8 || chunk_rows < 1) return LX_ERR_INVALID_ARG;
  if (BT == 0) return LX_OK;
  const bool has_t = x_t != nullptr || w_t != nullptr;
  if (!x_s || !w_s || !target || !ce || !lse_s || (has_t && (!x_t || !w_t || !tvd || !lse_t || !sigma)))
    return LX_ERR_INVALID_ARG;
  if (H_s < 8 || H_s % 8 || H_s > lx::kGemmMaxLd || (has_t && (H_t < 8 || H_t % 8 || H_t > lx::kGemmMaxLd)))
    return LX_ERR_INVALID_ARG;
  if (BT > (int64_t)INT_MAX || V > INT64_MAX / 4 / (H_s > H_t ? H_s : H_t) || BT > INT64_MAX / 4 / H_s ||
      (has_t && BT > INT64_MAX / 4 / H_t))
    return LX_ERR_INVALID_ARG;
  if (!aligned(x_s, 16) || !aligned(w_s, 16) || (has_t && (!aligned(x_t, 16) || !aligned(w_t, 16))) ||
      !aligned(target, 8) || !aligned(ce, 4) || !aligned(lse_s, 4) || !aligned(g_scale, 4) ||
      !aligned(grad_x_s, 4) || !aligned(grad_w_s, 4) ||
      (has_t && (!aligned(tvd, 4) || !aligned(lse_t, 4) || !aligned(sigma, 4))))
    return LX_ERR_INVALID_ARG;
  const size_t need = lx_ce_tvd_linear_workspace_bytes(BT, V, H_s, has_t, chunk_rows);
  if (!need) return LX_ERR_INVALID_ARG;
  const int64_t fb = BT * 4;
  // 0..5 inputs (may overlap each other), 6..13 outputs and the workspace
  const Span sp[14] = {span(x_s, BT * H_s * 2), span(w_s, V * H_s * 2), span(has_t ? x_t : nullptr, BT * H_t * 2),
                       span(has_t ? w_t : nullptr, V * H_t * 2), span(target, BT * 8), span(g_scale, 4),
                       span(ce, fb), span(lse_s, fb), span(has_t ? tvd : nullptr, fb),
                       span(has_t ? lse_t : nullptr, fb), span(has_t ? sigma : nullptr, fb),
                       span(grad_x_s, BT * H_s * 4), span(grad_w_s, V * H_s * 4),
                       span(workspace, (int64_t)need)};
  for (int o = 6; o < 14; ++o)
    for (int i = 0; i < 14; ++i)
      if (i != o && overlaps(sp[o], sp[i])) return LX_ERR_ALIAS;
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return LX_ERR_WORKSPACE;
  lx::LinearArgs a{};
  a.x_s = static_cast<const uint16_t*>(x_s);
  a.w_s = static_cast<const uint16_t*>(w_s);
  a.x_t = has_t ? static_cast<const uint16_t*>(x_t) : nullptr;
  a.w_t = has_t ? static_cast<const uint16_t*>(w_t) : nullptr;
  a.H_s = H_s;
  a.H_t = has_t ? H_t : 0;
  a.target = target;
  a.BT = BT;
  a.V = V;
  a.ignore_index = ignore_index;
  a.ce = ce;
  a.tvd = tvd;
  a.lse_s = lse_s;
  a.lse_t = lse_t;
  a.sigma = sigma;
  a.grad_x_s = grad_x_s;
  a.grad_w_s = grad_w_s;
  a.g_ce = g_ce;
  a.g_tvd = g_tvd;
  a.g_scale = g_scale;
  a.chunk_rows = chunk_rows;
  a.workspace = workspace;
  return from_hip(lx::run_linear(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
