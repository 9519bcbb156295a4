// Host-side launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "lx_ce_tvd.h"

namespace lx {

// How the forward is run for a shape.
//   split == 1: one workgroup per row ("row path").
//   split  > 1: each row is cut into `split` chunks handled by separate
//               workgroups; per-chunk partials go through the workspace and
//               are merged in chunk order ("split-V path").
//   cluster.K > 0: long bf16 rows with a teacher; each row is cut into K
//               member chunks kept in registers by K cooperating workgroups,
//               so the logits are read once ("read-once path").  Taken when
//               the student and teacher rows are 16-byte aligned; otherwise
//               the forward falls back to the row or split-V path.
constexpr int kClusterMaxK = 32;

// Logits (and gradient) element type.
enum class Dt { F32, BF16, F16 };

struct ClusterPlan {
  int K;    // member workgroups per row (0: not applicable)
  int gpm;  // groups of 8 elements per member
  size_t workspace_bytes;
};

ClusterPlan plan_cluster(int64_t BT, int64_t V, int esize, bool teacher);
// Plan of the fused forward + backward kernel (same conditions, its own chunk size).
ClusterPlan plan_fused(int64_t BT, int64_t V, int esize, bool teacher);

struct FwdPlan {
  int split;
  ClusterPlan cluster;
  size_t workspace_bytes;  // enough for whichever path the call takes
};

FwdPlan plan_forward(int64_t BT, int64_t V, int esize, bool teacher);

// Row r of a logits array starts at element r * ld (ld >= V: the row stride).
struct FwdArgs {
  const void* student;
  const void* teacher;  // nullptr: CE-only
  const int64_t* target;
  int64_t BT, V, ignore_index;
  int64_t lds, ldt;     // row strides of student and teacher
  float *ce, *tvd, *lse_s, *lse_t, *sigma;
  int vec;     // every row of every tensor shares one address modulo 16: 16-byte vector path usable
  int rows16;  // every row of every tensor starts on a 16-byte boundary (read-once / one-pass paths)
  void* workspace;
};

struct BwdArgs {
  void* grad;
  const void* student;
  const void* teacher;  // nullptr: CE-only
  const int64_t* target;
  int64_t BT, V, ignore_index;
  int64_t ldg, lds, ldt;  // row strides of grad, student and teacher
  const float *lse_s, *lse_t, *sigma;
  float g_ce, g_tvd;
  const float *gce_rows, *gtvd_rows;  // per-row factors of g_ce and g_tvd, or nullptr
  const float* g_scale;
  int vec;
  // Column shard: these V columns are columns [v0, v0 + V) of rows of V_total
  // (v0 = 0 and V_total = V for whole rows).  Targets index the whole row.
  int64_t v0, V_total;
};

hipError_t launch_forward(const FwdArgs& a, const FwdPlan& plan, Dt dt, hipStream_t stream);
hipError_t launch_forward_cluster(const FwdArgs& a, const ClusterPlan& c, Dt dt, hipStream_t stream);

// Gradient arguments of the fused forward + backward.
struct FusedGrad {
  void* grad;
  int64_t ldg;
  float g_ce, g_tvd;
  const float *gce_rows, *gtvd_rows;
  const float* g_scale;
};
hipError_t launch_fused_cluster(const FwdArgs& a, const FusedGrad& g, const ClusterPlan& c, Dt dt,
                                hipStream_t stream);
hipError_t launch_backward(const BwdArgs& a, Dt dt, hipStream_t stream);
// One pass over fp32 logits with a teacher (V a multiple of 4, rows on
// 16-byte boundaries), the student gradient in bf16 (g.grad, row stride
// g.ldg): the lm_head path's loss.  launch_fused_cluster with Dt::F32 runs
// the same kernel with an fp32 gradient.
ClusterPlan plan_linear_onepass(int64_t BT, int64_t V);
hipError_t launch_linear_onepass(const FwdArgs& a, const FusedGrad& g, const ClusterPlan& c, hipStream_t stream);
// fp32 logits, bf16 gradient (rounded to nearest even); vec must be 0 unless
// every logits row and gradient row share one address modulo 16 in elements
// of their own size, i.e. pass vec = 0 when in doubt.
hipError_t launch_backward_f32_to_bf16(const BwdArgs& a, hipStream_t stream);
// Vocabulary-parallel pieces (vocab_parallel.hip): the shard holds columns
// [v0, v0 + Vs) of rows of the whole vocabulary.
struct VpArgs {
  const void* student;
  const void* teacher;  // nullptr: CE-only (stats only)
  const int64_t* target;
  int64_t BT, Vs, v0, ignore_index;
  const float *lse_s, *lse_t;  // vp_tv only
  float* out;                  // stats [BT][5 or 3] or tv [BT][2]
  int vec;
};
hipError_t launch_vp_stats(const VpArgs& a, Dt dt, hipStream_t stream);
hipError_t launch_vp_tv(const VpArgs& a, Dt dt, hipStream_t stream);
hipError_t launch_vp_merge_stats(const float* stats, int64_t N, const int64_t* target, int64_t BT, int64_t V,
                                 int64_t ignore_index, bool teacher, float* ce, float* lse_s, float* lse_t,
                                 hipStream_t stream);
// As launch_vp_merge_stats, also writing each row's target logit (the sum of
// the shards' target parts; 0 for ignored rows) to zt (nullptr: not written).
hipError_t launch_vp_merge_stats_zt(const float* stats, int64_t N, const int64_t* target, int64_t BT, int64_t V,
                                    int64_t ignore_index, bool teacher, float* ce, float* lse_s, float* lse_t,
                                    float* zt, hipStream_t stream);
hipError_t launch_vp_merge_tv(const float* tv, int64_t N, const int64_t* target, int64_t BT, int64_t ignore_index,
                              float* tvd, float* sigma, hipStream_t stream);

// Reference streams (stream.hip): bytes a multiple of 16, buffers 16-byte aligned.
hipError_t launch_stream_read(const void* src, int64_t bytes, unsigned* sink, hipStream_t stream);
hipError_t launch_stream_read2_write(const void* a, const void* b, void* out, int64_t bytes, hipStream_t stream);

// Records e as the calling thread's last HIP error (lx_last_hip_error).
void record_hip_error(hipError_t e);

// Supplies `need` bytes of scratch memory of the library's own (*ws, with its
// size in *bytes), or an error status.
typedef lx_status (*ScratchProvider)(size_t need, void** ws, size_t* bytes);
// lx_ce_tvd_forward_backward with the scratch memory from `scratch`, asked for
// after the arguments are validated.
lx_status forward_backward_scratch(const void* student, const void* teacher, const int64_t* target, int64_t BT,
                                   int64_t V, int64_t ignore_index, float* ce, float* tvd, float* lse_s,
                                   float* lse_t, float* sigma, void* grad, float g_ce, float g_tvd,
                                   const float* g_scale, lx_dtype dt, void* stream, ScratchProvider scratch);

hipError_t launch_reduce_mean(const float* ce, const float* tvd, const int64_t* target, int64_t BT,
                              int64_t ignore_index, float* mean_out, int64_t* n_valid, float* inv_n_valid,
                              hipStream_t stream);

}  // namespace lx
