// Host interface of the lm_head product + CE + TVD path (linear.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lx {

struct LinearArgs {
  const uint16_t *x_s, *w_s;  // bf16 (BT, H_s), (V, H_s)
  const uint16_t *x_t, *w_t;  // bf16 (BT, H_t), (V, H_t), or nullptr: CE-only
  int64_t H_s, H_t;
  const int64_t* target;
  int64_t BT, V, ignore_index;
  float *ce, *tvd, *lse_s, *lse_t, *sigma;
  float* grad_x_s;  // (BT, H_s) or nullptr
  float* grad_w_s;  // (V, H_s) or nullptr
  float g_ce, g_tvd;
  const float* g_scale;
  int64_t chunk_rows;
  void* workspace;
};

// Workspace for BT rows processed in chunks of at most chunk_rows rows.
size_t linear_workspace_bytes(int64_t BT, int64_t chunk_rows, int64_t V, int64_t Hs, bool teacher);
hipError_t run_linear(const LinearArgs& a, hipStream_t stream);

}  // namespace lx
