// Forward kernels of the fused CE + TVD loss.
//
// The computation per row is the one of the "Forward Pass" section of the
// Liger-Kernel PR #1384 analysis page: step 1 streams the vocabulary once and
// keeps a running max and sum of exponentials for student and teacher
// together, giving both log-sum-exps; step 2 streams it again, forms p and q
// from those log-sum-exps and accumulates sum |p - q| and sum p * sign(p - q);
// the outputs are ce = lse_s - z[t], tvd = 0.5 * sum |p - q|, lse_s, lse_t,
// sigma.
//
// Row path (many rows): one workgroup owns a row; step 2 walks the row in the
// reverse order of step 1 so that the lines read last in step 1, the ones
// most likely still in L2 / Infinity Cache, are the first ones read again.
//
// Split-V path (few rows, long rows): each row is cut into S chunks, one
// workgroup per (row, chunk).  Stage 1 writes per-chunk (max, sum-exp)
// partials; stage 2 merges a row's partials in chunk order (every workgroup of
// the row gets the bit-identical lse), then accumulates its chunk's
// (sum |p - q|, sum p * sign) partials; stage 3 adds those in chunk order.
// No atomics, so results are deterministic, and the workspace needs no
// clearing.
#include "common.hpp"
#include "launch.hpp"

namespace lx {

constexpr int kRowThreads = 1024;     // workgroup size of the row path
constexpr int kSplitThreads = 256;    // workgroup size of the split-V stages
constexpr int64_t kRowPathMinRows = 512;
constexpr int kSplitTargetBlocks = 2048;
constexpr int kSplitMinChunk = 4096;  // elements
constexpr int kMaxGrid = 1 << 20;

FwdPlan plan_forward(int64_t BT, int64_t V, int esize, bool teacher) {
  FwdPlan p{1, plan_cluster(BT, V, esize, teacher), 0};
  if (BT > 0 && BT < kRowPathMinRows) {
    int64_t s = (kSplitTargetBlocks + BT - 1) / BT;
    const int64_t cap = (V + kSplitMinChunk - 1) / kSplitMinChunk;
    if (s > cap) s = cap;
    if (s > 1024) s = 1024;
    if (s > 1) {
      p.split = (int)s;
      const size_t per = teacher ? 6 : 2;
      p.workspace_bytes = ((size_t)BT * (size_t)s * per * sizeof(float) + 255) & ~(size_t)255;
    }
  }
  if (p.cluster.workspace_bytes > p.workspace_bytes) p.workspace_bytes = p.cluster.workspace_bytes;
  return p;
}

// ce = lse_s - z[t]; a target outside [0, V) stores NaN (as bits)
template <typename T>
__device__ __forceinline__ void store_ce(float* ce, const T* z, int64_t t, int V, float lse_s) {
  if (t < 0 || t >= V) {
    store_nan(ce);
  } else {
    *ce = lse_s - load1(z + t);
  }
}

// ---------------------------------------------------------------- row path

// Step-1 load of the row path: a CE-only row is read exactly once (streamed),
// a CE+TVD row is read again by step 2 and keeps the default cache policy.
template <bool STREAM, typename T>
__device__ __forceinline__ void load8_row(const T* p, float (&x)[8]) {
  if (STREAM) load8_stream(p, x); else load8(p, x);
}

template <typename T, bool TEACHER, int NT>
__global__ __launch_bounds__(NT) void fwd_row_kernel(
    const T* __restrict__ student, const T* __restrict__ teacher, const int64_t* __restrict__ target,
    int64_t BT, int V, int64_t lds, int64_t ldt, int64_t ignore_index, int vec,
    float* __restrict__ ce, float* __restrict__ tvd, float* __restrict__ lse_s_out,
    float* __restrict__ lse_t_out, float* __restrict__ sigma_out) {
  __shared__ Lse red_s[NT / 64];
  __shared__ Lse red_t[NT / 64];
  __shared__ float red_f[2][NT / 64];
  const int tid = tid_x();

  for (int64_t r = bid_x(); r < BT; r += nblocks_x()) {
    const int64_t t = target[r];
    if (t == ignore_index) {
      if (tid == 0) {
        ce[r] = 0.0f;
        lse_s_out[r] = 0.0f;
        if (TEACHER) { tvd[r] = 0.0f; lse_t_out[r] = 0.0f; sigma_out[r] = 0.0f; }
      }
      continue;
    }
    const T* z = student + r * lds;
    const T* u = TEACHER ? teacher + r * ldt : nullptr;
    const RowLayout L = row_layout(z, V, vec);
    const int nsc = L.head + L.tail;
    const T* zb = z + L.head;
    const T* ub = TEACHER ? u + L.head : nullptr;

    // ---- step 1: running max / sum-exp for both rows
    Lse as = lse_init(), at = lse_init();
    for (int i = tid; i < nsc; i += NT) {
      const int e = scalar_elem(L, i);
      lse_add1(as, load1(z + e));
      if (TEACHER) lse_add1(at, load1(u + e));
    }
    int g = tid;
    for (; g + NT < L.groups; g += 2 * NT) {
      float x0[8], x1[8], y0[8], y1[8];
      load8_row<!TEACHER>(zb + 8 * g, x0);
      load8_row<!TEACHER>(zb + 8 * (g + NT), x1);
      if (TEACHER) { load8(ub + 8 * g, y0); load8(ub + 8 * (g + NT), y1); }
      lse_add8(as, x0);
      lse_add8(as, x1);
      if (TEACHER) { lse_add8(at, y0); lse_add8(at, y1); }
    }
    if (g < L.groups) {
      float x0[8], y0[8];
      load8_row<!TEACHER>(zb + 8 * g, x0);
      if (TEACHER) load8(ub + 8 * g, y0);
      lse_add8(as, x0);
      if (TEACHER) lse_add8(at, y0);
    }
    const float lse_s = lse_value(block_lse<NT>(as, red_s));
    float lse_t = 0.0f;
    if (TEACHER) lse_t = lse_value(block_lse<NT>(at, red_t));

    if (!TEACHER) {
      if (tid == 0) {
        store_ce(ce + r, z, t, V, lse_s);
        lse_s_out[r] = lse_s;
      }
      __syncthreads();  // red_s is reused by the next row
      continue;
    }

    // ---- step 2: total variation and sigma, walking the groups backwards
    const float nbs = pq_bias(lse_s), nbt = pq_bias(lse_t);
    float Q0 = 0.f, Q1 = 0.f, S0 = 0.f, S1 = 0.f;
    for (int i = tid; i < nsc; i += NT) {
      const int e = scalar_elem(L, i);
      tv_add1(load1(z + e), load1(u + e), nbs, nbt, Q0, S0);
    }
    if (tid < L.groups) {
      int gl = tid + ((L.groups - 1 - tid) / NT) * NT;  // this thread's last group
      for (; gl - NT >= 0; gl -= 2 * NT) {
        float x0[8], x1[8], y0[8], y1[8];
        load8(zb + 8 * gl, x0);
        load8(zb + 8 * (gl - NT), x1);
        load8(ub + 8 * gl, y0);
        load8(ub + 8 * (gl - NT), y1);
        tv_add8(x0, y0, nbs, nbt, Q0, Q1, S0, S1);
        tv_add8(x1, y1, nbs, nbt, Q0, Q1, S0, S1);
      }
      if (gl >= 0) {
        float x0[8], y0[8];
        load8(zb + 8 * gl, x0);
        load8(ub + 8 * gl, y0);
        tv_add8(x0, y0, nbs, nbt, Q0, Q1, S0, S1);
      }
    }
    const float Q = block_sum_t0<NT>(Q0 + Q1, red_f[0]);
    const float S = block_sum_t0<NT>(S0 + S1, red_f[1]);
    if (tid == 0) {
      store_ce(ce + r, z, t, V, lse_s);
      tvd[r] = 0.5f * ((S - Q) * kTvScale);
      lse_s_out[r] = lse_s;
      lse_t_out[r] = lse_t;
      sigma_out[r] = S * kTvScale;
    }
    __syncthreads();  // shared buffers are reused by the next row
  }
}

// ---------------------------------------------------------------- split-V path

struct ChunkRange {
  int s0, s1;  // scalar elements [s0, s1)
  int g0, g1;  // groups [g0, g1)
};

__device__ __forceinline__ ChunkRange chunk_range(const RowLayout& L, int c, int S) {
  ChunkRange R;
  const int nsc = L.head + L.tail;
  const int spc = (nsc + S - 1) / S;
  R.s0 = min(nsc, c * spc);
  R.s1 = min(nsc, R.s0 + spc);
  const int gpc = (L.groups + S - 1) / S;
  R.g0 = min(L.groups, c * gpc);
  R.g1 = min(L.groups, R.g0 + gpc);
  return R;
}

template <typename T, bool TEACHER, int NT>
__global__ __launch_bounds__(NT) void fwd_split_stage1(
    const T* __restrict__ student, const T* __restrict__ teacher, const int64_t* __restrict__ target,
    int64_t BT, int V, int64_t lds, int64_t ldt, int64_t ignore_index, int vec, int S, float* __restrict__ ws1) {
  __shared__ Lse red_s[NT / 64];
  __shared__ Lse red_t[NT / 64];
  const int tid = tid_x();
  const int64_t tiles = BT * (int64_t)S;
  for (int64_t tile = bid_x(); tile < tiles; tile += nblocks_x()) {
    const int64_t r = tile / S;
    const int c = (int)(tile - r * S);
    if (target[r] == ignore_index) continue;
    const T* z = student + r * lds;
    const T* u = TEACHER ? teacher + r * ldt : nullptr;
    const RowLayout L = row_layout(z, V, vec);
    const ChunkRange R = chunk_range(L, c, S);
    Lse as = lse_init(), at = lse_init();
    for (int i = R.s0 + tid; i < R.s1; i += NT) {
      const int e = scalar_elem(L, i);
      lse_add1(as, load1(z + e));
      if (TEACHER) lse_add1(at, load1(u + e));
    }
    const T* zb = z + L.head;
    const T* ub = TEACHER ? u + L.head : nullptr;
    for (int g = R.g0 + tid; g < R.g1; g += NT) {
      float x[8], y[8];
      load8(zb + 8 * g, x);
      if (TEACHER) load8(ub + 8 * g, y);
      lse_add8(as, x);
      if (TEACHER) lse_add8(at, y);
    }
    const Lse fs = block_lse<NT>(as, red_s);
    Lse ft{0.f, 0.f};
    if (TEACHER) ft = block_lse<NT>(at, red_t);
    if (tid == 0) {
      float* w = ws1 + tile * (TEACHER ? 4 : 2);
      w[0] = fs.m;
      w[1] = fs.s;
      if (TEACHER) { w[2] = ft.m; w[3] = ft.s; }
    }
    __syncthreads();
  }
}

template <typename T, bool TEACHER, int NT>
__global__ __launch_bounds__(NT) void fwd_split_stage2(
    const T* __restrict__ student, const T* __restrict__ teacher, const int64_t* __restrict__ target,
    int64_t BT, int V, int64_t lds, int64_t ldt, int64_t ignore_index, int vec, int S,
    const float* __restrict__ ws1,
    float* __restrict__ ws2, float* __restrict__ ce, float* __restrict__ lse_s_out,
    float* __restrict__ lse_t_out) {
  __shared__ float red_f[2][NT / 64];
  const int tid = tid_x();
  const int per = TEACHER ? S : 1;  // CE-only: one workgroup per row merges and stores
  const int64_t tiles = BT * (int64_t)per;
  for (int64_t tile = bid_x(); tile < tiles; tile += nblocks_x()) {
    const int64_t r = tile / per;
    const int c = (int)(tile - r * per);
    const int64_t t = target[r];
    if (t == ignore_index) {
      if (c == 0 && tid == 0) {
        ce[r] = 0.0f;
        lse_s_out[r] = 0.0f;
        if (TEACHER) lse_t_out[r] = 0.0f;
      }
      continue;
    }
    // merge the row's stage-1 partials in chunk order
    const float* w = ws1 + r * (int64_t)S * (TEACHER ? 4 : 2);
    Lse fs{w[0], w[1]};
    Lse ft{0.f, 0.f};
    if (TEACHER) ft = Lse{w[2], w[3]};
    for (int k = 1; k < S; ++k) {
      const float* wk = w + k * (TEACHER ? 4 : 2);
      lse_merge(fs, Lse{wk[0], wk[1]});
      if (TEACHER) lse_merge(ft, Lse{wk[2], wk[3]});
    }
    const float lse_s = lse_value(fs);
    const float lse_t = TEACHER ? lse_value(ft) : 0.0f;
    const T* z = student + r * lds;
    if (c == 0 && tid == 0) {
      store_ce(ce + r, z, t, V, lse_s);
      lse_s_out[r] = lse_s;
      if (TEACHER) lse_t_out[r] = lse_t;
    }
    if (!TEACHER) continue;

    const T* u = teacher + r * ldt;
    const RowLayout L = row_layout(z, V, vec);
    const ChunkRange R = chunk_range(L, c, S);
    const float nbs = pq_bias(lse_s), nbt = pq_bias(lse_t);
    float Q0 = 0.f, Q1 = 0.f, S0 = 0.f, S1 = 0.f;
    for (int i = R.s0 + tid; i < R.s1; i += NT) {
      const int e = scalar_elem(L, i);
      tv_add1(load1(z + e), load1(u + e), nbs, nbt, Q0, S0);
    }
    const T* zb = z + L.head;
    const T* ub = u + L.head;
    for (int g = R.g0 + tid; g < R.g1; g += NT) {
      float x[8], y[8];
      load8(zb + 8 * g, x);
      load8(ub + 8 * g, y);
      tv_add8(x, y, nbs, nbt, Q0, Q1, S0, S1);
    }
    const float Q = block_sum_t0<NT>(Q0 + Q1, red_f[0]);
    const float Sg = block_sum_t0<NT>(S0 + S1, red_f[1]);
    if (tid == 0) {
      ws2[tile * 2 + 0] = (Sg - Q) * kTvScale;  // this chunk's sum |p - q|
      ws2[tile * 2 + 1] = Sg * kTvScale;        // and sum p * sign
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void fwd_split_stage3(const int64_t* __restrict__ target, int64_t BT,
                                                        int64_t ignore_index, int S,
                                                        const float* __restrict__ ws2,
                                                        float* __restrict__ tvd, float* __restrict__ sigma) {
  for (int64_t r = bid_x() * (int64_t)bdim_x() + tid_x(); r < BT; r += (int64_t)nblocks_x() * bdim_x()) {
    if (target[r] == ignore_index) {
      tvd[r] = 0.0f;
      sigma[r] = 0.0f;
      continue;
    }
    const float* w = ws2 + r * (int64_t)S * 2;
    float A = w[0], Sg = w[1];
    for (int k = 1; k < S; ++k) {
      A += w[2 * k];
      Sg += w[2 * k + 1];
    }
    tvd[r] = 0.5f * A;
    sigma[r] = Sg;
  }
}

// ---------------------------------------------------------------- launch

template <typename T, bool TEACHER>
static hipError_t launch_forward_t(const FwdArgs& a, const FwdPlan& plan, hipStream_t st) {
  (void)hipGetLastError();  // drop an error left by an earlier, unrelated call
  const T* zs = static_cast<const T*>(a.student);
  const T* us = static_cast<const T*>(a.teacher);
  const int V = (int)a.V;
  if (plan.split <= 1) {
    const int grid = (int)(a.BT < kMaxGrid ? a.BT : kMaxGrid);
    hipLaunchKernelGGL((fwd_row_kernel<T, TEACHER, kRowThreads>), dim3(grid), dim3(kRowThreads), 0, st,
                       zs, us, a.target, a.BT, V, a.lds, a.ldt, a.ignore_index, a.vec, a.ce, a.tvd, a.lse_s,
                       a.lse_t, a.sigma);
    return hipGetLastError();
  }
  const int S = plan.split;
  float* ws1 = static_cast<float*>(a.workspace);
  float* ws2 = ws1 + a.BT * (int64_t)S * (TEACHER ? 4 : 2);
  const int64_t tiles = a.BT * (int64_t)S;
  const int g1 = (int)(tiles < kMaxGrid ? tiles : kMaxGrid);
  hipLaunchKernelGGL((fwd_split_stage1<T, TEACHER, kSplitThreads>), dim3(g1), dim3(kSplitThreads), 0, st,
                     zs, us, a.target, a.BT, V, a.lds, a.ldt, a.ignore_index, a.vec, S, ws1);
  const int64_t tiles2 = TEACHER ? tiles : a.BT;
  const int g2 = (int)(tiles2 < kMaxGrid ? tiles2 : kMaxGrid);
  hipLaunchKernelGGL((fwd_split_stage2<T, TEACHER, kSplitThreads>), dim3(g2), dim3(kSplitThreads), 0, st,
                     zs, us, a.target, a.BT, V, a.lds, a.ldt, a.ignore_index, a.vec, S, ws1, ws2, a.ce, a.lse_s,
                     a.lse_t);
  if (TEACHER) {
    const int64_t b3 = (a.BT + 255) / 256;
    const int g3 = (int)(b3 < kMaxGrid ? b3 : kMaxGrid);
    hipLaunchKernelGGL(fwd_split_stage3, dim3(g3), dim3(256), 0, st, a.target, a.BT, a.ignore_index, S, ws2,
                       a.tvd, a.sigma);
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_forward_dt(const FwdArgs& a, const FwdPlan& plan, hipStream_t stream) {
  return a.teacher ? launch_forward_t<T, true>(a, plan, stream) : launch_forward_t<T, false>(a, plan, stream);
}

hipError_t launch_forward(const FwdArgs& a, const FwdPlan& plan, Dt dt, hipStream_t stream) {
  // the read-once path needs every student and teacher row on a 16-byte boundary
  if (plan.cluster.K > 0 && a.rows16) return launch_forward_cluster(a, plan.cluster, dt, stream);
  switch (dt) {
    case Dt::BF16: return launch_forward_dt<uint16_t>(a, plan, stream);
    case Dt::F16: return launch_forward_dt<_Float16>(a, plan, stream);
    default: return launch_forward_dt<float>(a, plan, stream);
  }
}

}  // namespace lx
