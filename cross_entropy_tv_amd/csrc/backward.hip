// Backward kernel of the fused CE + TVD loss.
//
// The "Backward Pass" section of the Liger-Kernel PR #1384 analysis page: the
// logits are streamed again, p and q are recomputed from the forward's stored
// log-sum-exps, and the student gradient
//
//   g_v = k * ( g_ce * (p_v - [v == t]) + g_tvd * 0.5 * p_v * (s_v - sigma) ),
//   s_v = sign(p_v - q_v), sign(0) = 0,
//
// is written, with the target element's -g_ce added by the lane that owns it.
// g_ce and g_tvd may carry per-row factors (the upstream gradient of an
// unreduced, per-row loss), read once per (row, chunk).
// Per row this is p_v * (alpha + beta * s_v) with alpha = k * (g_ce - 0.5 *
// g_tvd * sigma) and beta = 0.5 * k * g_tvd.  The sign is read off the
// exponent arguments of p and q (common.hpp), so q itself is never formed:
// each element costs one exponential, two argument FMAs, a clamp and two FMAs.
//
// The same kernel serves a column shard of a vocabulary-parallel layout: the
// row then holds columns [v0, v0 + V) of V_total, the target still indexes
// the whole row, and only the shard that holds it subtracts g_ce.
//
// Work is tiled over (row, chunk) with a grid-stride loop; each lane reads an
// element group before it writes the same group, so the gradient may be the
// student buffer itself (in place).  Ignored rows are only written (+0.0),
// never read.
#include "common.hpp"
#include "launch.hpp"

namespace lx {

// 256 threads x 2 groups of 8 elements per lane: chunks of 4096 elements, so a
// launch has hundreds of thousands of short workgroups.  On the 8192 x 151936
// training batch (CE+TVD, one device): 256 x 2 1.196 ms, 128 x 2 1.21,
// 512 x 1 1.22, 256 x 1 1.23, 512 x 2 1.27, 64 x 4 1.30, 128 x 1 1.48.
constexpr int kBwdThreads = 256;
constexpr int kBwdUnroll = 2;  // groups of 8 elements per lane per chunk
constexpr int kBwdGroupsPerChunk = kBwdThreads * kBwdUnroll;
constexpr int kMaxGrid = 1 << 20;

// TG: the gradient's element type (T, or bf16 for the fp32 logits of the
// linear path, whose gradient feeds bf16 matrix products).
template <typename T, bool TEACHER, int NT, int UNR, typename TG = T>
__global__ __launch_bounds__(NT) void bwd_kernel(
    TG* grad, const T* student, const T* __restrict__ teacher, const int64_t* __restrict__ target,
    int64_t BT, int V, int64_t ldg, int64_t lds, int64_t ldt, int64_t v0, int64_t V_total,
    int64_t ignore_index, int vec, int chunks_per_row,
    const float* __restrict__ lse_s, const float* __restrict__ lse_t, const float* __restrict__ sigma,
    float g_ce, float g_tvd, const float* __restrict__ gce_rows, const float* __restrict__ gtvd_rows,
    const float* __restrict__ g_scale) {
  const int tid = tid_x();
  const float k = g_scale ? *g_scale : 1.0f;
  const int64_t tiles = BT * (int64_t)chunks_per_row;
  for (int64_t tile = bid_x(); tile < tiles; tile += nblocks_x()) {
    const int64_t r = tile / chunks_per_row;
    const int c = (int)(tile - r * chunks_per_row);
    const int64_t t = target[r];
    TG* gr = grad + r * ldg;
    const T* z = student + r * lds;
    const T* u = TEACHER ? teacher + r * ldt : nullptr;
    const RowLayout L = row_layout(z, V, vec);
    const int nsc = L.head + L.tail;
    // this chunk's groups and scalar elements
    const int g0 = c * (NT * UNR);
    const int g1 = min(L.groups, g0 + NT * UNR);
    const int s0 = c * (NT * UNR * 8);
    const int s1 = min(nsc, s0 + NT * UNR * 8);
    TG* gb = gr + L.head;
    const T* zb = z + L.head;
    const T* ub = TEACHER ? u + L.head : nullptr;

    if (t == ignore_index || t < 0 || t >= V_total) {
      // ignored row: +0.0; invalid target: NaN (the loud failure of the ABI contract)
      const uint32_t fill = (t == ignore_index) ? 0u : kQNaN32;
      for (int i = s0 + tid; i < s1; i += NT) store_bits1(gr + scalar_elem(L, i), fill);
      for (int g = g0 + tid; g < g1; g += NT) store_bits8(gb + 8 * g, fill);
      continue;
    }

    // with a teacher p' = 2^kPqBias * p and the sign come from the biased
    // arguments the forward used (sign_eps), so alpha and beta are rescaled:
    // g = p' * (a' + b' * s') = p * (alpha + beta * sign)
    // the target's column within this row's V columns, -1 when it lies outside
    const int tc = (t >= v0 && t - v0 < V) ? (int)(t - v0) : -1;
    const float nbs = TEACHER ? pq_bias(lse_s[r]) : neg_scaled(lse_s[r]);
    const float nbt = TEACHER ? pq_bias(lse_t[r]) : 0.0f;
    const float kce = k * g_ce * (gce_rows ? gce_rows[r] : 1.0f);
    const float beta = TEACHER ? 0.5f * k * g_tvd * (gtvd_rows ? gtvd_rows[r] : 1.0f) : 0.0f;
    const float alpha = TEACHER ? kce - beta * sigma[r] : kce;
    const float a1 = TEACHER ? alpha * 0x1p-15f : alpha;
    const float b1 = beta * kTvScale;
    static_assert(kPqBias == 15.0f, "a1 undoes the bias");

    for (int i = s0 + tid; i < s1; i += NT) {
      const int e = scalar_elem(L, i);
      const float ap = exparg(load1(z + e), nbs);
      float gv;
      if (TEACHER) {
        gv = exp2_hw(ap) * __builtin_fmaf(sign_eps(ap, exparg(load1(u + e), nbt)), b1, a1);
      } else {
        gv = exp2_hw(ap) * a1;
      }
      if (e == tc) gv -= kce;
      store1(gr + e, gv);
    }

#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const int g = g0 + j * NT + tid;
      if (g < g1) {
        float x[8], y[8], o[8];
        load8_stream(zb + 8 * g, x);
        if (TEACHER) load8_stream(ub + 8 * g, y);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float ap = exparg(x[e], nbs);
          if (TEACHER) {
            o[e] = exp2_hw(ap) * __builtin_fmaf(sign_eps(ap, exparg(y[e], nbt)), b1, a1);
          } else {
            o[e] = exp2_hw(ap) * a1;
          }
        }
        const int rel = tc - (L.head + 8 * g);
        if ((unsigned)rel < 8u) {
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = (e == rel) ? o[e] - kce : o[e];
        }
        store8_stream(gb + 8 * g, o);
      }
    }
  }
}

template <typename T, bool TEACHER, typename TG = T>
static hipError_t launch_backward_t(const BwdArgs& a, hipStream_t st) {
  (void)hipGetLastError();  // drop an error left by an earlier, unrelated call
  const int V = (int)a.V;
  // chunks needed by the longest layout: groups (vector path) or scalar elements
  const int64_t per_chunk_groups = kBwdGroupsPerChunk;
  const int64_t cpr = a.vec ? (a.V / 8 + per_chunk_groups - 1) / per_chunk_groups
                            : (a.V + per_chunk_groups * 8 - 1) / (per_chunk_groups * 8);
  const int chunks = (int)(cpr < 1 ? 1 : cpr);
  const int64_t tiles = a.BT * (int64_t)chunks;
  const int grid = (int)(tiles < kMaxGrid ? tiles : kMaxGrid);
  hipLaunchKernelGGL((bwd_kernel<T, TEACHER, kBwdThreads, kBwdUnroll, TG>), dim3(grid), dim3(kBwdThreads), 0, st,
                     static_cast<TG*>(a.grad), static_cast<const T*>(a.student), static_cast<const T*>(a.teacher),
                     a.target, a.BT, V, a.ldg, a.lds, a.ldt, a.v0, a.V_total, a.ignore_index, a.vec, chunks, a.lse_s,
                     a.lse_t, a.sigma, a.g_ce, a.g_tvd, a.gce_rows, a.gtvd_rows, a.g_scale);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_backward_dt(const BwdArgs& a, hipStream_t stream) {
  return a.teacher ? launch_backward_t<T, true>(a, stream) : launch_backward_t<T, false>(a, stream);
}

hipError_t launch_backward_f32_to_bf16(const BwdArgs& a, hipStream_t stream) {
  return a.teacher ? launch_backward_t<float, true, uint16_t>(a, stream)
                   : launch_backward_t<float, false, uint16_t>(a, stream);
}

hipError_t launch_backward(const BwdArgs& a, Dt dt, hipStream_t stream) {
  switch (dt) {
    case Dt::BF16: return launch_backward_dt<uint16_t>(a, stream);
    case Dt::F16: return launch_backward_dt<_Float16>(a, stream);
    default: return launch_backward_dt<float>(a, stream);
  }
}

}  // namespace lx
