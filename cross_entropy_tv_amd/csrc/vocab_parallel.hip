// Vocabulary-parallel (column-sharded) pieces of the fused CE + TVD loss.
//
// With the vocabulary split over N devices (a sharded lm_head), device n holds
// columns [v0_n, v0_n + Vs_n) of every row.  The two steps of the "Forward
// Pass" section of the Liger-Kernel PR #1384 analysis page then each need one
// exchange across the shards:
//
//   1. vp_stats: per row and shard, the (max, sum-exp) pairs of student and
//      teacher over the shard, and the target logit if the shard holds the
//      target column (+0 otherwise).  vp_merge_stats merges the N partials in
//      shard order (the (max, sum-exp) merge of step 1, and a plain sum of the
//      target-logit parts, exactly one of which is non-zero) into lse_s,
//      lse_t and ce = lse_s - z_t.
//   2. vp_tv: per row and shard, (sum |p - q|, sum p * sign(p - q)) over the
//      shard from the global log-sum-exps, with the same arguments and sign
//      rule as every other kernel here (common.hpp).  vp_merge_tv adds the N
//      partials in shard order into tvd = 0.5 * sum |p - q| and sigma.
//
// Between the steps the partials travel between devices (an all-gather of
// 20 bytes per row and shard after step 1, 8 after step 2); on one device the
// merge kernels read the gathered [N][BT][.] arrays directly.  The backward
// needs no exchange (the backward kernel runs on the shard with the target
// column offset).  Merges run in shard order, so results are deterministic
// and do not depend on how the exchange is ordered.
#include "common.hpp"
#include "launch.hpp"

namespace lx {

namespace {

constexpr int kVpThreads = 256;
constexpr int kVpUnits = 10;  // 16-byte units per thread and tensor held at once
constexpr int kVpMergeThreads = 256;
constexpr int kMaxGrid = 1 << 20;

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// A 16-byte unit of logits widened to f32: 8 bf16 or binary16 logits, or 4 fp32.
template <typename T>
struct Unit;
template <>
struct Unit<uint16_t> {
  static constexpr int E = 8;
  static __device__ __forceinline__ void get(const u32x4_t& w, float (&x)[8]) {
    const unsigned w0 = w.x, w1 = w.y, w2 = w.z, w3 = w.w;  // copied out: see the one-pass kernels
    x[0] = __uint_as_float(w0 << 16); x[1] = __uint_as_float(w0 & 0xffff0000u);
    x[2] = __uint_as_float(w1 << 16); x[3] = __uint_as_float(w1 & 0xffff0000u);
    x[4] = __uint_as_float(w2 << 16); x[5] = __uint_as_float(w2 & 0xffff0000u);
    x[6] = __uint_as_float(w3 << 16); x[7] = __uint_as_float(w3 & 0xffff0000u);
  }
};
template <>
struct Unit<_Float16> {
  static constexpr int E = 8;
  static __device__ __forceinline__ void get(const u32x4_t& w, float (&x)[8]) {
    const unsigned w0 = w.x, w1 = w.y, w2 = w.z, w3 = w.w;
    unpack_f16x2(w0, x[0], x[1]); unpack_f16x2(w1, x[2], x[3]);
    unpack_f16x2(w2, x[4], x[5]); unpack_f16x2(w3, x[6], x[7]);
  }
};
template <>
struct Unit<float> {
  static constexpr int E = 4;
  static __device__ __forceinline__ void get(const u32x4_t& w, float (&x)[4]) {
    const unsigned w0 = w.x, w1 = w.y, w2 = w.z, w3 = w.w;
    x[0] = __uint_as_float(w0); x[1] = __uint_as_float(w1);
    x[2] = __uint_as_float(w2); x[3] = __uint_as_float(w3);
  }
};
constexpr int kRsrcFlags = 0x00020000;  // buffer resource word 3 for gfx9-family raw buffers
constexpr int kStreamPolicy = 2;        // non-temporal loads: every logit is read once

// Hides a held unit from common-subexpression elimination, so that the
// compiler keeps the 16 packed bytes (4 registers) until each use rather
// than the widened floats (8).
__device__ __forceinline__ void launder(u32x4_t& w) {
  unsigned a = w.x, b = w.y, c = w.z, d = w.w;
  asm volatile("" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
  w = (u32x4_t){a, b, c, d};
}

// Units [c, c + NT * U) of a row body of nu units: thread tid holds units
// c + tid + k * NT, k < n, all requested at once.  The loads go through a
// buffer resource covering just these units, so those past the body's end
// return 0 without touching memory and need no branch (w[k], k >= n, is
// never read).
template <typename T, int NT, int U>
__device__ __forceinline__ int load_units(const T* body, int nu, int c, int tid, u32x4_t (&w)[U]) {
  constexpr int E = Unit<T>::E;
  const int cnt = min(nu - c, NT * U);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(body + (int64_t)c * E), (short)0, cnt * 16, kRsrcFlags);
#pragma unroll
  for (int k = 0; k < U; ++k)
    w[k] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, (tid + k * NT) * 16, 0,
                                                                            kStreamPolicy));
  return tid < cnt ? min(U, (cnt - tid - 1) / NT + 1) : 0;
}

// (max, sum-exp) of n >= 1 held units merged into a: the sum is taken against
// the maximum of the first unit (no rescaling per unit); a logit ~69 above it
// takes the sum to kRefSumLimit, and then the sum is redone against the
// units' maximum.
template <typename T, int U>
__device__ __forceinline__ void units_lse(u32x4_t (&w)[U], int n, Lse& a) {
  constexpr int E = Unit<T>::E;
  float x[E];
  Unit<T>::get(w[0], x);
  float m = kMFloor;  // a floor, so that units of -inf logits give exp2(-inf) = 0, never inf - inf
#pragma unroll
  for (int e = 0; e < E; ++e) m = fmaxf(m, x[e]);
  float s0 = 0.0f, s1 = 0.0f;
  {
    const float nb = -(m * kLog2e);
#pragma unroll
    for (int k = 0; k < U; ++k) {
      if (k < n) {
        launder(w[k]);
        Unit<T>::get(w[k], x);
#pragma unroll
        for (int e = 0; e < E; e += 2) {
          s0 += exp2_hw(__builtin_fmaf(x[e], kLog2e, nb));
          s1 += exp2_hw(__builtin_fmaf(x[e + 1], kLog2e, nb));
        }
      }
    }
  }
  if (!(s0 + s1 < kRefSumLimit)) {
#pragma unroll
    for (int k = 1; k < U; ++k) {
      if (k < n) {
        launder(w[k]);
        Unit<T>::get(w[k], x);
#pragma unroll
        for (int e = 0; e < E; ++e) m = fmaxf(m, x[e]);
      }
    }
    const float nb = -(m * kLog2e);
    s0 = s1 = 0.0f;
#pragma unroll
    for (int k = 0; k < U; ++k) {
      if (k < n) {
        launder(w[k]);
        Unit<T>::get(w[k], x);
#pragma unroll
        for (int e = 0; e < E; e += 2) {
          s0 += exp2_hw(__builtin_fmaf(x[e], kLog2e, nb));
          s1 += exp2_hw(__builtin_fmaf(x[e + 1], kLog2e, nb));
        }
      }
    }
  }
  lse_merge(a, Lse{m, s0 + s1});
}

// One workgroup per row (grid-stride over rows): the shard's (max, sum-exp)
// pairs and its part of the target logit.  stats[r] = {m_s, s_s, m_t, s_t,
// zt} with a teacher, {m_s, s_s, zt} without; ignored rows get zeros.  Each
// thread requests up to U 16-byte units of each tensor before it works on
// any, so a row's loads are all in flight at once.
template <typename T, bool TEACHER, int NT, int U>
__global__ __launch_bounds__(NT) void vp_stats_kernel(const T* __restrict__ student, const T* __restrict__ teacher,
                                                      const int64_t* __restrict__ target, int64_t BT, int Vs,
                                                      int64_t v0, int64_t ignore_index, int vec,
                                                      float* __restrict__ stats) {
  constexpr int E = Unit<T>::E;
  __shared__ Lse red_s[NT / 64];
  __shared__ Lse red_t[NT / 64];
  constexpr int P = TEACHER ? 5 : 3;
  const int tid = tid_x();
  for (int64_t r = bid_x(); r < BT; r += nblocks_x()) {
    const int64_t t = target[r];
    float* o = stats + r * P;
    if (t == ignore_index) {
      if (tid < P) o[tid] = 0.0f;
      continue;
    }
    const T* z = student + r * (int64_t)Vs;
    const T* u = TEACHER ? teacher + r * (int64_t)Vs : nullptr;
    // the target logit, requested now so that it has long arrived at the row's end
    const int64_t tc = t - v0;
    float zt = 0.0f;
    if (tid == 0 && tc >= 0 && tc < Vs) zt = load1(z + tc);
    const RowLayout L = row_layout(z, Vs, vec);
    const int nsc = L.head + L.tail;
    const int nu = L.groups * (8 / E);
    const T* zb = z + L.head;
    const T* ub = TEACHER ? u + L.head : nullptr;
    Lse as = lse_init(), at = lse_init();
    for (int c = 0; c < nu; c += NT * U) {
      u32x4_t wz[U], wu[U];
      const int n = load_units<T, NT, U>(zb, nu, c, tid, wz);
      if (TEACHER) load_units<T, NT, U>(ub, nu, c, tid, wu);
      if (n > 0) {
        units_lse<T, U>(wz, n, as);
        if (TEACHER) units_lse<T, U>(wu, n, at);
      }
    }
    for (int i = tid; i < nsc; i += NT) {
      const int e = scalar_elem(L, i);
      lse_add1(as, load1(z + e));
      if (TEACHER) lse_add1(at, load1(u + e));
    }
    const Lse fs = block_lse<NT>(as, red_s);
    Lse ft{0.0f, 0.0f};
    if (TEACHER) ft = block_lse<NT>(at, red_t);
    if (tid == 0) {
      o[0] = fs.m;
      o[1] = fs.s;
      if (TEACHER) {
        o[2] = ft.m;
        o[3] = ft.s;
      }
      o[P - 1] = zt;
    }
    __syncthreads();  // red_s / red_t are reused by the next row
  }
}

// One thread per row: the N shards' stats merged in shard order.
template <bool TEACHER>
__global__ __launch_bounds__(kVpMergeThreads) void vp_merge_stats_kernel(
    const float* __restrict__ stats, int N, int64_t BT, const int64_t* __restrict__ target, int64_t V,
    int64_t ignore_index, float* __restrict__ ce, float* __restrict__ lse_s, float* __restrict__ lse_t,
    float* __restrict__ zt_out) {
  constexpr int P = TEACHER ? 5 : 3;
  for (int64_t r = bid_x() * (int64_t)bdim_x() + tid_x(); r < BT; r += (int64_t)nblocks_x() * bdim_x()) {
    const int64_t t = target[r];
    if (t == ignore_index) {
      ce[r] = 0.0f;
      lse_s[r] = 0.0f;
      if (TEACHER) lse_t[r] = 0.0f;
      if (zt_out) zt_out[r] = 0.0f;
      continue;
    }
    const float* w = stats + r * P;
    const int64_t shard_stride = BT * P;
    Lse fs{w[0], w[1]};
    Lse ft{TEACHER ? w[2] : 0.0f, TEACHER ? w[3] : 0.0f};
    float zt = w[P - 1];
    for (int n = 1; n < N; ++n) {
      const float* wn = w + n * shard_stride;
      lse_merge(fs, Lse{wn[0], wn[1]});
      if (TEACHER) lse_merge(ft, Lse{wn[2], wn[3]});
      zt += wn[P - 1];
    }
    const float ls = lse_value(fs);
    if (t >= 0 && t < V) ce[r] = ls - zt; else store_nan(ce + r);
    lse_s[r] = ls;
    if (TEACHER) lse_t[r] = lse_value(ft);
    if (zt_out) zt_out[r] = zt;  // the target logit itself
  }
}

// One workgroup per row: the shard's (sum |p - q|, sum p * sign) from the
// global log-sum-exps; ignored rows get zeros.  Loads as vp_stats_kernel.
template <typename T, int NT, int U>
__global__ __launch_bounds__(NT) void vp_tv_kernel(const T* __restrict__ student, const T* __restrict__ teacher,
                                                   const int64_t* __restrict__ target, int64_t BT, int Vs,
                                                   int64_t ignore_index, int vec, const float* __restrict__ lse_s,
                                                   const float* __restrict__ lse_t, float* __restrict__ tv) {
  constexpr int E = Unit<T>::E;
  __shared__ float red_f[2][NT / 64];
  const int tid = tid_x();
  for (int64_t r = bid_x(); r < BT; r += nblocks_x()) {
    const int64_t t = target[r];
    if (t == ignore_index) {
      if (tid < 2) tv[2 * r + tid] = 0.0f;
      continue;
    }
    const T* z = student + r * (int64_t)Vs;
    const T* u = teacher + r * (int64_t)Vs;
    const RowLayout L = row_layout(z, Vs, vec);
    const int nsc = L.head + L.tail;
    const int nu = L.groups * (8 / E);
    const float nbs = pq_bias(lse_s[r]), nbt = pq_bias(lse_t[r]);
    float Q0 = 0.f, Q1 = 0.f, S0 = 0.f, S1 = 0.f;
    for (int c = 0; c < nu; c += NT * U) {
      u32x4_t wz[U], wu[U];
      const int n = load_units<T, NT, U>(z + L.head, nu, c, tid, wz);
      load_units<T, NT, U>(u + L.head, nu, c, tid, wu);
#pragma unroll
      for (int k = 0; k < U; ++k) {
        if (k < n) {
          float x[E], y[E];
          Unit<T>::get(wz[k], x);
          Unit<T>::get(wu[k], y);
#pragma unroll
          for (int e = 0; e < E; e += 2) {
            tv_add1(x[e], y[e], nbs, nbt, Q0, S0);
            tv_add1(x[e + 1], y[e + 1], nbs, nbt, Q1, S1);
          }
        }
      }
    }
    for (int i = tid; i < nsc; i += NT) {
      const int e = scalar_elem(L, i);
      tv_add1(load1(z + e), load1(u + e), nbs, nbt, Q0, S0);
    }
    const float Q = block_sum_t0<NT>(Q0 + Q1, red_f[0]);
    const float S = block_sum_t0<NT>(S0 + S1, red_f[1]);
    if (tid == 0) {
      tv[2 * r] = (S - Q) * kTvScale;
      tv[2 * r + 1] = S * kTvScale;
    }
    __syncthreads();  // red_f is reused by the next row
  }
}

// One thread per row: the N shards' (sum |p - q|, sum p * sign) added in
// shard order.
__global__ __launch_bounds__(kVpMergeThreads) void vp_merge_tv_kernel(
    const float* __restrict__ tv, int N, int64_t BT, const int64_t* __restrict__ target, int64_t ignore_index,
    float* __restrict__ tvd, float* __restrict__ sigma) {
  for (int64_t r = bid_x() * (int64_t)bdim_x() + tid_x(); r < BT; r += (int64_t)nblocks_x() * bdim_x()) {
    if (target[r] == ignore_index) {
      tvd[r] = 0.0f;
      sigma[r] = 0.0f;
      continue;
    }
    float A = tv[2 * r], S = tv[2 * r + 1];
    for (int n = 1; n < N; ++n) {
      const float* w = tv + (int64_t)n * BT * 2 + 2 * r;
      A += w[0];
      S += w[1];
    }
    tvd[r] = 0.5f * A;
    sigma[r] = S;
  }
}

int row_grid(int64_t BT) { return (int)(BT < kMaxGrid ? BT : kMaxGrid); }
int merge_grid(int64_t BT) {
  const int64_t b = (BT + kVpMergeThreads - 1) / kVpMergeThreads;
  return (int)(b < kMaxGrid ? b : kMaxGrid);
}

template <typename T>
hipError_t launch_vp_stats_t(const VpArgs& a, hipStream_t st) {
  (void)hipGetLastError();
  const T* z = static_cast<const T*>(a.student);
  const T* u = static_cast<const T*>(a.teacher);
  if (u) {
    hipLaunchKernelGGL((vp_stats_kernel<T, true, kVpThreads, kVpUnits>), dim3(row_grid(a.BT)), dim3(kVpThreads), 0, st, z,
                       u, a.target, a.BT, (int)a.Vs, a.v0, a.ignore_index, a.vec, a.out);
  } else {
    hipLaunchKernelGGL((vp_stats_kernel<T, false, kVpThreads, kVpUnits>), dim3(row_grid(a.BT)), dim3(kVpThreads), 0, st,
                       z, u, a.target, a.BT, (int)a.Vs, a.v0, a.ignore_index, a.vec, a.out);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_vp_tv_t(const VpArgs& a, hipStream_t st) {
  (void)hipGetLastError();
  hipLaunchKernelGGL((vp_tv_kernel<T, kVpThreads, kVpUnits>), dim3(row_grid(a.BT)), dim3(kVpThreads), 0, st,
                     static_cast<const T*>(a.student), static_cast<const T*>(a.teacher), a.target, a.BT, (int)a.Vs,
                     a.ignore_index, a.vec, a.lse_s, a.lse_t, a.out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_vp_stats(const VpArgs& a, Dt dt, hipStream_t st) {
  switch (dt) {
    case Dt::BF16: return launch_vp_stats_t<uint16_t>(a, st);
    case Dt::F16: return launch_vp_stats_t<_Float16>(a, st);
    default: return launch_vp_stats_t<float>(a, st);
  }
}

hipError_t launch_vp_tv(const VpArgs& a, Dt dt, hipStream_t st) {
  switch (dt) {
    case Dt::BF16: return launch_vp_tv_t<uint16_t>(a, st);
    case Dt::F16: return launch_vp_tv_t<_Float16>(a, st);
    default: return launch_vp_tv_t<float>(a, st);
  }
}

hipError_t launch_vp_merge_stats_zt(const float* stats, int64_t N, const int64_t* target, int64_t BT, int64_t V,
                                    int64_t ignore_index, bool teacher, float* ce, float* lse_s, float* lse_t,
                                    float* zt, hipStream_t st) {
  (void)hipGetLastError();
  if (teacher) {
    hipLaunchKernelGGL((vp_merge_stats_kernel<true>), dim3(merge_grid(BT)), dim3(kVpMergeThreads), 0, st, stats,
                       (int)N, BT, target, V, ignore_index, ce, lse_s, lse_t, zt);
  } else {
    hipLaunchKernelGGL((vp_merge_stats_kernel<false>), dim3(merge_grid(BT)), dim3(kVpMergeThreads), 0, st, stats,
                       (int)N, BT, target, V, ignore_index, ce, lse_s, lse_t, zt);
  }
  return hipGetLastError();
}

hipError_t launch_vp_merge_stats(const float* stats, int64_t N, const int64_t* target, int64_t BT, int64_t V,
                                 int64_t ignore_index, bool teacher, float* ce, float* lse_s, float* lse_t,
                                 hipStream_t st) {
  return launch_vp_merge_stats_zt(stats, N, target, BT, V, ignore_index, teacher, ce, lse_s, lse_t, nullptr, st);
}

hipError_t launch_vp_merge_tv(const float* tv, int64_t N, const int64_t* target, int64_t BT, int64_t ignore_index,
                              float* tvd, float* sigma, hipStream_t st) {
  (void)hipGetLastError();
  hipLaunchKernelGGL(vp_merge_tv_kernel, dim3(merge_grid(BT)), dim3(kVpMergeThreads), 0, st, tv, (int)N, BT, target,
                     ignore_index, tvd, sigma);
  return hipGetLastError();
}

}  // namespace lx
