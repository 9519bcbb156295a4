// Device helpers shared by the CE + TVD kernels (gfx950, wave64).
//
// Numerics (the same helpers serve the forward and the backward, so both
// passes form p, q and sign(p - q) with the same instruction sequence):
//   * logits are widened to f32 (bf16 and binary16 -> f32 are exact), all
//     arithmetic is f32;
//   * exp(x - lse) is evaluated as exp2(fma(x, log2 e, -lse * log2 e)), one
//     rounding before the hardware v_exp_f32;
//   * running maxima start at kMFloor, a finite floor, so every rescale factor
//     exp2((m_old - m_new) * log2 e) is finite (no inf - inf) even for rows
//     holding -inf entries;
//   * the total variation forms p and q scaled by 2^15 (the exponent bias
//     raised by 15, pq_bias) from the arguments a = fma(x, log2 e, bias), and
//     reads sign(p - q) off the arguments: p - q has the sign of a_p - a_q
//     wherever fp32 resolves the two (elsewhere |p / q - 1| is a few 2^-20, a
//     near tie), and med3(a_p - a_q, -2^-24, 2^-24) is 2^-24 * sign, with
//     sign 0 exactly when the arguments are equal, and a fraction of 2^-24
//     only where |a_p - a_q| < 2^-24 (|p / q - 1| < 4e-8).  The forward sums
//     S = sum p s and Q = sum q s, so sum |p - q| = S - Q; the backward needs
//     no q at all.  Forward and backward form the arguments from the same
//     stored lse with the same instructions, so sigma and the backward's
//     signs agree element for element.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ids.hpp"

namespace lx {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kMFloor = -1.0e30f;
// A thread's sum of exponentials taken against a reference maximum (its first
// group's) is redone against its true maximum once it reaches 2^100 (a logit
// ~69 above the reference): every such partial is then below 2^100 + the
// count of its terms, so the merges of up to 2^27 of them (lanes, waves,
// members or chunks, shards) cannot overflow fp32.
constexpr float kRefSumLimit = 0x1p100f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ loads

// 8 consecutive logits at a 16-byte-aligned address, widened to f32.
__device__ __forceinline__ void load8(const uint16_t* p, float (&x)[8]) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  x[0] = __uint_as_float(w.x << 16); x[1] = __uint_as_float(w.x & 0xffff0000u);
  x[2] = __uint_as_float(w.y << 16); x[3] = __uint_as_float(w.y & 0xffff0000u);
  x[4] = __uint_as_float(w.z << 16); x[5] = __uint_as_float(w.z & 0xffff0000u);
  x[6] = __uint_as_float(w.w << 16); x[7] = __uint_as_float(w.w & 0xffff0000u);
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
typedef unsigned u32x4v_t __attribute__((ext_vector_type(4)));

// As load8, with a non-temporal (streamed once) cache policy: for data that is
// not read again by this kernel.  On the training batch this takes the
// backward from 1.40 to 1.31 ms together with store8_stream.
__device__ __forceinline__ void load8_stream(const uint16_t* p, float (&x)[8]) {
  const u32x4v_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x4v_t*>(p));
  x[0] = __uint_as_float(w.x << 16); x[1] = __uint_as_float(w.x & 0xffff0000u);
  x[2] = __uint_as_float(w.y << 16); x[3] = __uint_as_float(w.y & 0xffff0000u);
  x[4] = __uint_as_float(w.z << 16); x[5] = __uint_as_float(w.z & 0xffff0000u);
  x[6] = __uint_as_float(w.w << 16); x[7] = __uint_as_float(w.w & 0xffff0000u);
}
__device__ __forceinline__ void load8_stream(const float* p, float (&x)[8]) {
  typedef float f32x4v_t __attribute__((ext_vector_type(4)));
  const f32x4v_t a = __builtin_nontemporal_load(reinterpret_cast<const f32x4v_t*>(p));
  const f32x4v_t b = __builtin_nontemporal_load(reinterpret_cast<const f32x4v_t*>(p) + 1);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ float load1(const uint16_t* p) { return __uint_as_float((uint32_t)(*p) << 16); }
__device__ __forceinline__ float load1(const float* p) { return *p; }

// IEEE binary16 logits: widened to f32 exactly (v_cvt_f32_f16).
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void unpack_f16x2(uint32_t w, float& a, float& b) {
  const f16x2_t h = __builtin_bit_cast(f16x2_t, w);
  a = (float)h.x;
  b = (float)h.y;
}
__device__ __forceinline__ void load8(const _Float16* p, float (&x)[8]) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  unpack_f16x2(w.x, x[0], x[1]); unpack_f16x2(w.y, x[2], x[3]);
  unpack_f16x2(w.z, x[4], x[5]); unpack_f16x2(w.w, x[6], x[7]);
}
__device__ __forceinline__ void load8_stream(const _Float16* p, float (&x)[8]) {
  const u32x4v_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x4v_t*>(p));
  const uint32_t w0 = w.x, w1 = w.y, w2 = w.z, w3 = w.w;
  unpack_f16x2(w0, x[0], x[1]); unpack_f16x2(w1, x[2], x[3]);
  unpack_f16x2(w2, x[4], x[5]); unpack_f16x2(w3, x[6], x[7]);
}
__device__ __forceinline__ float load1(const _Float16* p) { return (float)*p; }

// ------------------------------------------------------------------ stores

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}
__device__ __forceinline__ void store8(uint16_t* p, const float (&g)[8]) {
  uint4 w;
  w.x = pack_bf16x2(g[0], g[1]); w.y = pack_bf16x2(g[2], g[3]);
  w.z = pack_bf16x2(g[4], g[5]); w.w = pack_bf16x2(g[6], g[7]);
  *reinterpret_cast<uint4*>(p) = w;
}
__device__ __forceinline__ void store8(float* p, const float (&g)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(g[0], g[1], g[2], g[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(g[4], g[5], g[6], g[7]);
}
// As store8, non-temporal (written once, not read again by this kernel).
__device__ __forceinline__ void store8_stream(uint16_t* p, const float (&g)[8]) {
  u32x4v_t w;
  w.x = pack_bf16x2(g[0], g[1]); w.y = pack_bf16x2(g[2], g[3]);
  w.z = pack_bf16x2(g[4], g[5]); w.w = pack_bf16x2(g[6], g[7]);
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4v_t*>(p));
}
__device__ __forceinline__ void store8_stream(float* p, const float (&g)[8]) {
  typedef float f32x4v_t __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store((f32x4v_t){g[0], g[1], g[2], g[3]}, reinterpret_cast<f32x4v_t*>(p));
  __builtin_nontemporal_store((f32x4v_t){g[4], g[5], g[6], g[7]}, reinterpret_cast<f32x4v_t*>(p) + 1);
}
__device__ __forceinline__ void store1(uint16_t* p, float g) {
  *p = (uint16_t)(pack_bf16x2(g, 0.0f) & 0xffffu);
}
__device__ __forceinline__ void store1(float* p, float g) { *p = g; }

// binary16 gradients: rounded to nearest even (v_cvt_pk_f16_f32)
__device__ __forceinline__ uint32_t pack_f16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, (f16x2_t){(_Float16)a, (_Float16)b});
}
__device__ __forceinline__ void store8(_Float16* p, const float (&g)[8]) {
  uint4 w;
  w.x = pack_f16x2_rne(g[0], g[1]); w.y = pack_f16x2_rne(g[2], g[3]);
  w.z = pack_f16x2_rne(g[4], g[5]); w.w = pack_f16x2_rne(g[6], g[7]);
  *reinterpret_cast<uint4*>(p) = w;
}
__device__ __forceinline__ void store8_stream(_Float16* p, const float (&g)[8]) {
  u32x4v_t w;
  w.x = pack_f16x2_rne(g[0], g[1]); w.y = pack_f16x2_rne(g[2], g[3]);
  w.z = pack_f16x2_rne(g[4], g[5]); w.w = pack_f16x2_rne(g[6], g[7]);
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4v_t*>(p));
}
__device__ __forceinline__ void store1(_Float16* p, float g) { *p = (_Float16)g; }

// Quiet-NaN bit patterns.  The kernels are compiled with NaNs assumed absent
// from floating-point arithmetic, so a NaN the ABI promises as an output is
// written as an integer bit pattern and never produced by an FP operation.
constexpr uint32_t kQNaN32 = 0x7fc00000u;
constexpr uint16_t kQNaN16 = 0x7fc0u;      // bf16
constexpr uint16_t kQNaNHalf = 0x7e00u;    // binary16

__device__ __forceinline__ void store_bits1(uint16_t* p, uint32_t f32bits) { *p = (uint16_t)(f32bits >> 16); }
__device__ __forceinline__ void store_bits1(float* p, uint32_t f32bits) { *reinterpret_cast<uint32_t*>(p) = f32bits; }
// 8 copies of one f32 bit pattern (bf16: its upper half), stored as integers
__device__ __forceinline__ void store_bits8(uint16_t* p, uint32_t f32bits) {
  const uint32_t h = f32bits >> 16, w = h | (h << 16);
  *reinterpret_cast<uint4*>(p) = make_uint4(w, w, w, w);
}
__device__ __forceinline__ void store_bits8(float* p, uint32_t f32bits) {
  reinterpret_cast<uint4*>(p)[0] = make_uint4(f32bits, f32bits, f32bits, f32bits);
  reinterpret_cast<uint4*>(p)[1] = make_uint4(f32bits, f32bits, f32bits, f32bits);
}
// binary16: the fills are +0.0 (f32 bits 0) and a quiet NaN (any other pattern)
__device__ __forceinline__ uint16_t half_fill(uint32_t f32bits) { return f32bits ? kQNaNHalf : (uint16_t)0; }
__device__ __forceinline__ void store_bits1(_Float16* p, uint32_t f32bits) {
  *reinterpret_cast<uint16_t*>(p) = half_fill(f32bits);
}
__device__ __forceinline__ void store_bits8(_Float16* p, uint32_t f32bits) {
  const uint32_t h = half_fill(f32bits), w = h | (h << 16);
  *reinterpret_cast<uint4*>(p) = make_uint4(w, w, w, w);
}
__device__ __forceinline__ void store_nan(float* p) { *reinterpret_cast<uint32_t*>(p) = kQNaN32; }

// ------------------------------------------------------------------ math

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// -lse * log2(e): the bias every probability of the row is formed with.
__device__ __forceinline__ float neg_scaled(float lse) { return -(lse * kLog2e); }


// Total-variation arguments (see the header comment): p' = exp2(exparg(x,
// pq_bias(lse))) = 2^kPqBias * exp(x - lse), and sign_eps(a_p, a_q) =
// kSignEps * sign(p - q).  Sums of p' * sign_eps come back to sums of
// p * sign with the factor kTvScale.
constexpr float kPqBias = 15.0f;
constexpr float kSignEps = 0x1p-24f;
constexpr float kTvScale = 0x1p9f;  // 2^24 * 2^-15
__device__ __forceinline__ float pq_bias(float lse) { return neg_scaled(lse) + kPqBias; }
__device__ __forceinline__ float exparg(float x, float nb) { return __builtin_fmaf(x, kLog2e, nb); }
__device__ __forceinline__ float sign_eps(float ap, float aq) {
  return __builtin_amdgcn_fmed3f(ap - aq, -kSignEps, kSignEps);
}

__device__ __forceinline__ float max8(const float (&x)[8]) {
  return fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
}

// Online log-sum-exp state: sum_i exp(x_i - m) = s.
struct Lse {
  float m, s;
};

__device__ __forceinline__ Lse lse_init() { return Lse{kMFloor, 0.0f}; }

__device__ __forceinline__ void lse_add8(Lse& a, const float (&x)[8]) {
  const float mn = fmaxf(a.m, max8(x));
  const float nb = -(mn * kLog2e);
  float s0 = a.s * exp2_hw((a.m - mn) * kLog2e);
  float s1 = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; k += 2) {
    s0 += exp2_hw(__builtin_fmaf(x[k], kLog2e, nb));
    s1 += exp2_hw(__builtin_fmaf(x[k + 1], kLog2e, nb));
  }
  a.m = mn;
  a.s = s0 + s1;
}

__device__ __forceinline__ void lse_add1(Lse& a, float x) {
  const float mn = fmaxf(a.m, x);
  a.s = a.s * exp2_hw((a.m - mn) * kLog2e) + exp2_hw((x - mn) * kLog2e);
  a.m = mn;
}

// Merge b into a.  Both maxima are >= kMFloor, so no NaN can arise.
__device__ __forceinline__ void lse_merge(Lse& a, const Lse& b) {
  const float mn = fmaxf(a.m, b.m);
  a.s = a.s * exp2_hw((a.m - mn) * kLog2e) + b.s * exp2_hw((b.m - mn) * kLog2e);
  a.m = mn;
}

__device__ __forceinline__ float lse_value(const Lse& a) { return a.m + logf(a.s); }

// ------------------------------------------------------------------ wave / block reductions

// The wave's (max, sum-exp): the maximum first, then each lane's sum rescaled
// to it once and the sums added (one exponential per lane instead of two per
// butterfly step).  Every lane ends with the same pair.
__device__ __forceinline__ Lse wave_lse(Lse a) {
  float m = a.m;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  float s = a.s * exp2_hw((a.m - m) * kLog2e);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  return Lse{m, s};
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// ------------------------------------------------------------------ block reductions and TV sums

template <int NT>
__device__ __forceinline__ Lse block_lse(Lse a, Lse* red) {
  constexpr int W = NT / 64;
  a = wave_lse(a);
  if ((tid_x() & 63) == 0) red[tid_x() >> 6] = a;
  __syncthreads();
  Lse f = red[0];
#pragma unroll
  for (int w = 1; w < W; ++w) lse_merge(f, red[w]);
  return f;  // identical in every thread
}

template <int NT>
__device__ __forceinline__ float block_sum_t0(float v, float* red) {
  constexpr int W = NT / 64;
  v = wave_sum(v);
  if ((tid_x() & 63) == 0) red[tid_x() >> 6] = v;
  __syncthreads();
  float f = 0.0f;
  if (tid_x() == 0) {
    f = red[0];
#pragma unroll
    for (int w = 1; w < W; ++w) f += red[w];
  }
  return f;  // valid in thread 0
}

// step-2 accumulation for one group of 8, nbs and nbt from pq_bias:
// S += p' * s' and Q += q' * s' (s' = sign_eps), so that, scaled by
// kTvScale, S is sum p * sign and S - Q is sum |p - q|
__device__ __forceinline__ void tv_add8(const float (&x)[8], const float (&y)[8], float nbs, float nbt,
                                        float& Q0, float& Q1, float& S0, float& S1) {
#pragma unroll
  for (int k = 0; k < 8; k += 2) {
    const float ap0 = exparg(x[k], nbs), aq0 = exparg(y[k], nbt);
    const float ap1 = exparg(x[k + 1], nbs), aq1 = exparg(y[k + 1], nbt);
    const float s0 = sign_eps(ap0, aq0), s1 = sign_eps(ap1, aq1);
    S0 = __builtin_fmaf(exp2_hw(ap0), s0, S0);
    Q0 = __builtin_fmaf(exp2_hw(aq0), s0, Q0);
    S1 = __builtin_fmaf(exp2_hw(ap1), s1, S1);
    Q1 = __builtin_fmaf(exp2_hw(aq1), s1, Q1);
  }
}

__device__ __forceinline__ void tv_add1(float x, float y, float nbs, float nbt, float& Q, float& S) {
  const float ap = exparg(x, nbs), aq = exparg(y, nbt);
  const float s = sign_eps(ap, aq);
  S = __builtin_fmaf(exp2_hw(ap), s, S);
  Q = __builtin_fmaf(exp2_hw(aq), s, Q);
}

// ------------------------------------------------------------------ row layout

// A row of V elements starting at `row` is cut into a scalar head [0, head),
// body groups of 8 elements [head, head + 8 * groups) that start on a
// 16-byte boundary, and a scalar tail.  With vec == 0 every element is
// scalar (head = V, groups = 0).
struct RowLayout {
  int head, groups, tail;
};

template <typename T>
__device__ __forceinline__ RowLayout row_layout(const T* row, int V, int vec) {
  RowLayout L;
  if (!vec) {
    L.head = V; L.groups = 0; L.tail = 0;
    return L;
  }
  const int mis = (int)((16u - ((uint32_t)(uintptr_t)row & 15u)) & 15u) / (int)sizeof(T);
  L.head = mis < V ? mis : V;
  L.groups = (V - L.head) / 8;
  L.tail = V - L.head - 8 * L.groups;
  return L;
}

// i-th scalar element (0 <= i < head + tail) of the row.
__device__ __forceinline__ int scalar_elem(const RowLayout& L, int i) {
  return i < L.head ? i : L.head + 8 * L.groups + (i - L.head);
}

}  // namespace lx
