// Device-side building blocks shared by the conv3x3 kernels: vector types,
// the MFMA steps, and the pixel-block coordinate helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "activation.hpp"

namespace conv3x3 {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// D(32x32) += A(32x2) * B(2x32), fp32 in, fp32 accumulate.  Lane l supplies
// A[l % 32][l / 32] and B[l / 32][l % 32]; accumulator register v of lane l
// holds D[8 * (v / 4) + 4 * (l / 32) + v % 4][l % 32].
__device__ __forceinline__ f32x16 mfma_32x32x2_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// D(32x32) += A(32x16) * B(16x32), bf16 in, fp32 accumulate.  Lane l
// supplies A[l % 32][8 * (l / 32) + 0..7] and B[8 * (l / 32) + 0..7][l % 32];
// the accumulator layout is the one of the fp32 step above.
__device__ __forceinline__ f32x16 mfma_32x32x16_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Row of the 32x32 accumulator held by register v of this lane.
__device__ __forceinline__ int acc_row(int v, int hi) { return 8 * (v >> 2) + 4 * hi + (v & 3); }

// Decode a workgroup's pixel block origin from its linear block index.
struct BlockOrigin {
  int n0, h0, w0;
};

template <int TW, int TH, int IMGS>
__device__ __forceinline__ BlockOrigin block_origin(int b, int tiles_w, int tiles_h) {
  BlockOrigin o;
  const int tw_i = b % tiles_w;
  b /= tiles_w;
  const int th_i = b % tiles_h;
  const int tn_i = b / tiles_h;
  o.n0 = tn_i * IMGS;
  o.h0 = th_i * TH;
  o.w0 = tw_i * TW;
  return o;
}

}  // namespace conv3x3

namespace conv3x3 {

// Raw buffer view of a tensor for the vector staging paths.  Loads take a
// per-lane byte offset; an offset at or past the view's size reads zeros
// (the hardware range check), which is how out-of-image halo rows and
// columns, and items past a tile's edge, become zero without branches.  Only
// the per-lane offset is range-checked, so callers keep every term of the
// address in it.  Views are limited to tensors of fewer than 2^31 bytes;
// kOutside + any in-range offset stays below 2^32 and past the view.
constexpr uint32_t kOutside = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_view(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t v, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(v, (int)off, 0, 0));
}
__device__ __forceinline__ uint32_t buffer_load4(__amdgpu_buffer_rsrc_t v, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(v, (int)off, 0, 0);
}
// Two consecutive floats at byte offset off (two 32-bit loads, which the
// compiler merges into one 64-bit load).  Returned as scalars: a bit-cast of
// an ext-vector lane (v.y) reads lane x with this compiler.
__device__ __forceinline__ void buffer_load_2f(__amdgpu_buffer_rsrc_t v, uint32_t off, float& a,
                                               float& b) {
  a = __builtin_bit_cast(float, (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(v, (int)off, 0, 0));
  b = __builtin_bit_cast(float,
                         (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(v, (int)(off + 4u), 0, 0));
}
__device__ __forceinline__ uint32_t buffer_load2(__amdgpu_buffer_rsrc_t v, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(v, (int)off, 0, 0);
}
// Eight bytes at byte offset off (one 64-bit load); callers split the words
// with shifts, not ext-vector lanes.
__device__ __forceinline__ uint64_t buffer_load8(__amdgpu_buffer_rsrc_t v, uint32_t off) {
  return __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(v, (int)off, 0, 0));
}

// Four bfloat16 values (words a = e0 | e1 << 16, b = e2 | e3 << 16) spread
// over eight pixels.  Nearest-neighbour 2x along a row: e0 e0 e1 e1 e2 e2 e3 e3.
__device__ __forceinline__ u32x4 bf16x4_repeat2(uint32_t a, uint32_t b) {
  return {(a & 0xffffu) | (a << 16), (a >> 16) | (a & 0xffff0000u), (b & 0xffffu) | (b << 16),
          (b >> 16) | (b & 0xffff0000u)};
}
// Zero insertion along a row: e0 0 e1 0 e2 0 e3 0.
__device__ __forceinline__ u32x4 bf16x4_zero_insert(uint32_t a, uint32_t b) {
  return {a & 0xffffu, a >> 16, b & 0xffffu, b >> 16};
}

// Store one float at byte offset voff + soff of a view; soff is uniform
// across the wave (a scalar register).  The range check applies to voff, so
// a lane with voff = kOutside stores nothing.
__device__ __forceinline__ void buffer_store4(__amdgpu_buffer_rsrc_t v, uint32_t voff,
                                              uint32_t soff, float x) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), v, (int)voff,
                                        (int)soff, 0);
}

// Store the low 16 bits of x at byte offset voff + soff of a view (same
// range check as buffer_store4).
__device__ __forceinline__ void buffer_store2(__amdgpu_buffer_rsrc_t v, uint32_t voff,
                                              uint32_t soff, uint32_t x) {
  __builtin_amdgcn_raw_buffer_store_b16((unsigned short)x, v, (int)voff, (int)soff, 0);
}

// float32 -> bfloat16 bits, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// The bfloat16 passes' fused gradient operand: g = gy * act'(z) for a
// bfloat16 gy and a float32 z, rounded to the nearest bfloat16 value (ties
// to even) as the exact product rounds.  The float32 product p decides
// unless the interval p +- |gy| 2^-17 -- wider than p's error: the slope's
// absolute error stays below 1e-6 for every z (the exponential's error
// scales with s (1 - s), which vanishes where |z| is large), and p's own
// rounding is 2^-24 relative -- holds a bfloat16 rounding boundary, or p
// is one; then the product is formed again in double precision (a few
// elements in a thousand).
__device__ __forceinline__ uint32_t bf16_rne_f64(double g) {
  if (g != g) return 0x7fc0u;
  if (__builtin_fabs(g) < 0x1p-120) return bf16_rne((float)g);  // (no such g in practice)
  uint64_t u = __builtin_bit_cast(uint64_t, g);
  // keep 7 of the 52 fraction bits, round to nearest even on the other 45
  u = (u + 0x00000FFFFFFFFFFFull + ((u >> 45) & 1u)) & ~0x00001FFFFFFFFFFFull;
  return __builtin_bit_cast(uint32_t, (float)__builtin_bit_cast(double, u)) >> 16;
}

// e^x in double precision for that rare path, inline (a library call would
// give the kernels a call frame in scratch memory): x = k ln2 + r with
// |r| <= ln2 / 2 (to within the rounding of k ln2, about 1e-14 absolute,
// far below what the rounding decision needs), e^r by its Taylor series up
// to r^13 / 13! (the remainder is below 2e-16 relative), and 2^k formed in
// the exponent field in two halves so that each stays a normal double.
__device__ __forceinline__ double exp_f64(double x) {
  if (x > 709.0) return __builtin_inf();
  if (x < -745.0) return 0.0;
  const double k = __builtin_rint(x * 1.4426950408889634);  // x / ln2
  const double r = x - k * 0.6931471805599453;              // x - k ln2
  // sum_{n=0}^{13} r^n / n!, Horner form
  double p = 1.0 / 6227020800.0;                  // 1 / 13!
  p = p * r + 1.0 / 479001600.0;                  // 1 / 12!
  p = p * r + 1.0 / 39916800.0;                   // 1 / 11!
  p = p * r + 1.0 / 3628800.0;                    // 1 / 10!
  p = p * r + 1.0 / 362880.0;                     // 1 / 9!
  p = p * r + 1.0 / 40320.0;                      // 1 / 8!
  p = p * r + 1.0 / 5040.0;                       // 1 / 7!
  p = p * r + 1.0 / 720.0;                        // 1 / 6!
  p = p * r + 1.0 / 120.0;                        // 1 / 5!
  p = p * r + 1.0 / 24.0;                         // 1 / 4!
  p = p * r + 1.0 / 6.0;                          // 1 / 3!
  p = p * r + 0.5;                                // 1 / 2!
  p = p * r + 1.0;
  p = p * r + 1.0;
  const int ki = (int)k, k1 = ki / 2, k2 = ki - k1;  // each in [-538, 512]
  const double f1 = __builtin_bit_cast(double, (uint64_t)(k1 + 1023) << 52);
  const double f2 = __builtin_bit_cast(double, (uint64_t)(k2 + 1023) << 52);
  return p * f1 * f2;
}

__device__ __forceinline__ uint32_t act_grad_bf16_f64_inl(float gy, float z, int act) {
  double sl = 1.0;
  if (act == kActSilu) {
    const double zd = z, s = 1.0 / (1.0 + exp_f64(-zd));
    sl = s * (1.0 + zd * (1.0 - s));
  } else if (act == kActLrelu) {
    sl = z > 0.f ? 1.0 : 0.2;
  }
  return bf16_rne_f64((double)gy * sl);
}

// The same as a call (kernels whose register budget cannot hold the double
// precision path inline at every staged element).
__device__ __noinline__ uint32_t act_grad_bf16_f64_call(float gy, float z, int act) {
  return act_grad_bf16_f64_inl(gy, z, act);
}

// INL: the rare double-precision path inline (true) or as a call (false).
template <bool INL>
__device__ __forceinline__ uint32_t act_grad_bf16_f32(float gy, float z, int act) {
  const float p = gy * act_slope(act, z);
  const float e = __builtin_fabsf(gy) * 0x1p-17f;
  const uint32_t r = bf16_rne(p);
  const bool tie = (__builtin_bit_cast(uint32_t, p) & 0xffffu) == 0x8000u;
  if (!tie && bf16_rne(p - e) == r && bf16_rne(p + e) == r) return r;
  return INL ? act_grad_bf16_f64_inl(gy, z, act) : act_grad_bf16_f64_call(gy, z, act);
}

// The bfloat16 input prologue's operand: a = SiLU(u), u = x * scale +
// shift, for a bfloat16 x, rounded to the nearest bfloat16 value as the
// exact a rounds.  The float32 value (u by one fused multiply-add, the fast
// sigmoid) is within |u| 1.2e-6 of the exact one; it decides unless
// a +- |u| 2^-17 holds a rounding boundary (or a is one), and then a is
// formed again in double precision.
__device__ __forceinline__ uint32_t silu_affine_bf16_f64_inl(float x, float s, float t) {
  const double u = (double)x * (double)s + (double)t;
  return bf16_rne_f64(u / (1.0 + exp_f64(-u)));
}

__device__ __noinline__ uint32_t silu_affine_bf16_f64_call(float x, float s, float t) {
  return silu_affine_bf16_f64_inl(x, s, t);
}

template <bool INL>
__device__ __forceinline__ uint32_t silu_affine_bf16_f32(float x, float s, float t) {
  const float u = __builtin_fmaf(x, s, t);
  const float a = u * sigmoid_fast(u);
  const float e = __builtin_fabsf(u) * 0x1p-17f;
  const uint32_t r = bf16_rne(a);
  const bool tie = (__builtin_bit_cast(uint32_t, a) & 0xffffu) == 0x8000u;
  if (!tie && bf16_rne(a - e) == r && bf16_rne(a + e) == r) return r;
  return INL ? silu_affine_bf16_f64_inl(x, s, t) : silu_affine_bf16_f64_call(x, s, t);
}

// xp packs two bfloat16 inputs of one channel (the first in the low half).
template <bool INL>
__device__ __forceinline__ uint32_t silu_affine_bf16x2(uint32_t xp, float s, float t) {
  return silu_affine_bf16_f32<INL>(__builtin_bit_cast(float, xp << 16), s, t) |
         (silu_affine_bf16_f32<INL>(__builtin_bit_cast(float, xp & 0xffff0000u), s, t) << 16);
}

template <bool INL>
__device__ __forceinline__ uint32_t silu_affine_bf16(uint32_t x, float s, float t) {
  return silu_affine_bf16_f32<INL>(__builtin_bit_cast(float, (x & 0xffffu) << 16), s, t);
}

// gp packs two bfloat16 gradients (the first in the low half); the result
// packs the two operands the same way.
template <bool INL>
__device__ __forceinline__ uint32_t act_grad_bf16x2(uint32_t gp, float z0, float z1, int act) {
  return act_grad_bf16_f32<INL>(__builtin_bit_cast(float, gp << 16), z0, act) |
         (act_grad_bf16_f32<INL>(__builtin_bit_cast(float, gp & 0xffff0000u), z1, act) << 16);
}

template <bool INL>
__device__ __forceinline__ uint32_t act_grad_bf16(uint32_t g, float z, int act) {
  return act_grad_bf16_f32<INL>(__builtin_bit_cast(float, (g & 0xffffu) << 16), z, act);
}

}  // namespace conv3x3
