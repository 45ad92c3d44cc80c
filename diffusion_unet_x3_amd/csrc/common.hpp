// Device-side building blocks shared by the conv3x3 kernels: vector types,
// the MFMA steps, and the pixel-block coordinate helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

}  // namespace conv3x3
