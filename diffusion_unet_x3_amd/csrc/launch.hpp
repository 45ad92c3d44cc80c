// Host launchers of the conv3x3 kernel families (one per source file).
// Each returns false when the plan names a variant the file does not hold.
#pragma once

#include <hip/hip_runtime.h>

#include "activation.hpp"
#include "planner.hpp"

namespace conv3x3 {

// Resampling geometry of the bfloat16 kernels' scalar staging paths (the
// stride-2 and upsampling entry points): the kernel runs the stride-1
// convolution over the full-resolution grid (its H x W) and
//   kGeoUp   : reads its source at (h / 2, w / 2) of an H/2 x W/2 tensor
//              (nearest 2x upsampling of the input);
//   kGeoZero : reads it there only at even (h, w), zero elsewhere (the
//              zero-inserted gradient of a stride-2 convolution);
//   kGeoSub  : (forward) stores only the even pixels, to (h / 2, w / 2) of
//              an H/2 x W/2 output (the stride-2 convolution's outputs).
enum Geo { kGeoPlain = 0, kGeoUp = 1, kGeoZero = 2, kGeoSub = 3 };

// A channel axis held by two tensors: channels [0, c0) in p0 and [c0, C) in
// p1 (the concatenation [p0 ; p1]).  One tensor is c0 = C (p1 unused).
template <typename T>
struct Split {
  T* p0 = nullptr;
  T* p1 = nullptr;
  int c0 = 0;
};

// Forward (pl.pass == kFwd; src = x, Cin = C, Cout = K) or backward-data
// (pl.pass == kBwdData; src = g, Cin = K, Cout = C; bias ignored), float32.
// a: forward -- a.act and a.zout fused into the epilogue (dst one tensor);
// backward-data -- the source is multiplied by act'(a.zsrc) as it is staged
// (a.zsrc has the source's shape; src one tensor).  pl.split > 1 (plain
// passes only): the reduction is split as for bfloat16 below, partial sums
// in ws.
bool launch_fwd_f32(const Plan& pl, bool vec, Split<const float> src, const float* wt,
                    const float* bias, Split<float> dst, int N, int Cin, int Cout, int H, int W,
                    const ActArgs& a, float* ws, hipStream_t stream);

// Slot-order sum of the S float32 partial outputs (slot floats each) of a
// split forward / backward-data reduction into dst (float32, no activation).
void launch_split_reduce(const float* part, int S, long slot, float* dst, hipStream_t stream);

// dx[p, i, j] = the sum of du[p, 2i .. 2i + 1, 2j .. 2j + 1] in a fixed
// order, for planes p < planes of an H x W dx (du: 2H x 2W planes).
void launch_block_sum2(const float* du, float* dx, long planes, int H, int W,
                       hipStream_t stream);

// Same, bfloat16 inputs (raw 16-bit patterns); outputs float32, or bfloat16
// (round to nearest even) when out_bf16 (dst then points to 16-bit values;
// a.zout stays float32).  a.up2 (forward: x upsampled) and a.s2 (forward:
// strided outputs; backward-data: g zero-inserted) run the plan's
// full-resolution grid with the resampling modes (Geo above) in the vector
// and the scalar staging paths.  pl.split > 1: the reduction is split over
// pl.split workgroups per tile, their partial sums kept in ws (pl.split
// float32 copies of the output) and added by a second kernel.
bool launch_fwd_bf16(const Plan& pl, bool vec, Split<const uint16_t> src, const uint16_t* wt,
                     const float* bias, Split<float> dst, int N, int Cin, int Cout, int H, int W,
                     const ActArgs& a, bool out_bf16, float* ws, hipStream_t stream);

// Backward-weight (+ optional db), float32; ws holds the per-slice partials
// when pl.split > 1.  g is multiplied by act'(a.zsrc) as it is staged.
bool launch_wgrad_f32(const Plan& pl, bool vec, Split<const float> x, const float* g, float* dw,
                      float* db, float* ws, int N, int C, int K, int H, int W, const ActArgs& a,
                      hipStream_t stream);

// Fixed-order sum of the split-K partial slots (both dtypes).
void launch_wgrad_reduce(const float* ws, float* dw, float* db, int split, int C, int K,
                         hipStream_t stream);

// Backward-weight (+ optional db) of a convolution with at most four input
// channels (one tensor; plans with 256 threads): the (channel, tap) pairs
// are the MFMA's columns.  float32 or bfloat16 inputs (raw 16-bit
// patterns); ws holds the per-slice partials when pl.split > 1.
bool launch_wgrad_stem_f32(const Plan& pl, bool vec, const float* x, const float* g, float* dw,
                           float* db, float* ws, int N, int C, int K, int H, int W,
                           hipStream_t stream);
bool launch_wgrad_stem_bf16(const Plan& pl, bool vec, const uint16_t* x, const uint16_t* g,
                            float* dw, float* db, float* ws, int N, int C, int K, int H, int W,
                            hipStream_t stream);

// Forward (+ bias; float32 outputs, no fused activation) of a convolution
// with at most four input channels, bfloat16 inputs (raw 16-bit patterns;
// one tensor; plans with pl.stem): the (channel, tap) pairs are the MFMA's
// reduction, the weights stay in registers, the workgroups loop over
// 128-pixel tiles.
bool launch_fwd_stem_bf16(const Plan& pl, const uint16_t* x, const uint16_t* w,
                          const float* bias, float* y, int N, int C, int K, int H, int W,
                          hipStream_t stream);

// Backward-data with at most three dx channels (plan.stem): P = w^T g per
// band of image rows on MFMA, then the nine shifted taps summed per pixel.
// g through a 32-bit buffer view (N*K*H*W elements below 2 GiB).  bfloat16:
// dx float32, or bfloat16 (nearest even) when outb.
bool launch_bwd_data_stem_f32(const Plan& pl, const float* g, const float* w, float* dx, int N,
                              int C, int K, int H, int W, hipStream_t stream);
bool launch_bwd_data_stem_bf16(const Plan& pl, const uint16_t* g, const uint16_t* w, float* dx,
                               int N, int C, int K, int H, int W, bool outb,
                               hipStream_t stream);

// Same, bfloat16 inputs; a.up2 stages x upsampled, a.s2 stages g
// zero-inserted, over the plan's full-resolution grid (vector or scalar
// staging).
bool launch_wgrad_bf16(const Plan& pl, bool vec, Split<const uint16_t> x, const uint16_t* g,
                       float* dw,
                       float* db, float* ws, int N, int C, int K, int H, int W, const ActArgs& a,
                       hipStream_t stream);

}  // namespace conv3x3
