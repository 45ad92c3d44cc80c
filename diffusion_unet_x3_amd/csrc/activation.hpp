// Activation fused into the convolution's forward epilogue and into the
// gradient loader of its backward passes.
//
// The project-guide page on StyleGAN2's custom kernels fuses a bias and an
// activation (a leaky ReLU with a bias term) into one operation to save
// memory traffic; here the activation acts on the biased convolution output
// z held in the accumulators:
//   kActNone   act(z) = z
//   kActSilu   act(z) = z * sigmoid(z)
//   kActLrelu  act(z) = z for z >= 0, 0.2 z below (no gain)
// and the backward passes run on g = gy * act'(z), gy being the gradient at
// the activation's output:
//   SiLU        act'(z) = s (1 + z (1 - s)),  s = 1 / (1 + e^-z)
//   leaky ReLU  act'(z) = 1 for z > 0, 0.2 otherwise
//
// Input prologue (GroupNorm-apply + SiLU fused into the loader of the
// convolution that follows it in a UNet residual block): the convolution's
// input is a = SiLU(u), u = x * scale[n, c] + shift[n, c], zero-padded after
// the activation.  The forward and backward-weight loaders form a from x as
// they stage it; backward-data returns du = (its result) * SiLU'(u), reading
// x, scale and shift in its epilogue.
#pragma once

#include <hip/hip_runtime.h>

namespace conv3x3 {

enum Act { kActNone = 0, kActSilu = 1, kActLrelu = 2 };

// What a launch fuses.  zout: where the forward also writes z (may be null).
// zsrc: z for the backward passes' gradient source (null: g is used as is).
// pscale / pshift ([N][C] float32, null: no prologue): the input prologue's
// scale and shift; px: x for backward-data's SiLU'(u) (same shape as dx;
// for the bfloat16 kernels it points to bfloat16 values).
struct ActArgs {
  int act = kActNone;
  float* zout = nullptr;
  const float* zsrc = nullptr;
  const float* pscale = nullptr;
  const float* pshift = nullptr;
  const float* px = nullptr;
  // the source (forward) or x (backward-weight) is upsampled 2x by nearest
  // neighbour as it is staged; the problem's H, W are the upsampled sizes
  bool up2 = false;
  // stride 2 (H, W even, the input's sizes; the output and g are H/2 x W/2):
  // the forward and backward-weight read x at stride 2 over the output grid;
  // backward-data runs one dense convolution of g per output-pixel parity
  // class
  bool s2 = false;
};

// sigmoid(z) = 1 / (1 + e^-z) with the hardware exponential and reciprocal
// (about 1 ulp each, far inside the float32 bar; an IEEE division would
// cost a dozen instructions per staged element).  e^-z overflows to +inf
// for z < -88 and the reciprocal of +inf is 0, the limit.
__device__ __forceinline__ float sigmoid_fast(float z) {
  return __builtin_amdgcn_rcpf(1.f + __expf(-z));
}

__device__ __forceinline__ float act_value(int act, float z) {
  if (act == kActSilu) return z * sigmoid_fast(z);
  if (act == kActLrelu) return z >= 0.f ? z : 0.2f * z;
  return z;
}

__device__ __forceinline__ float act_slope(int act, float z) {
  if (act == kActSilu) {
    const float s = sigmoid_fast(z);
    return s * (1.f + z * (1.f - s));
  }
  if (act == kActLrelu) return z > 0.f ? 1.f : 0.2f;
  return 1.f;
}

}  // namespace conv3x3
