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
#pragma once

#include <hip/hip_runtime.h>

namespace conv3x3 {

enum Act { kActNone = 0, kActSilu = 1, kActLrelu = 2 };

// What a launch fuses.  zout: where the forward also writes z (may be null).
// zsrc: z for the backward passes' gradient source (null: g is used as is).
struct ActArgs {
  int act = kActNone;
  float* zout = nullptr;
  const float* zsrc = nullptr;
};

__device__ __forceinline__ float act_value(int act, float z) {
  if (act == kActSilu) return z / (1.f + __expf(-z));
  if (act == kActLrelu) return z >= 0.f ? z : 0.2f * z;
  return z;
}

__device__ __forceinline__ float act_slope(int act, float z) {
  if (act == kActSilu) {
    const float s = 1.f / (1.f + __expf(-z));
    return s * (1.f + z * (1.f - s));
  }
  if (act == kActLrelu) return z > 0.f ? 1.f : 0.2f;
  return 1.f;
}

}  // namespace conv3x3
