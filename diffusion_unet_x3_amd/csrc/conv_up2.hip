// The adjoint of nearest-neighbour 2x upsampling: each pixel of the small
// grid receives the sum of the four values of its 2x2 block on the
// upsampled grid (backward-data of a convolution that reads its input
// upsampled).  Fixed order: (row 2i: 2j, 2j+1), then (row 2i+1: 2j, 2j+1).
#include "common.hpp"
#include "launch.hpp"

namespace conv3x3 {

// Two small-grid pixels per thread when pairs (Ws even, big 16-byte
// aligned: 16-byte reads of the two big rows), one otherwise.
__global__ __launch_bounds__(256) void downsum2_kernel(const float* __restrict__ big,
                                                       float* __restrict__ small, long planes,
                                                       int Hs, int Ws, int pairs_ok) {
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  const int Wb = 2 * Ws;
  if (pairs_ok) {
    const long pairs = planes * Hs * (Ws / 2);
    if (t >= pairs) return;
    const long p = t / ((long)Hs * (Ws / 2));
    const int r = (int)(t % ((long)Hs * (Ws / 2)));
    const int i = r / (Ws / 2), j = 2 * (r % (Ws / 2));
    const float* b0 = big + (p * 2 * Hs + 2 * i) * Wb + 2 * j;
    const f32x4 u = *reinterpret_cast<const f32x4*>(b0);
    const f32x4 v = *reinterpret_cast<const f32x4*>(b0 + Wb);
    float* s = small + (p * Hs + i) * Ws + j;
    s[0] = ((u.x + u.y) + v.x) + v.y;
    s[1] = ((u.z + u.w) + v.z) + v.w;
    return;
  }
  const long n = planes * Hs * Ws;
  if (t >= n) return;
  const long p = t / ((long)Hs * Ws);
  const int r = (int)(t % ((long)Hs * Ws));
  const int i = r / Ws, j = r % Ws;
  const float* b0 = big + (p * 2 * Hs + 2 * i) * Wb + 2 * j;
  small[t] = ((b0[0] + b0[1]) + b0[Wb]) + b0[Wb + 1];
}

void launch_downsum2(const float* big, float* small, long planes, int Hs, int Ws,
                     hipStream_t stream) {
  const bool pairs_ok = Ws % 2 == 0 && (reinterpret_cast<uintptr_t>(big) & 15) == 0;
  const long work = pairs_ok ? planes * Hs * (Ws / 2) : planes * Hs * Ws;
  dim3 grid((unsigned)((work + 255) / 256)), block(256);
  hipLaunchKernelGGL(downsum2_kernel, grid, block, 0, stream, big, small, planes, Hs, Ws,
                     pairs_ok ? 1 : 0);
}

}  // namespace conv3x3
