// conv3x3_bwd_weight_noalloc: conv3x3_bwd_weight with its split-K partial
// sums in a device array the library holds, for callers that cannot
// allocate device memory.  The kernels are conv3x3_bwd_weight's; only the
// workspace they are given differs.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/conv3x3.h"

namespace {

// One copy per GPU, at its own device address.  In host code this name is
// only a handle for hipGetSymbolAddress: the address passed to kernels is
// the one that lookup returns.
static __device__ __align__(256) unsigned char scratch[CONV3X3_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices];  // device address of `scratch`, per device; null until looked up

// Device address of `scratch` on the current device, looked up (with that
// device current) the first time a call needs it there.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CONV3X3_ERR_HIP;
  std::lock_guard<std::mutex> hold(g_lock);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CONV3X3_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return CONV3X3_OK;
}

}  // namespace

extern "C" int conv3x3_bwd_weight_noalloc(const void* x, const void* g, float* dw, float* db,
                                          int N, int C, int K, int H, int W, int dtype,
                                          conv3x3_stream_t stream) {
  const size_t need = conv3x3_bwd_weight_workspace_size(N, C, K, H, W, dtype);
  if (need == (size_t)-1)  // invalid arguments: the plain entry point names the error
    return conv3x3_bwd_weight(x, g, dw, db, nullptr, 0, N, C, K, H, W, dtype, stream);
  void* ws = nullptr;
  if (need > 0) {
    // Validation first: without a workspace the plain entry point checks
    // every argument and, when all are valid, stops at the missing
    // workspace -- before anything is enqueued.
    const int vrc = conv3x3_bwd_weight(x, g, dw, db, nullptr, 0, N, C, K, H, W, dtype, stream);
    if (vrc != CONV3X3_ERR_WORKSPACE) return vrc;
    if (need > CONV3X3_NOALLOC_SCRATCH_BYTES) return CONV3X3_ERR_NOALLOC;
    // the array used is the current device's, so the stream must run there
    if (stream) {
      int cur = -1, sdev = -1;
      if (hipGetDevice(&cur) != hipSuccess ||
          hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &sdev) != hipSuccess)
        return CONV3X3_ERR_HIP;
      if (sdev != cur) return CONV3X3_ERR_NOALLOC;
    }
    const int rc = scratch_address(&ws);
    if (rc) return rc;
  }
  return conv3x3_bwd_weight(x, g, dw, db, ws, need, N, C, K, H, W, dtype, stream);
}
