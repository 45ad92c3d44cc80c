// C ABI of the conv3x3 library: argument validation, planning and launch.
// Declarations and the operation's definition are in include/conv3x3.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/conv3x3.h"
#include "launch.hpp"
#include "planner.hpp"

using namespace conv3x3;

namespace {

constexpr long kMaxElems = 2147483647L;  // every tensor must hold < 2^31 elements

int check_dims(int N, int C, int K, int H, int W) {
  if (N < 1 || C < 1 || K < 1 || H < 1 || W < 1) return CONV3X3_ERR_BAD_SHAPE;
  const long hw = (long)H * W;
  if (hw > kMaxElems) return CONV3X3_ERR_BAD_SHAPE;
  // Products in long (64-bit): each factor is < 2^31 and the running product
  // is checked before the next multiplication.
  if ((long)N * C > kMaxElems || (long)N * C * hw >= kMaxElems + 1L) return CONV3X3_ERR_BAD_SHAPE;
  if ((long)N * K > kMaxElems || (long)N * K * hw >= kMaxElems + 1L) return CONV3X3_ERR_BAD_SHAPE;
  if ((long)K * C > kMaxElems / 9) return CONV3X3_ERR_BAD_SHAPE;
  return CONV3X3_OK;
}

int check_dtype(int dtype) {
  return (dtype == CONV3X3_F32 || dtype == CONV3X3_BF16) ? CONV3X3_OK : CONV3X3_ERR_BAD_DTYPE;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The bf16 vector paths read through 32-bit buffer offsets.
bool buffer_sized(long elems) { return elems * 2 < 2147483648L; }

int launch_status() {
  return hipGetLastError() == hipSuccess ? CONV3X3_OK : CONV3X3_ERR_HIP;
}

int check_act(int act) {
  return (act >= CONV3X3_ACT_NONE && act <= CONV3X3_ACT_LRELU) ? CONV3X3_OK : CONV3X3_ERR_BAD_ACT;
}

int fwd_impl(const void* x, const void* w, const float* bias, float* y, float* z, int N, int C,
             int K, int H, int W, int dtype, int act, conv3x3_stream_t stream) {
  if (!x || !w || !y) return CONV3X3_ERR_NULL_POINTER;
  int rc = check_dims(N, C, K, H, W);
  if (rc) return rc;
  rc = check_dtype(dtype);
  if (rc) return rc;
  rc = check_act(act);
  if (rc) return rc;
  if ((const void*)y == x || (const void*)y == w || (bias && y == bias)) return CONV3X3_ERR_ALIAS;
  if (z && ((const void*)z == x || (const void*)z == w || z == bias || z == y))
    return CONV3X3_ERR_ALIAS;
  Plan pl;
  if (!plan(Problem{kFwd, dtype, N, C, K, H, W}, &pl)) return CONV3X3_ERR_BAD_SHAPE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  ActArgs a;
  a.act = act;
  a.zout = z;
  bool ok;
  if (dtype == CONV3X3_F32) {
    const bool vec = W % 4 == 0 && C % 4 == 0 && aligned16(x) && aligned16(w) &&
                     buffer_sized(2L * N * C * H * W) && buffer_sized(2L * K * C * 9);
    ok = launch_fwd_f32(pl, vec, (const float*)x, (const float*)w, bias, y, N, C, K, H, W, a, s);
  } else {
    const bool vec = W % 8 == 0 && C % 16 == 0 && aligned16(x) && aligned16(w) &&
                     buffer_sized((long)N * C * H * W) && buffer_sized((long)K * C * 9);
    ok = launch_fwd_bf16(pl, vec, (const uint16_t*)x, (const uint16_t*)w, bias, y, N, C, K, H, W,
                         a, s);
  }
  if (!ok) return CONV3X3_ERR_BAD_SHAPE;
  return launch_status();
}

int bwd_data_impl(const void* g, const float* z, const void* w, float* dx, int N, int C, int K,
                  int H, int W, int dtype, int act, conv3x3_stream_t stream) {
  if (!g || !w || !dx) return CONV3X3_ERR_NULL_POINTER;
  int rc = check_dims(N, C, K, H, W);
  if (rc) return rc;
  rc = check_dtype(dtype);
  if (rc) return rc;
  rc = check_act(act);
  if (rc) return rc;
  if (act != CONV3X3_ACT_NONE && !z) return CONV3X3_ERR_NULL_POINTER;
  if (act != CONV3X3_ACT_NONE && dtype != CONV3X3_F32) return CONV3X3_ERR_UNSUPPORTED;
  if ((const void*)dx == g || (const void*)dx == w || (act != CONV3X3_ACT_NONE && dx == z))
    return CONV3X3_ERR_ALIAS;
  Plan pl;
  if (!plan(Problem{kBwdData, dtype, N, C, K, H, W}, &pl)) return CONV3X3_ERR_BAD_SHAPE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  ActArgs a;
  if (act != CONV3X3_ACT_NONE) {
    a.act = act;
    a.zsrc = z;
  }
  bool ok;
  if (dtype == CONV3X3_F32) {
    const bool vec = W % 4 == 0 && C % 4 == 0 && aligned16(g) && aligned16(w) &&
                     (!a.zsrc || aligned16(a.zsrc)) && buffer_sized(2L * N * K * H * W) &&
                     buffer_sized(2L * K * C * 9);
    ok = launch_fwd_f32(pl, vec, (const float*)g, (const float*)w, nullptr, dx, N, K, C, H, W, a,
                        s);
  } else {
    const bool vec = W % 8 == 0 && K % 16 == 0 && C % 8 == 0 && aligned16(g) && aligned16(w) &&
                     buffer_sized((long)N * K * H * W) && buffer_sized((long)K * C * 9);
    ok = launch_fwd_bf16(pl, vec, (const uint16_t*)g, (const uint16_t*)w, nullptr, dx, N, K, C, H,
                         W, a, s);
  }
  if (!ok) return CONV3X3_ERR_BAD_SHAPE;
  return launch_status();
}

int bwd_weight_impl(const void* x, const void* g, const float* z, float* dw, float* db,
                    void* workspace, size_t workspace_bytes, int N, int C, int K, int H, int W,
                    int dtype, int act, conv3x3_stream_t stream) {
  if (!x || !g || !dw) return CONV3X3_ERR_NULL_POINTER;
  int rc = check_dims(N, C, K, H, W);
  if (rc) return rc;
  rc = check_dtype(dtype);
  if (rc) return rc;
  rc = check_act(act);
  if (rc) return rc;
  if (act != CONV3X3_ACT_NONE && !z) return CONV3X3_ERR_NULL_POINTER;
  if (act != CONV3X3_ACT_NONE && dtype != CONV3X3_F32) return CONV3X3_ERR_UNSUPPORTED;
  if ((const void*)dw == x || (const void*)dw == g || (db && ((const void*)db == x ||
                                                              (const void*)db == g || db == dw)))
    return CONV3X3_ERR_ALIAS;
  if (act != CONV3X3_ACT_NONE && (dw == z || (db && db == z))) return CONV3X3_ERR_ALIAS;
  Plan pl;
  if (!plan(Problem{kBwdWeight, dtype, N, C, K, H, W}, &pl)) return CONV3X3_ERR_BAD_SHAPE;
  if (pl.workspace_bytes > 0 && (!workspace || workspace_bytes < pl.workspace_bytes))
    return CONV3X3_ERR_WORKSPACE;
  if (workspace && (workspace == x || workspace == g || workspace == dw ||
                    (db && workspace == db) || (act != CONV3X3_ACT_NONE && workspace == z)))
    return CONV3X3_ERR_ALIAS;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  ActArgs a;
  if (act != CONV3X3_ACT_NONE) {
    a.act = act;
    a.zsrc = z;
  }
  bool ok;
  if (dtype == CONV3X3_F32) {
    const bool vec = W % 4 == 0 && aligned16(x) && aligned16(g) &&
                     (!a.zsrc || aligned16(a.zsrc)) && buffer_sized(2L * N * C * H * W) &&
                     buffer_sized(2L * N * K * H * W);
    ok = launch_wgrad_f32(pl, vec, (const float*)x, (const float*)g, dw, db, (float*)workspace, N,
                          C, K, H, W, a, s);
  } else {
    const bool vec = W % 8 == 0 && aligned16(x) && aligned16(g) &&
                     buffer_sized((long)N * C * H * W) && buffer_sized((long)N * K * H * W);
    ok = launch_wgrad_bf16(pl, vec, (const uint16_t*)x, (const uint16_t*)g, dw, db,
                           (float*)workspace, N, C, K, H, W, a, s);
  }
  if (!ok) return CONV3X3_ERR_BAD_SHAPE;
  return launch_status();
}

}  // namespace

extern "C" {

const char* conv3x3_status_string(int status) {
  switch (status) {
    case CONV3X3_OK: return "success";
    case CONV3X3_ERR_NULL_POINTER: return "a required pointer is NULL";
    case CONV3X3_ERR_BAD_SHAPE: return "invalid shape: every dimension must be >= 1 and every tensor < 2^31 elements";
    case CONV3X3_ERR_BAD_DTYPE: return "unknown dtype (expected CONV3X3_F32 or CONV3X3_BF16)";
    case CONV3X3_ERR_WORKSPACE: return "workspace missing or smaller than conv3x3_bwd_weight_workspace_size()";
    case CONV3X3_ERR_ALIAS: return "an output aliases an input";
    case CONV3X3_ERR_HIP: return "the HIP runtime rejected a kernel launch";
    case CONV3X3_ERR_BAD_PASS: return "unknown pass";
    case CONV3X3_ERR_BAD_ACT: return "unknown activation (expected a conv3x3_act_t value)";
    case CONV3X3_ERR_UNSUPPORTED: return "this dtype's backward pass has no fused activation";
    default: return "unknown status code";
  }
}

int conv3x3_plan(int pass, int N, int C, int K, int H, int W, int dtype, conv3x3_plan_t* out) {
  if (!out) return CONV3X3_ERR_NULL_POINTER;
  if (pass < CONV3X3_PASS_FWD || pass > CONV3X3_PASS_BWD_WEIGHT) return CONV3X3_ERR_BAD_PASS;
  int rc = check_dims(N, C, K, H, W);
  if (rc) return rc;
  rc = check_dtype(dtype);
  if (rc) return rc;
  Plan pl;
  if (!plan(Problem{pass, dtype, N, C, K, H, W}, &pl)) return CONV3X3_ERR_BAD_PASS;
  out->pass = pl.pass;
  out->dtype = pl.dtype;
  out->kernel = pl.wave_co;
  out->tile_m = pl.tile_co;
  out->tile_n = pass == CONV3X3_PASS_BWD_WEIGHT ? pl.tile_ci : pl.imgs * pl.th * pl.tw;
  out->tile_imgs = pl.imgs;
  out->tile_h = pl.th;
  out->tile_w = pl.tw;
  out->chunk = pl.chunk;
  out->threads = pl.threads;
  out->grid_x = pl.grid_x;
  out->grid_y = pl.grid_y;
  out->grid_z = pl.grid_z;
  out->lds_bytes = pl.lds_bytes;
  out->split = pl.split;
  out->workspace_bytes = pl.workspace_bytes;
  return CONV3X3_OK;
}

int conv3x3_fwd(const void* x, const void* w, const float* bias, float* y, int N, int C, int K,
                int H, int W, int dtype, conv3x3_stream_t stream) {
  return fwd_impl(x, w, bias, y, nullptr, N, C, K, H, W, dtype, CONV3X3_ACT_NONE, stream);
}

int conv3x3_bwd_data(const void* g, const void* w, float* dx, int N, int C, int K, int H, int W,
                     int dtype, conv3x3_stream_t stream) {
  return bwd_data_impl(g, nullptr, w, dx, N, C, K, H, W, dtype, CONV3X3_ACT_NONE, stream);
}

int conv3x3_fwd_act(const void* x, const void* w, const float* bias, float* y, float* z, int N,
                    int C, int K, int H, int W, int dtype, int act, conv3x3_stream_t stream) {
  return fwd_impl(x, w, bias, y, z, N, C, K, H, W, dtype, act, stream);
}

int conv3x3_bwd_data_act(const void* gy, const float* z, const void* w, float* dx, int N, int C,
                         int K, int H, int W, int dtype, int act, conv3x3_stream_t stream) {
  return bwd_data_impl(gy, z, w, dx, N, C, K, H, W, dtype, act, stream);
}

size_t conv3x3_bwd_weight_workspace_size(int N, int C, int K, int H, int W, int dtype) {
  if (check_dims(N, C, K, H, W) || check_dtype(dtype)) return (size_t)-1;
  Plan pl;
  if (!plan(Problem{kBwdWeight, dtype, N, C, K, H, W}, &pl)) return (size_t)-1;
  return pl.workspace_bytes;
}

int conv3x3_bwd_weight(const void* x, const void* g, float* dw, float* db, void* workspace,
                       size_t workspace_bytes, int N, int C, int K, int H, int W, int dtype,
                       conv3x3_stream_t stream) {
  return bwd_weight_impl(x, g, nullptr, dw, db, workspace, workspace_bytes, N, C, K, H, W, dtype,
                         CONV3X3_ACT_NONE, stream);
}

int conv3x3_bwd_weight_act(const void* x, const void* gy, const float* z, float* dw, float* db,
                           void* workspace, size_t workspace_bytes, int N, int C, int K, int H,
                           int W, int dtype, int act, conv3x3_stream_t stream) {
  return bwd_weight_impl(x, gy, z, dw, db, workspace, workspace_bytes, N, C, K, H, W, dtype, act,
                         stream);
}

}  // extern "C"
