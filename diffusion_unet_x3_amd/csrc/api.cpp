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

// The kernels address every tensor through 32-bit buffer offsets, so each
// one (counted as float32: the outputs y, dx, dw are float32 in every mode)
// must stay below 2 GiB: N*C*H*W, N*K*H*W and 9*K*C below 2^29 elements.
// H, W: the call's largest grid.
int check_bytes(int N, int C, int K, int H, int W) {
  constexpr long kLimit = 2147483648L;
  const long hw = (long)H * W;
  if (4L * N * C * hw >= kLimit || 4L * N * K * hw >= kLimit || 36L * K * C >= kLimit)
    return CONV3X3_ERR_UNSUPPORTED;
  return CONV3X3_OK;
}

int check_dtype(int dtype) {
  return (dtype == CONV3X3_F32 || dtype == CONV3X3_BF16 || dtype == CONV3X3_BF16_IO)
             ? CONV3X3_OK
             : CONV3X3_ERR_BAD_DTYPE;
}

// The planner's dtype: the arithmetic (both bf16 modes run the bf16 kernels).
int kdt(int dtype) { return dtype == CONV3X3_F32 ? kF32 : kBF16; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The bf16 vector paths read through 32-bit buffer offsets.
bool buffer_sized(long elems) { return elems * 2 < 2147483648L; }

int launch_status() {
  return hipGetLastError() == hipSuccess ? CONV3X3_OK : CONV3X3_ERR_HIP;
}

int check_act(int act) {
  return (act >= CONV3X3_ACT_NONE && act <= CONV3X3_ACT_LRELU) ? CONV3X3_OK : CONV3X3_ERR_BAD_ACT;
}

// x (or dx) as one tensor or as the concatenation of two: channels
// [0, c0) at p0 and [c0, C) at p1.  A part with no channels may be NULL.
template <typename T>
Split<T> one(T* p, int C) {
  Split<T> s;
  s.p0 = p;
  s.c0 = C;
  return s;
}

// Channel counts of a concatenation: both >= 0, at least one channel, and a
// sum that fits an int (the other limits are check_dims' on the sum).
int check_halves(int C0, int C1) {
  if (C0 < 0 || C1 < 0 || (long)C0 + C1 < 1 || (long)C0 + C1 > kMaxElems)
    return CONV3X3_ERR_BAD_SHAPE;
  return CONV3X3_OK;
}

template <typename T>
bool parts_present(const Split<T>& s, int C) {
  return (s.c0 == 0 || s.p0) && (s.c0 == C || s.p1);
}

template <typename T>
bool parts_aligned(const Split<T>& s) {
  return aligned16(s.p0) && aligned16(s.p1);
}

// p (non-null) is the base pointer of one of the parts
// Whether the byte ranges [a, a + na) and [b, b + nb) intersect.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

template <typename T>
bool is_part(const Split<T>& s, const void* p) {
  return p && (p == (const void*)s.p0 || p == (const void*)s.p1);
}

// The input prologue's per-sample, per-channel scale and shift (both or
// neither).
struct Prologue {
  const float* scale = nullptr;
  const float* shift = nullptr;
  bool on() const { return scale || shift; }
};

int check_prologue(const Prologue& pr) {
  if (!pr.on()) return CONV3X3_OK;
  if (!pr.scale || !pr.shift) return CONV3X3_ERR_NULL_POINTER;
  return CONV3X3_OK;
}

// ws_call: the *_ws entry points -- the caller passes a workspace (possibly
// NULL when conv3x3_workspace_size says 0), so a bf16 plan may split its
// reduction.
int fwd_impl(Split<const void> x, const void* w, const float* bias, float* y, float* z, int N,
             int C, int K, int H, int W, int dtype, int act, conv3x3_stream_t stream,
             Prologue pr = Prologue(), bool ws_call = false, void* ws = nullptr,
             size_t ws_bytes = 0, int geom = 0) {
  // geom 1 (upsampling): H, W are the output's (upsampled) sizes, x is
  // H/2 x W/2; geom 2 (stride 2): H, W are x's, y is H/2 x W/2
  if (!parts_present(x, C) || !w || !y) return CONV3X3_ERR_NULL_POINTER;
  int rc = check_dims(N, C, K, H, W);
  if (rc) return rc;
  rc = check_bytes(N, C, K, H, W);
  if (rc) return rc;
  rc = check_dtype(dtype);
  if (rc) return rc;
  rc = check_act(act);
  if (rc) return rc;
  rc = check_prologue(pr);
  if (rc) return rc;
  if (is_part(x, y) || (const void*)y == w || (bias && y == bias)) return CONV3X3_ERR_ALIAS;
  if (z && (is_part(x, z) || (const void*)z == w || z == bias || z == y)) return CONV3X3_ERR_ALIAS;
  if (pr.on() && (y == pr.scale || y == pr.shift)) return CONV3X3_ERR_ALIAS;
  Plan pl;
  // float32: a stride-2 forward tiles its H/2 x W/2 output, an upsampling
  // one the H/2 x W/2 input (each tile computing the four output parity
  // classes); bfloat16 runs the stride-1 convolution over the full H x W
  // grid (the upsampled input read at half coordinates; the stride-2
  // outputs kept at the even pixels)
  const bool fgeo = geom && dtype == CONV3X3_F32;
  Problem pb{kFwd, kdt(dtype), N, C, K, fgeo ? H / 2 : H, fgeo ? W / 2 : W, x.c0};
  pb.stride2 = fgeo && geom == 2;
  pb.quad = fgeo && geom == 1;
  pb.allow_split = ws_call && aligned16(y) && act == CONV3X3_ACT_NONE && !z && !pr.on() && !geom;
  // (bf16 prologue: four-wave tiles, whose staging threads hold scale and
  // shift beside the x rows)
  pb.four_waves = dtype != CONV3X3_F32 && pr.on();
  // at most four input channels, bfloat16 inputs, float32 outputs, no
  // fusion: the packed-pair forward
  pb.stem = C <= 4 && x.c0 == C && !geom && !pr.on() && dtype == CONV3X3_BF16 &&
            act == CONV3X3_ACT_NONE && !z;
  if (!plan(pb, &pl)) return CONV3X3_ERR_BAD_SHAPE;
  if (pl.workspace_bytes > 0 && (!ws || ws_bytes < pl.workspace_bytes))
    return CONV3X3_ERR_WORKSPACE;
  if (pl.workspace_bytes > 0 &&
      (is_part(x, ws) || ws == w || ws == (const void*)bias || ws == (void*)y))
    return CONV3X3_ERR_ALIAS;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  ActArgs a;
  a.act = act;
  a.zout = z;
  a.pscale = pr.scale;
  a.pshift = pr.shift;
  a.up2 = geom == 1;
  a.s2 = geom == 2;
  const long hw = (long)H * W;
  bool ok;
  if (pl.stem) {
    ok = launch_fwd_stem_bf16(pl, (const uint16_t*)x.p0, (const uint16_t*)w, bias, y, N, C, K,
                              H, W, s);
  } else if (dtype == CONV3X3_F32) {
    // (3 input channels in one tensor: the packed-tap forward, vector x
    // loads and scalar weight loads)
    const bool pack3 = C == 3 && x.c0 == C && !pr.on();
    // (upsampling: the staged rows are the small input's, W/2 floats)
    const bool vec = W % (geom == 1 ? 8 : 4) == 0 && ((C % 4 == 0 && x.c0 % 4 == 0) || pack3) &&
                     parts_aligned(x) && aligned16(w) && buffer_sized(2L * N * C * hw) &&
                     buffer_sized(2L * K * C * 9);
    Split<const float> xs{(const float*)x.p0, (const float*)x.p1, x.c0};
    ok = launch_fwd_f32(pl, vec, xs, (const float*)w, bias, one(y, K), N, C, K, H, W, a,
                        (float*)ws, s);
  } else {
    const bool vec = W % 8 == 0 && C % 16 == 0 && x.c0 % 16 == 0 && parts_aligned(x) &&
                     aligned16(w) && (!pr.on() || (aligned16(pr.scale) && aligned16(pr.shift))) &&
                     buffer_sized((long)N * C * hw) && buffer_sized((long)K * C * 9);
    Split<const uint16_t> xs{(const uint16_t*)x.p0, (const uint16_t*)x.p1, x.c0};
    ok = launch_fwd_bf16(pl, vec, xs, (const uint16_t*)w, bias, one(y, K), N, C, K, H, W, a,
                         dtype == CONV3X3_BF16_IO, (float*)ws, s);
  }
  if (!ok) return CONV3X3_ERR_BAD_SHAPE;
  return launch_status();
}

int bwd_data_impl(const void* g, const float* z, const void* w, Split<float> dx, int N, int C,
                  int K, int H, int W, int dtype, int act, conv3x3_stream_t stream,
                  Prologue pr = Prologue(), const void* px = nullptr, bool ws_call = false,
                  void* ws = nullptr, size_t ws_bytes = 0, int geom = 0) {
  // geom 1 (upsampling): H, W are g's, dx is H/2 x W/2; geom 2 (stride 2):
  // H, W are dx's, g is H/2 x W/2
  const bool s2 = geom == 2;
  if (!g || !w || !parts_present(dx, C)) return CONV3X3_ERR_NULL_POINTER;
  if (pr.on() && !px) return CONV3X3_ERR_NULL_POINTER;
  int rc = check_dims(N, C, K, H, W);
  if (rc) return rc;
  rc = check_bytes(N, C, K, H, W);
  if (rc) return rc;
  rc = check_dtype(dtype);
  if (rc) return rc;
  rc = check_act(act);
  if (rc) return rc;
  if (act != CONV3X3_ACT_NONE && !z) return CONV3X3_ERR_NULL_POINTER;
  rc = check_prologue(pr);
  if (rc) return rc;
  if (is_part(dx, g) || is_part(dx, w) || (act != CONV3X3_ACT_NONE && is_part(dx, z)) ||
      (dx.c0 > 0 && dx.c0 < C && dx.p0 == dx.p1))
    return CONV3X3_ERR_ALIAS;
  if (pr.on() && (is_part(dx, px) || is_part(dx, pr.scale) || is_part(dx, pr.shift)))
    return CONV3X3_ERR_ALIAS;
  // du's epilogue reads x through a 32-bit buffer view, like the stores
  if (pr.on() && 4L * N * C * H * W >= 2147483648L) return CONV3X3_ERR_UNSUPPORTED;
  Plan pl;
  // float32 stride 2: the plan tiles g's H/2 x W/2 grid, each tile
  // computing the four output-pixel parity classes of its pixels;
  // upsampling: it tiles dx's H/2 x W/2 grid and stages g at stride 2.
  // bfloat16 stride 2: the stride-1 backward-data over dx's full grid, g
  // read zero-inserted (upsampling is composed by its entry point).
  if (geom == 1 && dtype != CONV3X3_F32) return CONV3X3_ERR_UNSUPPORTED;
  const bool fgeo = geom && dtype == CONV3X3_F32;
  Problem pb{kBwdData, kdt(dtype), N, C, K, fgeo ? H / 2 : H, fgeo ? W / 2 : W, dx.c0};
  pb.quad = fgeo && s2;
  pb.stride2 = fgeo && geom == 1;
  pb.allow_split = ws_call && aligned16(dx.p0) && act == CONV3X3_ACT_NONE && !pr.on() && !geom;
  pb.four_waves = dtype != CONV3X3_F32 && (act != CONV3X3_ACT_NONE || pr.on());
  // (at most three dx channels in one tensor, no fusion: the (channel,
  // tap)-row kernel; g through a 32-bit buffer view)
  pb.stem = dx.c0 == C && geom == 0 && act == CONV3X3_ACT_NONE && !pr.on() &&
            stem_bwd_data_fits(C, K, W) &&
            (long)N * K * H * W * (dtype == CONV3X3_F32 ? 4 : 2) < 2147483648L;
  if (!plan(pb, &pl)) return CONV3X3_ERR_BAD_SHAPE;
  if (pl.workspace_bytes > 0 && (!ws || ws_bytes < pl.workspace_bytes))
    return CONV3X3_ERR_WORKSPACE;
  if (pl.workspace_bytes > 0 && (ws == g || ws == w || is_part(dx, ws)))
    return CONV3X3_ERR_ALIAS;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (pl.stem) {
    const bool ok =
        dtype == CONV3X3_F32
            ? launch_bwd_data_stem_f32(pl, (const float*)g, (const float*)w, dx.p0, N, C, K, H, W,
                                       s)
            : launch_bwd_data_stem_bf16(pl, (const uint16_t*)g, (const uint16_t*)w, dx.p0, N, C,
                                        K, H, W, dtype == CONV3X3_BF16_IO, s);
    if (!ok) return CONV3X3_ERR_BAD_SHAPE;
    return launch_status();
  }
  ActArgs a;
  if (act != CONV3X3_ACT_NONE) {
    a.act = act;
    a.zsrc = z;
  }
  a.pscale = pr.scale;
  a.pshift = pr.shift;
  a.px = (const float*)px;
  a.s2 = s2;
  a.up2 = geom == 1;
  const long hw = (long)H * W;
  bool ok;
  if (dtype == CONV3X3_F32) {
    // (stride 2: g's rows, W/2 floats, hold whole float4 items)
    const bool vec = W % (s2 ? 8 : 4) == 0 && C % 4 == 0 && dx.c0 % 4 == 0 && aligned16(g) &&
                     aligned16(w) && (!a.zsrc || aligned16(a.zsrc)) &&
                     buffer_sized(2L * N * K * hw) && buffer_sized(2L * K * C * 9);
    ok = launch_fwd_f32(pl, vec, one((const float*)g, K), (const float*)w, nullptr, dx, N, K, C,
                        H, W, a, (float*)ws, s);
  } else {
    const bool vec = W % 8 == 0 && K % 16 == 0 && C % 8 == 0 && dx.c0 % 8 == 0 &&
                     aligned16(g) && aligned16(w) && (!a.zsrc || aligned16(a.zsrc)) &&
                     buffer_sized((long)N * K * hw) && buffer_sized((long)K * C * 9);
    ok = launch_fwd_bf16(pl, vec, one((const uint16_t*)g, K), (const uint16_t*)w, nullptr, dx, N,
                         K, C, H, W, a, dtype == CONV3X3_BF16_IO, (float*)ws, s);
  }
  if (!ok) return CONV3X3_ERR_BAD_SHAPE;
  return launch_status();
}

int bwd_weight_impl(Split<const void> x, const void* g, const float* z, float* dw, float* db,
                    void* workspace, size_t workspace_bytes, int N, int C, int K, int H, int W,
                    int dtype, int act, conv3x3_stream_t stream, Prologue pr = Prologue(),
                    int geom = 0) {
  // geom 1: x is upsampled (H, W are g's, x is H/2 x W/2); geom 2: stride 2
  // (H, W are x's, g is H/2 x W/2)
  if (!parts_present(x, C) || !g || !dw) return CONV3X3_ERR_NULL_POINTER;
  int rc = check_dims(N, C, K, H, W);
  if (rc) return rc;
  rc = check_bytes(N, C, K, H, W);
  if (rc) return rc;
  rc = check_dtype(dtype);
  if (rc) return rc;
  rc = check_act(act);
  if (rc) return rc;
  if (act != CONV3X3_ACT_NONE && !z) return CONV3X3_ERR_NULL_POINTER;
  if (is_part(x, dw) || (const void*)dw == g ||
      (db && (is_part(x, db) || (const void*)db == g || db == dw)))
    return CONV3X3_ERR_ALIAS;
  if (act != CONV3X3_ACT_NONE && (dw == z || (db && db == z))) return CONV3X3_ERR_ALIAS;
  rc = check_prologue(pr);
  if (rc) return rc;
  if (pr.on() && (dw == pr.scale || dw == pr.shift ||
                  (db && (db == pr.scale || db == pr.shift))))
    return CONV3X3_ERR_ALIAS;
  Plan pl;
  // float32 stride 2: the pixel chunks tile g's H/2 x W/2 grid; bfloat16
  // stride 2 runs the full H x W grid with g read zero-inserted
  const bool fs2 = geom == 2 && dtype == CONV3X3_F32;
  Problem pb{kBwdWeight, kdt(dtype), N, C, K, fs2 ? H / 2 : H, fs2 ? W / 2 : W, x.c0};
  pb.stride2 = fs2;
  // (at most four input channels, no fusion: the packed-pair kernel)
  pb.stem = C <= 4 && x.c0 == C && geom == 0 && act == CONV3X3_ACT_NONE && !pr.on();
  if (!plan(pb, &pl)) return CONV3X3_ERR_BAD_SHAPE;
  if (pl.workspace_bytes > 0 && (!workspace || workspace_bytes < pl.workspace_bytes))
    return CONV3X3_ERR_WORKSPACE;
  if (workspace && (is_part(x, workspace) || workspace == g || workspace == dw ||
                    (db && workspace == db) || (act != CONV3X3_ACT_NONE && workspace == z) ||
                    (pr.on() && (workspace == pr.scale || workspace == pr.shift))))
    return CONV3X3_ERR_ALIAS;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  ActArgs a;
  if (act != CONV3X3_ACT_NONE) {
    a.act = act;
    a.zsrc = z;
  }
  a.pscale = pr.scale;
  a.pshift = pr.shift;
  a.up2 = geom == 1;
  a.s2 = geom == 2;
  const long hw = (long)H * W;
  bool ok;
  if (pl.stem) {
    // packed (channel, tap) pairs; 128-bit g loads need whole 16-byte
    // pixel runs
    const bool f32 = dtype == CONV3X3_F32;
    const bool vs = W % (f32 ? 4 : 8) == 0 && aligned16(g);
    ok = f32 ? launch_wgrad_stem_f32(pl, vs, (const float*)x.p0, (const float*)g, dw, db,
                                     (float*)workspace, N, C, K, H, W, s)
             : launch_wgrad_stem_bf16(pl, vs, (const uint16_t*)x.p0, (const uint16_t*)g, dw, db,
                                      (float*)workspace, N, C, K, H, W, s);
  } else if (dtype == CONV3X3_F32) {
    // (stride 2: g's rows, W/2 floats, must hold whole float4 items too)
    const bool vec = W % (geom == 2 ? 8 : 4) == 0 && parts_aligned(x) && aligned16(g) &&
                     (!a.zsrc || aligned16(a.zsrc)) && buffer_sized(2L * N * C * hw) &&
                     buffer_sized(2L * N * K * hw);
    Split<const float> xs{(const float*)x.p0, (const float*)x.p1, x.c0};
    ok = launch_wgrad_f32(pl, vec, xs, (const float*)g, dw, db, (float*)workspace, N, C, K, H, W,
                          a, s);
  } else {
    const bool vec = W % 8 == 0 && parts_aligned(x) && aligned16(g) &&
                     (!a.zsrc || aligned16(a.zsrc)) && buffer_sized((long)N * C * hw) &&
                     buffer_sized((long)N * K * hw);
    Split<const uint16_t> xs{(const uint16_t*)x.p0, (const uint16_t*)x.p1, x.c0};
    ok = launch_wgrad_bf16(pl, vec, xs, (const uint16_t*)g, dw, db, (float*)workspace, N, C, K, H,
                           W, a, s);
  }
  if (!ok) return CONV3X3_ERR_BAD_SHAPE;
  return launch_status();
}

int fill_plan(const Plan& pl, int pass, conv3x3_plan_t* out) {
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

int plan_impl(int pass, int N, int C, int K, int H, int W, int dtype, int C0,
              conv3x3_plan_t* out) {
  if (!out) return CONV3X3_ERR_NULL_POINTER;
  if (pass < CONV3X3_PASS_FWD || pass > CONV3X3_PASS_BWD_WEIGHT) return CONV3X3_ERR_BAD_PASS;
  int rc = check_dims(N, C, K, H, W);
  if (rc) return rc;
  rc = check_dtype(dtype);
  if (rc) return rc;
  Plan pl;
  Problem pb{pass, kdt(dtype), N, C, K, H, W, C0};
  // the plan of the plain call (a fused pass with a few-channel input runs
  // the general kernels; a backward-weight's workspace size is the same)
  pb.stem = ((pass == CONV3X3_PASS_BWD_WEIGHT ||
              (pass == CONV3X3_PASS_FWD && dtype == CONV3X3_BF16)) &&
             C <= 4 && (C0 < 0 || C0 == C)) ||
            (pass == CONV3X3_PASS_BWD_DATA && (C0 < 0 || C0 == C) &&
             stem_bwd_data_fits(C, K, W) &&
             (long)N * K * H * W * (dtype == CONV3X3_F32 ? 4 : 2) < 2147483648L);
  if (!plan(pb, &pl)) return CONV3X3_ERR_BAD_PASS;
  rc = fill_plan(pl, pass, out);
  out->dtype = dtype;
  return rc;
}

}  // namespace

extern "C" {

const char* conv3x3_status_string(int status) {
  switch (status) {
    case CONV3X3_OK: return "success";
    case CONV3X3_ERR_NULL_POINTER: return "a required pointer is NULL";
    case CONV3X3_ERR_BAD_SHAPE: return "invalid shape: every dimension must be >= 1 and every tensor < 2^31 elements";
    case CONV3X3_ERR_BAD_DTYPE: return "unknown dtype (expected a conv3x3_dtype_t value)";
    case CONV3X3_ERR_WORKSPACE: return "workspace missing or smaller than conv3x3_bwd_weight_workspace_size()";
    case CONV3X3_ERR_ALIAS: return "an output aliases an input";
    case CONV3X3_ERR_HIP: return "the HIP runtime rejected a kernel launch";
    case CONV3X3_ERR_BAD_PASS: return "unknown pass";
    case CONV3X3_ERR_BAD_ACT: return "unknown activation (expected a conv3x3_act_t value)";
    case CONV3X3_ERR_UNSUPPORTED: return "not provided for this dtype or size (fusions by dtype; every tensor must be below 2 GiB as float32)";
    case CONV3X3_ERR_NOALLOC: return "conv3x3_bwd_weight_noalloc: the problem needs more scratch than the library's array holds, or the stream is not on the current device";
    default: return "unknown status code";
  }
}

int conv3x3_plan(int pass, int N, int C, int K, int H, int W, int dtype, conv3x3_plan_t* out) {
  return plan_impl(pass, N, C, K, H, W, dtype, -1, out);
}

int conv3x3_plan_cat(int pass, int N, int C0, int C1, int K, int H, int W, int dtype,
                     conv3x3_plan_t* out) {
  const int rc = check_halves(C0, C1);
  if (rc) return rc;
  return plan_impl(pass, N, C0 + C1, K, H, W, dtype, C0, out);
}

int conv3x3_fwd(const void* x, const void* w, const float* bias, float* y, int N, int C, int K,
                int H, int W, int dtype, conv3x3_stream_t stream) {
  return fwd_impl(one(x, C), w, bias, y, nullptr, N, C, K, H, W, dtype, CONV3X3_ACT_NONE, stream);
}

int conv3x3_bwd_data(const void* g, const void* w, float* dx, int N, int C, int K, int H, int W,
                     int dtype, conv3x3_stream_t stream) {
  return bwd_data_impl(g, nullptr, w, one(dx, C), N, C, K, H, W, dtype, CONV3X3_ACT_NONE,
                       stream);
}

int conv3x3_fwd_act(const void* x, const void* w, const float* bias, float* y, float* z, int N,
                    int C, int K, int H, int W, int dtype, int act, conv3x3_stream_t stream) {
  return fwd_impl(one(x, C), w, bias, y, z, N, C, K, H, W, dtype, act, stream);
}

int conv3x3_bwd_data_act(const void* gy, const float* z, const void* w, float* dx, int N, int C,
                         int K, int H, int W, int dtype, int act, conv3x3_stream_t stream) {
  return bwd_data_impl(gy, z, w, one(dx, C), N, C, K, H, W, dtype, act, stream);
}

int conv3x3_fwd_cat(const void* x0, const void* x1, int C0, int C1, const void* w,
                    const float* bias, float* y, int N, int K, int H, int W, int dtype,
                    conv3x3_stream_t stream) {
  const int rc = check_halves(C0, C1);
  if (rc) return rc;
  return fwd_impl(Split<const void>{x0, x1, C0}, w, bias, y, nullptr, N, C0 + C1, K, H, W, dtype,
                  CONV3X3_ACT_NONE, stream);
}

int conv3x3_bwd_data_cat(const void* g, const void* w, float* dx0, float* dx1, int C0, int C1,
                         int N, int K, int H, int W, int dtype, conv3x3_stream_t stream) {
  const int rc = check_halves(C0, C1);
  if (rc) return rc;
  return bwd_data_impl(g, nullptr, w, Split<float>{dx0, dx1, C0}, N, C0 + C1, K, H, W, dtype,
                       CONV3X3_ACT_NONE, stream);
}

size_t conv3x3_bwd_weight_cat_workspace_size(int N, int C0, int C1, int K, int H, int W,
                                             int dtype) {
  if (check_halves(C0, C1) || check_dims(N, C0 + C1, K, H, W) || check_dtype(dtype))
    return (size_t)-1;
  Plan pl;
  if (!plan(Problem{kBwdWeight, kdt(dtype), N, C0 + C1, K, H, W, C0}, &pl)) return (size_t)-1;
  return pl.workspace_bytes;
}

int conv3x3_bwd_weight_cat(const void* x0, const void* x1, int C0, int C1, const void* g,
                           float* dw, float* db, void* workspace, size_t workspace_bytes, int N,
                           int K, int H, int W, int dtype, conv3x3_stream_t stream) {
  const int rc = check_halves(C0, C1);
  if (rc) return rc;
  return bwd_weight_impl(Split<const void>{x0, x1, C0}, g, nullptr, dw, db, workspace,
                         workspace_bytes, N, C0 + C1, K, H, W, dtype, CONV3X3_ACT_NONE, stream);
}

size_t conv3x3_bwd_weight_workspace_size(int N, int C, int K, int H, int W, int dtype) {
  if (check_dims(N, C, K, H, W) || check_dtype(dtype)) return (size_t)-1;
  Plan pl;
  if (!plan(Problem{kBwdWeight, kdt(dtype), N, C, K, H, W}, &pl)) return (size_t)-1;
  return pl.workspace_bytes;
}

int conv3x3_bwd_weight(const void* x, const void* g, float* dw, float* db, void* workspace,
                       size_t workspace_bytes, int N, int C, int K, int H, int W, int dtype,
                       conv3x3_stream_t stream) {
  return bwd_weight_impl(one(x, C), g, nullptr, dw, db, workspace, workspace_bytes, N, C, K, H,
                         W, dtype, CONV3X3_ACT_NONE, stream);
}

int conv3x3_bwd_weight_act(const void* x, const void* gy, const float* z, float* dw, float* db,
                           void* workspace, size_t workspace_bytes, int N, int C, int K, int H,
                           int W, int dtype, int act, conv3x3_stream_t stream) {
  return bwd_weight_impl(one(x, C), gy, z, dw, db, workspace, workspace_bytes, N, C, K, H, W,
                         dtype, act, stream);
}

int conv3x3_fwd_gnsilu(const void* x, const float* scale, const float* shift, const void* w,
                       const float* bias, float* y, int N, int C, int K, int H, int W, int dtype,
                       conv3x3_stream_t stream) {
  if (!scale || !shift) return CONV3X3_ERR_NULL_POINTER;
  return fwd_impl(one(x, C), w, bias, y, nullptr, N, C, K, H, W, dtype, CONV3X3_ACT_NONE, stream,
                  Prologue{scale, shift});
}

int conv3x3_bwd_data_gnsilu(const void* g, const void* w, const void* x, const float* scale,
                            const float* shift, float* du, int N, int C, int K, int H, int W,
                            int dtype, conv3x3_stream_t stream) {
  if (!scale || !shift) return CONV3X3_ERR_NULL_POINTER;
  return bwd_data_impl(g, nullptr, w, one(du, C), N, C, K, H, W, dtype, CONV3X3_ACT_NONE, stream,
                       Prologue{scale, shift}, x);
}

int conv3x3_bwd_weight_gnsilu(const void* x, const float* scale, const float* shift,
                              const void* g, float* dw, float* db, void* workspace,
                              size_t workspace_bytes, int N, int C, int K, int H, int W,
                              int dtype, conv3x3_stream_t stream) {
  if (!scale || !shift) return CONV3X3_ERR_NULL_POINTER;
  return bwd_weight_impl(one(x, C), g, nullptr, dw, db, workspace, workspace_bytes, N, C, K, H,
                         W, dtype, CONV3X3_ACT_NONE, stream, Prologue{scale, shift});
}

size_t conv3x3_workspace_size(int pass, int N, int C, int K, int H, int W, int dtype) {
  if (pass < CONV3X3_PASS_FWD || pass > CONV3X3_PASS_BWD_WEIGHT) return (size_t)-1;
  if (check_dims(N, C, K, H, W) || check_dtype(dtype)) return (size_t)-1;
  Problem pb{pass, kdt(dtype), N, C, K, H, W};
  pb.allow_split = true;
  Plan pl;
  if (!plan(pb, &pl)) return (size_t)-1;
  return pl.workspace_bytes;
}

int conv3x3_fwd_ws(const void* x, const void* w, const float* bias, float* y, void* workspace,
                   size_t workspace_bytes, int N, int C, int K, int H, int W, int dtype,
                   conv3x3_stream_t stream) {
  return fwd_impl(one(x, C), w, bias, y, nullptr, N, C, K, H, W, dtype, CONV3X3_ACT_NONE, stream,
                  Prologue(), true, workspace, workspace_bytes);
}

int conv3x3_bwd_data_ws(const void* g, const void* w, float* dx, void* workspace,
                        size_t workspace_bytes, int N, int C, int K, int H, int W, int dtype,
                        conv3x3_stream_t stream) {
  return bwd_data_impl(g, nullptr, w, one(dx, C), N, C, K, H, W, dtype, CONV3X3_ACT_NONE, stream,
                       Prologue(), nullptr, true, workspace, workspace_bytes);
}

// ---- nearest 2x upsampling before the convolution (H, W: x's sizes) ----

namespace {

// The upsampled grid must satisfy the plain limits; float32, or bfloat16
// inputs with float32 outputs.
int check_up2(int N, int C, int K, int H, int W, int dtype) {
  if (H < 1 || W < 1 || H > (1 << 29) || W > (1 << 29)) return CONV3X3_ERR_BAD_SHAPE;
  int rc = check_dims(N, C, K, 2 * H, 2 * W);
  if (rc) return rc;
  rc = check_dtype(dtype);
  if (rc) return rc;
  return dtype == CONV3X3_F32 || dtype == CONV3X3_BF16 ? CONV3X3_OK : CONV3X3_ERR_UNSUPPORTED;
}

}  // namespace

size_t conv3x3_up2_workspace_size(int pass, int N, int C, int K, int H, int W, int dtype) {
  if (pass < CONV3X3_PASS_FWD || pass > CONV3X3_PASS_BWD_WEIGHT) return (size_t)-1;
  if (check_up2(N, C, K, H, W, dtype)) return (size_t)-1;
  if (pass == CONV3X3_PASS_FWD) return 0;
  // bfloat16 backward-data: the float32 gradient of the upsampled grid,
  // summed over 2 x 2 blocks afterwards
  if (pass == CONV3X3_PASS_BWD_DATA)
    return dtype == CONV3X3_F32 ? 0 : (size_t)N * C * 4 * (size_t)H * W * sizeof(float);
  Plan pl;
  if (!plan(Problem{kBwdWeight, kdt(dtype), N, C, K, 2 * H, 2 * W}, &pl)) return (size_t)-1;
  return pl.workspace_bytes;
}

int conv3x3_fwd_up2(const void* x, const void* w, const float* bias, float* y, int N, int C,
                    int K, int H, int W, int dtype, conv3x3_stream_t stream) {
  if (!x || !w || !y) return CONV3X3_ERR_NULL_POINTER;
  const int rc = check_up2(N, C, K, H, W, dtype);
  if (rc) return rc;
  return fwd_impl(one(x, C), w, bias, y, nullptr, N, C, K, 2 * H, 2 * W, dtype, CONV3X3_ACT_NONE,
                  stream, Prologue(), false, nullptr, 0, 1);
}

int conv3x3_bwd_data_up2(const void* g, const void* w, float* dx, void* workspace,
                         size_t workspace_bytes, int N, int C, int K, int H, int W, int dtype,
                         conv3x3_stream_t stream) {
  if (!g || !w || !dx) return CONV3X3_ERR_NULL_POINTER;
  int rc = check_up2(N, C, K, H, W, dtype);
  if (rc) return rc;
  if (dtype != CONV3X3_F32) {
    // bfloat16: the stride-1 backward-data over the upsampled grid into the
    // workspace (float32), then the sum of each 2 x 2 block into dx
    const size_t need = (size_t)N * C * 4 * (size_t)H * W * sizeof(float);
    if (!workspace || workspace_bytes < need) return CONV3X3_ERR_WORKSPACE;
    if (overlaps(workspace, need, g, (size_t)N * K * 4 * (size_t)H * W * 2) ||
        overlaps(workspace, need, w, (size_t)K * C * 9 * 2) ||
        overlaps(workspace, need, dx, (size_t)N * C * (size_t)H * W * sizeof(float)))
      return CONV3X3_ERR_ALIAS;
    rc = bwd_data_impl(g, nullptr, w, one((float*)workspace, C), N, C, K, 2 * H, 2 * W, dtype,
                       CONV3X3_ACT_NONE, stream);
    if (rc) return rc;
    launch_block_sum2((const float*)workspace, dx, (long)N * C, H, W,
                      reinterpret_cast<hipStream_t>(stream));
    return launch_status();
  }
  (void)workspace;  // float32: none needed (kept for the calling convention)
  (void)workspace_bytes;
  // one pass over dx's grid: each pixel gathers g's 4 x 4 window at stride 2
  return bwd_data_impl(g, nullptr, w, one(dx, C), N, C, K, 2 * H, 2 * W, dtype, CONV3X3_ACT_NONE,
                       stream, Prologue(), nullptr, false, nullptr, 0, 1);
}

int conv3x3_bwd_weight_up2(const void* x, const void* g, float* dw, float* db, void* workspace,
                           size_t workspace_bytes, int N, int C, int K, int H, int W, int dtype,
                           conv3x3_stream_t stream) {
  if (!x || !g || !dw) return CONV3X3_ERR_NULL_POINTER;
  const int rc = check_up2(N, C, K, H, W, dtype);
  if (rc) return rc;
  return bwd_weight_impl(one(x, C), g, nullptr, dw, db, workspace, workspace_bytes, N, C, K,
                         2 * H, 2 * W, dtype, CONV3X3_ACT_NONE, stream, Prologue(), 1);
}

// ---- stride-2 convolution (H, W: x's sizes, both even) ----

namespace {

int check_s2(int N, int C, int K, int H, int W, int dtype) {
  int rc = check_dims(N, C, K, H, W);
  if (rc) return rc;
  if (H % 2 || W % 2) return CONV3X3_ERR_BAD_SHAPE;
  rc = check_dtype(dtype);
  if (rc) return rc;
  return dtype == CONV3X3_F32 || dtype == CONV3X3_BF16 ? CONV3X3_OK : CONV3X3_ERR_UNSUPPORTED;
}

}  // namespace

int conv3x3_fwd_s2(const void* x, const void* w, const float* bias, float* y, int N, int C,
                   int K, int H, int W, int dtype, conv3x3_stream_t stream) {
  if (!x || !w || !y) return CONV3X3_ERR_NULL_POINTER;
  const int rc = check_s2(N, C, K, H, W, dtype);
  if (rc) return rc;
  return fwd_impl(one(x, C), w, bias, y, nullptr, N, C, K, H, W, dtype, CONV3X3_ACT_NONE, stream,
                  Prologue(), false, nullptr, 0, 2);
}

int conv3x3_bwd_data_s2(const void* g, const void* w, float* dx, int N, int C, int K, int H,
                        int W, int dtype, conv3x3_stream_t stream) {
  if (!g || !w || !dx) return CONV3X3_ERR_NULL_POINTER;
  const int rc = check_s2(N, C, K, H, W, dtype);
  if (rc) return rc;
  return bwd_data_impl(g, nullptr, w, one(dx, C), N, C, K, H, W, dtype, CONV3X3_ACT_NONE, stream,
                       Prologue(), nullptr, false, nullptr, 0, 2);
}

int conv3x3_bwd_weight_s2(const void* x, const void* g, float* dw, float* db, void* workspace,
                          size_t workspace_bytes, int N, int C, int K, int H, int W, int dtype,
                          conv3x3_stream_t stream) {
  if (!x || !g || !dw) return CONV3X3_ERR_NULL_POINTER;
  const int rc = check_s2(N, C, K, H, W, dtype);
  if (rc) return rc;
  return bwd_weight_impl(one(x, C), g, nullptr, dw, db, workspace, workspace_bytes, N, C, K, H, W,
                         dtype, CONV3X3_ACT_NONE, stream, Prologue(), 2);
}

}  // extern "C"
