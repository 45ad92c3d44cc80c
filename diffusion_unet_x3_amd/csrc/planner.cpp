// Launch planning (host only).  See planner.hpp for the tiling it describes.
#include "planner.hpp"

#include "lds_layout.hpp"

namespace conv3x3 {

namespace {

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Pixel block for the forward-type kernels: 128 pixels, as wide as the
// image allows (power of two, 8..64), two images per block for images of
// at most 8x8.
int fwd_geom(int H, int W) {
  if (W > 32) return kG64x2;
  if (W > 16) return kG32x4;
  if (W > 8) return kG16x8;
  if (H > 8) return kG8x16;
  return kG8x8x2;
}

// Pixel chunk for the weight-gradient kernel: 64 pixels.
int wgrad_geom(int W) {
  if (W > 32) return kG64x1;
  if (W > 16) return kG32x2;
  if (W > 8) return kG16x4;
  return kG8x8;
}

// Number of workgroups the weight-gradient pass aims for: one 12-wave
// workgroup per compute unit on a 256-CU device.
constexpr int kWgradTargetWGs = 256;

}  // namespace

size_t wgrad_workspace_bytes(const Plan& pl, int C, int K) {
  if (pl.split <= 1) return 0;
  return (size_t)pl.split * ((size_t)K * C * 9 + (size_t)K) * sizeof(float);
}

bool plan(const Problem& p, Plan* out) {
  Plan pl;
  pl.pass = p.pass;
  pl.dtype = p.dtype;
  if (p.pass == kFwd || p.pass == kBwdData) {
    const int cin = p.pass == kFwd ? p.C : p.K;
    const int cout = p.pass == kFwd ? p.K : p.C;
    (void)cin;
    pl.geom = fwd_geom(p.H, p.W);
    GeomDims d = geom_dims(pl.geom);
    pl.tw = d.tw;
    pl.th = d.th;
    pl.imgs = d.imgs;
    pl.tile_co = cout > 64 ? 128 : 64;
    // Channels per LDS fill: 16 with 64-channel tiles, 8 with 128-channel
    // tiles, so every fill holds the same 144 MFMA steps per wave.
    pl.chunk = p.dtype == kF32 ? (pl.tile_co == 64 ? 16 : 8) : 16;
    pl.tiles_w = ceil_div(p.W, pl.tw);
    pl.tiles_h = ceil_div(p.H, pl.th);
    pl.tiles_n = ceil_div(p.N, pl.imgs);
    pl.grid_x = pl.tiles_n * pl.tiles_h * pl.tiles_w;
    pl.grid_y = ceil_div(cout, pl.tile_co);
    pl.grid_z = 1;
    pl.threads = 256;
    pl.lds_bytes = p.dtype == kF32
        ? fwd_f32_lds_bytes(pl.chunk, pl.imgs, pl.th, pl.tw, pl.tile_co)
        : fwd_bf16_lds_bytes(pl.chunk, pl.imgs, pl.th, pl.tw, pl.tile_co, p.pass == kBwdData);
    pl.split = 1;
  } else if (p.pass == kBwdWeight) {
    // float32: 64-pixel chunks (32 MFMA steps); bfloat16: 128-pixel chunks
    // (8 MFMA steps of 16 pixels).
    pl.geom = p.dtype == kF32 ? wgrad_geom(p.W) : fwd_geom(p.H, p.W);
    GeomDims d = geom_dims(pl.geom);
    pl.tw = d.tw;
    pl.th = d.th;
    pl.imgs = d.imgs;
    pl.tile_co = 64;
    pl.tile_ci = 64;
    pl.chunk = d.tw * d.th * d.imgs;
    pl.tiles_w = ceil_div(p.W, pl.tw);
    pl.tiles_h = ceil_div(p.H, pl.th);
    pl.tiles_n = ceil_div(p.N, pl.imgs);
    pl.nchunks = pl.tiles_n * pl.tiles_h * pl.tiles_w;
    const int tiles = ceil_div(p.K, pl.tile_co) * ceil_div(p.C, pl.tile_ci);
    int split = ceil_div(kWgradTargetWGs, tiles);
    if (split > pl.nchunks) split = pl.nchunks;
    if (split < 1) split = 1;
    pl.chunks_per_split = ceil_div(pl.nchunks, split);
    pl.split = ceil_div(pl.nchunks, pl.chunks_per_split);  // no empty slices
    pl.grid_x = pl.split;
    pl.grid_y = ceil_div(p.C, pl.tile_ci);
    pl.grid_z = ceil_div(p.K, pl.tile_co);
    pl.threads = 768;
    pl.lds_bytes = p.dtype == kF32
        ? wgrad_f32_lds_bytes(pl.imgs, pl.th, pl.tw)
        : wgrad_bf16_lds_bytes(pl.imgs, pl.th, pl.tw);
    pl.workspace_bytes = wgrad_workspace_bytes(pl, p.C, p.K);
  } else {
    return false;
  }
  *out = pl;
  return true;
}

}  // namespace conv3x3
