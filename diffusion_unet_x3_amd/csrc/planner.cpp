// Launch planning (host only).  See planner.hpp for the tiling it describes.
#include "planner.hpp"

#include "lds_layout.hpp"
#include "tile_configs.hpp"

namespace conv3x3 {

namespace {

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Tiles of `tile` channels over C channels held by one tensor (c0 < 0 or
// c0 == C) or by two (c0 and C - c0 channels, tiled separately).
int channel_tiles(int C, int c0, int tile) {
  if (c0 < 0 || c0 >= C) return ceil_div(C, tile);
  return ceil_div(c0, tile) + ceil_div(C - c0, tile);
}

struct Block {
  int tw, th, imgs;
};

bool fwd_cfg_exists(int dtype, const Block& b, int co, int wco, int nw) {
#define CONV3X3_X5(TW, TH, IMGS, CO, WCO) \
  if (b.tw == TW && b.th == TH && b.imgs == IMGS && co == CO && wco == WCO && nw == 4) return true;
#define CONV3X3_X6(TW, TH, IMGS, CO, WCO, NW) \
  if (b.tw == TW && b.th == TH && b.imgs == IMGS && co == CO && wco == WCO && nw == NW) return true;
  if (dtype == kF32) {
    CONV3X3_FWD_F32_CONFIGS(CONV3X3_X5)
  } else {
    CONV3X3_FWD_BF16_CONFIGS(CONV3X3_X6)
  }
#undef CONV3X3_X5
#undef CONV3X3_X6
  return false;
}

bool wgrad_cfg_exists(int dtype, const Block& b) {
#define CONV3X3_X(TW, TH, IMGS) \
  if (b.tw == TW && b.th == TH && b.imgs == IMGS) return true;
  if (dtype == kF32) {
    CONV3X3_WGRAD_F32_CONFIGS(CONV3X3_X)
  } else {
    CONV3X3_WGRAD_BF16_CONFIGS(CONV3X3_X)
  }
#undef CONV3X3_X
  return false;
}

// A pixel block of `bm` pixels for an H x W image: as wide as the image
// allows (power of two, 8..64) and as tall as the block; when the image is
// shorter than the block, several images share it.
Block pick_block(int bm, int H, int W) {
  Block b;
  b.tw = W > 32 ? 64 : W > 16 ? 32 : W > 8 ? 16 : 8;
  const int rows = bm / b.tw;
  int hp = 1;
  while (hp < H) hp *= 2;
  if (rows <= hp) {
    b.th = rows;
    b.imgs = 1;
  } else {
    b.th = hp;
    b.imgs = rows / hp;
  }
  return b;
}

int blocks_of(const Block& b, int N, int H, int W) {
  return ceil_div(N, b.imgs) * ceil_div(H, b.th) * ceil_div(W, b.tw);
}

// Grids smaller than this leave compute units idle; the planner then falls
// back to smaller workgroup tiles.
constexpr int kMinWGs = 256;

// Number of workgroups the weight-gradient pass aims for: one 12-wave
// workgroup per compute unit on a 256-CU device.
constexpr int kWgradTargetWGs = 256;

}  // namespace

long fwd_slot_elems(const Problem& p) {
  return (long)p.N * (p.pass == kFwd ? p.K : p.C) * p.H * p.W;
}

size_t wgrad_workspace_bytes(const Plan& pl, int C, int K) {
  if (pl.split <= 1) return 0;
  return (size_t)pl.split * ((size_t)K * C * 9 + (size_t)K) * sizeof(float);
}

bool stem_bwd_data_fits(int C, int K, int W) {
  return C >= 1 && C <= 3 && K >= 1 && K <= kStemBdMaxK && stem_bd_rows(W) >= 1;
}

bool plan(const Problem& p, Plan* out) {
  Plan pl;
  pl.pass = p.pass;
  pl.dtype = p.dtype;
  if (p.pass == kBwdData && p.stem) {
    // At most three output channels: the (channel, tap)-row backward-data,
    // one workgroup per band of th output rows of one image.
    if (!stem_bwd_data_fits(p.C, p.K, p.W)) return false;
    pl.tw = p.W;
    pl.th = stem_bd_rows(p.W);
    pl.imgs = 1;
    pl.tile_co = p.C;
    pl.wave_co = 1;
    pl.chunk = p.K;
    pl.threads = 512;
    pl.tiles_w = 1;
    pl.tiles_h = ceil_div(p.H, pl.th);
    pl.tiles_n = p.N;
    pl.grid_x = p.N * pl.tiles_h;
    pl.grid_y = 1;
    pl.grid_z = 1;
    pl.split = 1;
    pl.stem = 1;
    pl.lds_bytes = stem_bd_lds_bytes();
    *out = pl;
    return true;
  }
  if (p.pass == kFwd && p.stem && p.dtype == kBF16) {
    // At most four input channels (bfloat16): the packed-pair forward -- 64
    // output channels x 128-pixel tiles (tw x th, tw the narrowest power of
    // two holding a row, 8 to 64), weights in registers, a persistent grid
    // of two workgroups per compute unit (or one per tile) looping over the
    // tiles, so that each wave's stores drain while it computes its next
    // tile (measured on N = 32, 3 -> 128, 64x64: one tile per workgroup
    // 28.2 us, four workgroups per unit 20.7, two 18.3, one 18.9).
    int tw = 8;
    while (tw < 64 && tw < p.W) tw *= 2;
    pl.tw = tw;
    pl.th = kStemFwdPix / tw;
    pl.imgs = 1;
    pl.tile_co = kStemFwdCo;
    pl.wave_co = 1;
    pl.tile_ci = p.C;
    pl.chunk = p.C;
    pl.threads = 256;
    pl.tiles_w = ceil_div(p.W, pl.tw);
    pl.tiles_h = ceil_div(p.H, pl.th);
    pl.tiles_n = p.N;
    pl.nchunks = pl.tiles_n * pl.tiles_h * pl.tiles_w;  // pixel tiles
    const int tiles_k = ceil_div(p.K, kStemFwdCo);
    int wgs = 2 * kMinWGs / tiles_k;
    if (wgs < 1) wgs = 1;
    pl.grid_x = pl.nchunks < wgs ? pl.nchunks : wgs;
    pl.grid_y = tiles_k;
    pl.grid_z = 1;
    pl.split = 1;
    pl.stem = 1;
    pl.lds_bytes = stem_fwd_lds_bytes(pl.th, pl.tw, p.C <= 3 ? 3 : 4);
    *out = pl;
    return true;
  }
  if (p.pass == kFwd || p.pass == kBwdData) {
    const int cout = p.pass == kFwd ? p.K : p.C;
    const int cout0 = p.pass == kFwd ? -1 : p.C0;  // backward-data: dx may be two tensors
    // Candidate workgroup tiles, preferred first: (pixels, channels, waves
    // along channels).
    struct Cand {
      int bm, co, wco, nw;
    };
    Cand cands[3];
    int ncand;
    if (p.dtype == kF32 && p.quad) {
      // four accumulator sets per wave (one per output parity class) fit
      // only with one 32 x 32 tile per wave
      cands[0] = Cand{64, 64, 2, 4};
      ncand = 1;
    } else if (p.dtype == kF32) {
      cands[0] = cout <= 64 ? Cand{256, 64, 1, 4} : Cand{128, 128, 2, 4};
      cands[1] = Cand{64, 64, 2, 4};
      ncand = 2;
    } else if (cout > 64 && !p.four_waves) {
      cands[0] = Cand{256, 128, 1, 8};
      cands[1] = Cand{128, 64, 2, 4};
      cands[2] = Cand{64, 64, 2, 4};
      ncand = 3;
    } else {
      cands[0] = Cand{128, 64, 2, 4};
      cands[1] = Cand{64, 64, 2, 4};
      ncand = 2;
    }
    // Take the first candidate that fills the device without wasting much of
    // its tile on pixels past the image (a block taller than the image or a
    // ragged edge); otherwise the last (smallest) one that fits.
    Block blks[3];
    double eff[3];
    int wgs[3];
    double best_eff = 0.0;
    for (int i = 0; i < ncand; ++i) {
      Block b = pick_block(cands[i].bm, p.H, p.W);
      if (!fwd_cfg_exists(p.dtype, b, cands[i].co, cands[i].wco, cands[i].nw))
        b = Block{b.tw, cands[i].bm / b.tw, 1};
      blks[i] = b;
      eff[i] = 0.0;
      wgs[i] = 0;
      if (!fwd_cfg_exists(p.dtype, b, cands[i].co, cands[i].wco, cands[i].nw)) continue;
      wgs[i] = blocks_of(b, p.N, p.H, p.W) * channel_tiles(cout, cout0, cands[i].co);
      eff[i] = (double)p.N * p.H * p.W * cout / ((double)wgs[i] * cands[i].bm * cands[i].co);
      if (eff[i] > best_eff) best_eff = eff[i];
    }
    int pick = -1;
    for (int i = 0; i < ncand; ++i) {
      if (wgs[i] == 0) continue;
      pick = i;
      if (wgs[i] >= kMinWGs && eff[i] >= 0.8 * best_eff) break;
    }
    // bf16 with a workspace: when the eight-wave 256 x 128 tile leaves the
    // device short of workgroups (small images) and the reduction is long
    // (>= 32 fills of 16 channels), keep that tile and split the reduction
    // instead of falling back to the smaller tiles, which re-stage all the
    // weights for every pixel tile.  The split stays within one round of
    // workgroups, keeps at least 8 fills per slice and must bring the grid
    // to three quarters of a round (measured: shorter reductions, a second
    // round of workgroups and split grids of half a round all lose to the
    // small tiles; 48- and 56-fill reductions on 16x16 images gain 10-16%).
    // From 24 fills a split in two (12+ fills per slice) pays too: 384 -> 384
    // channels at 16x16, N = 32: forward 45.6 -> 39.1 us, backward-data 40.7
    // -> 38.2 us against the 128 x 64 tile; a split in three (8 fills per
    // slice, 256 -> 384 backward-data) lost, 31.0 -> 33.2 us.
    int split = 1;
    const int cin = p.pass == kFwd ? p.C : p.K;
    const int fills = ceil_div(cin, p.dtype == kF32 ? 8 : 16);  // channels per fill
    if (p.allow_split && p.dtype == kBF16 && cout > 64 && wgs[0] > 0 && wgs[0] < kMinWGs &&
        fills >= 24 && eff[0] >= 0.8 * best_eff && (cout0 < 0 || cout0 >= cout)) {
      // (at least 4 fills per slice: the 512-channel 8x8 layers at N = 32,
      // 32 big tiles split in eight, forward 35.8 -> 28.3 us, backward-data
      // 28.9 -> 27.9 us against the 64 x 64 tile; at least 8 fills per
      // slice before the forward epilogue became branch-free)
      int s = kMinWGs / wgs[0];
      if (s > fills / 4) s = fills / 4;
      if (s > 8) s = 8;
      if (fills < 32 && s > 2) s = 2;
      if (s >= 2 && wgs[0] * s >= 3 * kMinWGs / 4) {
        pick = 0;
        split = s;
      }
    }
    // With a workspace, smallest tile (both dtypes): when the 64 x 64 tiles
    // make half a round to one round of workgroups and the reduction has >=
    // 32 fills, split it (bf16 in two, float32 in four: >= 8 fills of 8
    // channels per slice), so several workgroups share each compute unit and
    // cover each other's per-fill staging and barrier waits.  Measured on
    // 8x8 images with 512 channels: bf16 backward-data 33.5 -> 30.3 us,
    // forward 39.5 -> 37.5 us (a split of four is slower, and 24-fill
    // reductions gain nothing); float32 forward 117 -> 103 us, backward-data
    // 124 -> 103 us (a split of two: 109 / 110 us).
    if (split == 1 && p.allow_split && !p.quad && !p.stride2 && pick == ncand - 1 && wgs[pick] > 0 &&
        2 * wgs[pick] >= kMinWGs && wgs[pick] <= kMinWGs && fills >= 32 &&
        (cout0 < 0 || cout0 >= cout))
      split = p.dtype == kF32 ? 4 : 2;
    // float32, smallest tile, at most a quarter round of workgroups (a small
    // batch of small images): up to 4 slices of at least 2 fills, so that
    // more compute units share the reduction.  Measured on N = 2, 64 -> 64,
    // 32x32 (32 workgroups): forward and backward-data 15.9 -> 6.9 us plus a
    // 2.7 us reduce; 8 slices of one fill: 6.1 + 3.8 us.
    if (split == 1 && p.allow_split && p.dtype == kF32 && !p.quad && !p.stride2 &&
        pick == ncand - 1 && wgs[pick] > 0 && 4 * wgs[pick] <= kMinWGs && fills >= 4 &&
        (cout0 < 0 || cout0 >= cout)) {
      int s = kMinWGs / wgs[pick];
      if (s > fills / 2) s = fills / 2;
      if (s > 4) s = 4;
      if (s >= 2) split = s;
    }
    const Block blk = pick >= 0 ? blks[pick] : Block{};
    if (pick < 0) return false;
    pl.tw = blk.tw;
    pl.th = blk.th;
    pl.imgs = blk.imgs;
    pl.tile_co = cands[pick].co;
    pl.wave_co = cands[pick].wco;
    pl.chunk = p.dtype == kF32 ? 8 : 16;
    pl.tiles_w = ceil_div(p.W, pl.tw);
    pl.tiles_h = ceil_div(p.H, pl.th);
    pl.tiles_n = ceil_div(p.N, pl.imgs);
    pl.grid_x = pl.tiles_n * pl.tiles_h * pl.tiles_w;
    pl.grid_y = channel_tiles(cout, cout0, pl.tile_co);
    pl.grid_z = 1;
    pl.split = 1;
    if (split > 1) {
      pl.chunks_per_split = ceil_div(fills, split);
      pl.split = ceil_div(fills, pl.chunks_per_split);  // no empty slices
      pl.grid_z = pl.split;
      pl.workspace_bytes = (size_t)pl.split * (size_t)fwd_slot_elems(p) * sizeof(float);
    }
    pl.threads = 64 * cands[pick].nw;
    pl.lds_bytes = p.dtype == kF32
        ? (p.stride2 && p.pass == kFwd
               ? fwd_f32_s2_lds_bytes(pl.chunk, pl.imgs, pl.th, pl.tw, pl.tile_co)
           : p.stride2 ? fwd_f32_u2b_lds_bytes(pl.chunk, pl.imgs, pl.th, pl.tw, pl.tile_co)
                     : fwd_f32_lds_bytes(pl.chunk, pl.imgs, pl.th, pl.tw, pl.tile_co))
        : fwd_bf16_lds_bytes(pl.imgs, pl.th, pl.tw, pl.tile_co);
    if (p.pass == kFwd) pl.lds_bytes += 4 * pl.tile_co;  // the tile's biases
  } else if (p.pass == kBwdWeight) {
    // float32: 64-pixel chunks (32 MFMA steps); bfloat16: 128-pixel chunks
    // (8 MFMA steps of 16 pixels), 64 for images at most 8 wide.
    const int cp = p.dtype == kF32 ? 64 : (p.W <= 8 ? 64 : 128);
    Block b = pick_block(cp, p.H, p.W);
    if (!wgrad_cfg_exists(p.dtype, b)) b = Block{b.tw, cp / b.tw, 1};
    if (!wgrad_cfg_exists(p.dtype, b)) return false;
    pl.tw = b.tw;
    pl.th = b.th;
    pl.imgs = b.imgs;
    pl.tile_co = 64;
    pl.tile_ci = 64;
    pl.chunk = b.tw * b.th * b.imgs;
    pl.tiles_w = ceil_div(p.W, pl.tw);
    pl.tiles_h = ceil_div(p.H, pl.th);
    pl.tiles_n = ceil_div(p.N, pl.imgs);
    pl.nchunks = pl.tiles_n * pl.tiles_h * pl.tiles_w;
    // One round of 12-wave workgroups (one per compute unit): as many
    // reduction slices as fit next to the channel tiles.
    const int tiles = ceil_div(p.K, pl.tile_co) * channel_tiles(p.C, p.C0, pl.tile_ci);
    int split = kWgradTargetWGs / tiles;
    if (split > pl.nchunks) split = pl.nchunks;
    if (split < 1) split = 1;
    pl.chunks_per_split = ceil_div(pl.nchunks, split);
    pl.split = ceil_div(pl.nchunks, pl.chunks_per_split);  // no empty slices
    pl.grid_x = ceil_div(pl.split * tiles, 8) * 8;  // whole XCD rounds; spare WGs exit
    pl.grid_y = 1;
    pl.grid_z = 1;
    pl.threads = 768;
    pl.lds_bytes = p.dtype == kF32
        ? (p.stride2 ? wgrad_f32_s2_lds_bytes(pl.imgs, pl.th, pl.tw)
                     : wgrad_f32_lds_bytes(pl.imgs, pl.th, pl.tw))
        : wgrad_bf16_lds_bytes(pl.imgs, pl.th, pl.tw);
    pl.workspace_bytes = wgrad_workspace_bytes(pl, p.C, p.K);
    if (p.C <= 4 && (p.C0 < 0 || p.C0 >= p.C) && !p.stride2) {
      // At most four input channels: the packed-pair kernel -- 128 k rows
      // and all 9C (channel, tap) pairs per 256-thread workgroup, 64-pixel
      // chunks tw x th (the narrowest power-of-two width holding a row, 8
      // to 64), about two workgroups per compute unit.  Its workspace also
      // bounds the other backward-weight variants' of the shape (they share
      // the size query), so the larger of the two is reported.
      Plan st = pl;
      int tw = 8;
      while (tw < 64 && tw < p.W) tw *= 2;
      st.tw = tw;
      st.th = 64 / tw;
      st.imgs = 1;
      st.tile_co = 128;
      st.tile_ci = p.C;
      st.chunk = 64;
      st.tiles_w = ceil_div(p.W, st.tw);
      st.tiles_h = ceil_div(p.H, st.th);
      st.tiles_n = p.N;
      st.nchunks = st.tiles_n * st.tiles_h * st.tiles_w;
      const int tiles_k = ceil_div(p.K, 128);
      int sp = kWgradTargetWGs / tiles_k;
      if (sp > st.nchunks) sp = st.nchunks;
      if (sp < 1) sp = 1;
      st.chunks_per_split = ceil_div(st.nchunks, sp);
      st.split = ceil_div(st.nchunks, st.chunks_per_split);
      st.grid_x = st.split * tiles_k;
      st.grid_y = 1;
      st.grid_z = 1;
      st.threads = 64 * kStemWaves;
      st.stem = 1;
      st.lds_bytes = stem_lds_bytes(st.th, st.tw, p.C <= 3 ? 3 : 4);
      // slots [split][K][32 NB] (the 9C pairs and the bias column)
      st.workspace_bytes = st.split > 1 ? (size_t)st.split * p.K * stem_slot_columns(p.C) *
                                              sizeof(float)
                                        : 0;
      const size_t ws = st.workspace_bytes > pl.workspace_bytes ? st.workspace_bytes
                                                                : pl.workspace_bytes;
      if (p.stem) pl = st;
      pl.workspace_bytes = ws;
    }
  } else {
    return false;
  }
  *out = pl;
  return true;
}

}  // namespace conv3x3
