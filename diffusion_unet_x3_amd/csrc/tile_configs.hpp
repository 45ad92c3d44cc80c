// The tile configurations the conv3x3 kernels are instantiated for.  The
// planner only ever picks an entry of these lists, and each launcher
// dispatches over the same list, so a plan always has a kernel.
//
// Forward / backward-data entries: X(tw, th, imgs, co_tile, wave_co) -- a
// workgroup of 4 wave64s owns co_tile output channels x a pixel block of
// imgs x th x tw pixels; wave_co waves split the channels and 4 / wave_co
// the pixels, each wave accumulating (co_tile / wave_co) x (block / (4 /
// wave_co)) outputs in 32x32 MFMA tiles.
#pragma once

// float32: 64x64 wave tiles (4 MFMAs per reduction step) with 128-channel
// tiles over 128 pixels or 64-channel tiles over 256 pixels; 32x32 wave tiles
// (64 x 64 workgroup tiles) when the big tiles leave compute units idle.
#define CONV3X3_FWD_F32_CONFIGS(X)                                                    \
  X(64, 2, 1, 128, 2) X(32, 4, 1, 128, 2) X(16, 8, 1, 128, 2) X(8, 16, 1, 128, 2)     \
  X(8, 8, 2, 128, 2)                                                                  \
  X(64, 4, 1, 64, 1) X(32, 8, 1, 64, 1) X(16, 16, 1, 64, 1) X(16, 8, 2, 64, 1)        \
  X(8, 32, 1, 64, 1) X(8, 16, 2, 64, 1) X(8, 8, 4, 64, 1)                             \
  X(64, 1, 1, 64, 2) X(32, 2, 1, 64, 2) X(16, 4, 1, 64, 2) X(8, 8, 1, 64, 2)

// bfloat16: 64 x 128 wave tiles (8 MFMAs per step) over 256-pixel x
// 128-channel workgroup tiles; 32 x 64 wave tiles over 128 x 64; 32 x 32
// over 64 x 64 for layers with few output pixels.
#define CONV3X3_FWD_BF16_CONFIGS(X)                                                   \
  X(64, 4, 1, 128, 2) X(32, 8, 1, 128, 2) X(16, 16, 1, 128, 2) X(8, 32, 1, 128, 2)    \
  X(64, 2, 1, 64, 2) X(32, 4, 1, 64, 2) X(16, 8, 1, 64, 2) X(8, 16, 1, 64, 2)         \
  X(8, 8, 2, 64, 2)                                                                   \
  X(64, 1, 1, 64, 2) X(32, 2, 1, 64, 2) X(16, 4, 1, 64, 2) X(8, 8, 1, 64, 2)

// Backward-weight pixel chunks: X(tw, th, imgs).
#define CONV3X3_WGRAD_F32_CONFIGS(X) X(64, 1, 1) X(32, 2, 1) X(16, 4, 1) X(8, 8, 1)
#define CONV3X3_WGRAD_BF16_CONFIGS(X) X(64, 2, 1) X(32, 4, 1) X(16, 8, 1) X(8, 16, 1) X(8, 8, 2)
