// The tile configurations the conv3x3 kernels are instantiated for.  The
// planner only ever picks an entry of these lists, and each launcher
// dispatches over the same list, so a plan always has a kernel.
//
// Forward / backward-data entries: X(tw, th, imgs, co_tile, wave_co[, waves])
// -- a workgroup of `waves` wave64s (4 where not given) owns co_tile output
// channels x a pixel block of imgs x th x tw pixels; wave_co waves split the
// channels and waves / wave_co the pixels, each wave accumulating
// (co_tile / wave_co) x (block / (waves / wave_co)) outputs in 32x32 MFMA
// tiles.
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

// bfloat16: X(tw, th, imgs, co_tile, wave_co, waves).  Eight waves over
// 256-pixel x 128-channel tiles: the two waves of a SIMD split each fill's
// taps, each holding a 64-pixel x 128-channel wave tile; four waves over
// 128 x 64 (64 x 32 wave tiles) and 64 x 64 (32 x 32) for layers with few
// output pixels.
#define CONV3X3_FWD_BF16_CONFIGS(X)                                                   \
  X(64, 4, 1, 128, 1, 8) X(32, 8, 1, 128, 1, 8) X(16, 16, 1, 128, 1, 8)               \
  X(8, 32, 1, 128, 1, 8) X(8, 8, 4, 128, 1, 8)                                        \
  X(64, 2, 1, 64, 2, 4) X(32, 4, 1, 64, 2, 4) X(16, 8, 1, 64, 2, 4) X(8, 16, 1, 64, 2, 4) \
  X(8, 8, 2, 64, 2, 4)                                                                \
  X(64, 1, 1, 64, 2, 4) X(32, 2, 1, 64, 2, 4) X(16, 4, 1, 64, 2, 4) X(8, 8, 1, 64, 2, 4)

// Backward-weight pixel chunks: X(tw, th, imgs).
#define CONV3X3_WGRAD_F32_CONFIGS(X) X(64, 1, 1) X(32, 2, 1) X(16, 4, 1) X(8, 8, 1)
// bfloat16: 128-pixel chunks; 64 for images at most 8 wide (two buffers of
// the 8-wide layout at 128 pixels would not fit the LDS).
#define CONV3X3_WGRAD_BF16_CONFIGS(X) X(64, 2, 1) X(32, 4, 1) X(16, 8, 1) X(8, 16, 1) X(8, 8, 1)
