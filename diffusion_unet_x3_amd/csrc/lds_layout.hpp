// LDS layouts of the conv3x3 kernels, shared by the kernels and the planner.
//
// Forward / backward-data, float32 (MFMA 32x32x2, reduction pairs of input
// channels at one tap):
//   x tile : [chunk][imgs][th + 2][RS]  floats, RS = tw + 8.  Image column
//            cc in [-1, tw] of the block sits at row offset 4 + cc, so the
//            interior starts 16-byte aligned and each row is written with
//            128-bit stores; rows/columns outside the image hold zero.
//   w tile : [chunk][9][co_tile + 1]  floats (the +1 keeps the transposing
//            stores free of bank conflicts).
//
// Forward / backward-data, bfloat16 (MFMA 32x32x16, each lane supplies 8
// consecutive input channels at one tap; 16-channel fills; both tiles are
// double-buffered):
//   x tile : [2][plane] words, a plane = [imgs][th + 2][RS] 16-byte words,
//            one word = 8 channels of one pixel, so the MFMA operand is a
//            single 128-bit LDS read; RS = tw + 9 (24 for tw = 8), image column cc
//            at 4 + cc.
//   w tile : [9][2][co_tile] words (8 input channels of one tap and output
//            channel).
//
// Backward-weight, float32 (MFMA 32x32x2, reduction pairs of pixels):
//   g tile : [64 k][P + 1]  floats, P = imgs * th * tw pixels per chunk.
//   x tile : [64 c][PLW]  floats, PLW = imgs * (th + 2) * (tw + 2) rounded up
//            to odd so that 32 channels read at one pixel hit 32 banks;
//            image column cc in [-1, tw] sits at row offset 1 + cc.
#pragma once

#if defined(__HIPCC__)
#define CONV3X3_HD __host__ __device__
#else
#define CONV3X3_HD
#endif

namespace conv3x3 {

// ---- forward / backward-data, float32 ----
CONV3X3_HD constexpr int fwd_f32_rs(int tw) { return tw + 8; }
CONV3X3_HD constexpr int fwd_f32_plane(int imgs, int th, int tw) {
  return imgs * (th + 2) * fwd_f32_rs(tw);
}
CONV3X3_HD constexpr int fwd_f32_wstride(int co_tile) { return co_tile + 1; }
CONV3X3_HD constexpr int fwd_f32_x_floats(int cb, int imgs, int th, int tw) {
  return cb * fwd_f32_plane(imgs, th, tw);
}
CONV3X3_HD constexpr int fwd_f32_w_floats(int cb, int co_tile) {
  return cb * 9 * fwd_f32_wstride(co_tile);
}
CONV3X3_HD constexpr int fwd_f32_lds_bytes(int cb, int imgs, int th, int tw, int co_tile) {
  return 4 * (fwd_f32_x_floats(cb, imgs, th, tw) + fwd_f32_w_floats(cb, co_tile));
}

// Forward of a stride-2 convolution, float32: for an output block of th x tw
// pixels the input rows 2 h0 - 1 .. 2 h0 + 2 th - 1 are staged (2 th + 1 of
// them) with their columns split by parity: odd input columns 2 (w0 + j) - 1,
// j = 0..tw, at row offset kS2Odd + j, even columns 2 (w0 + j) at kS2Even(tw)
// + j.  The taps s = 0, 1, 2 of output column j then read odd j, even j and
// odd j + 1: unit stride across the lanes.  Both runs are 16-byte aligned
// where the loader writes them (odd j = 1.., even j = 0..).
constexpr int kS2Odd = 3;
CONV3X3_HD constexpr int fwd_f32_s2_even(int tw) { return tw + 8; }
CONV3X3_HD constexpr int fwd_f32_s2_rs(int tw) { return 2 * tw + 8; }
CONV3X3_HD constexpr int fwd_f32_s2_plane(int imgs, int th, int tw) {
  return imgs * (2 * th + 1) * fwd_f32_s2_rs(tw);
}
CONV3X3_HD constexpr int fwd_f32_s2_lds_bytes(int cb, int imgs, int th, int tw, int co_tile) {
  return 4 * (cb * fwd_f32_s2_plane(imgs, th, tw) + fwd_f32_w_floats(cb, co_tile));
}
// Backward-data of an upsampling convolution reads a 4 x 4 window of g at
// stride 2 per output pixel: one more staged row (2 th + 2) and one more
// even column (j = tw), so the row stride grows to keep the even run 16-byte
// aligned.
CONV3X3_HD constexpr int fwd_f32_u2b_rs(int tw) { return 2 * tw + 12; }
CONV3X3_HD constexpr int fwd_f32_u2b_plane(int imgs, int th, int tw) {
  return imgs * (2 * th + 2) * fwd_f32_u2b_rs(tw);
}
CONV3X3_HD constexpr int fwd_f32_u2b_lds_bytes(int cb, int imgs, int th, int tw, int co_tile) {
  return 4 * (cb * fwd_f32_u2b_plane(imgs, th, tw) + fwd_f32_w_floats(cb, co_tile));
}

// ---- forward / backward-data, bfloat16 ----
// Plane of one 8-channel group, in 16-byte words, padded to 8 mod 16 words
// so that the two groups' words written by one transpose step fall in
// different banks.
// Row stride in words.  A 128-bit LDS read serves the lane groups
// {0-7, 24-31} and {8-15, 16-23} (and the same in the upper half) together,
// and the 16 words of a group need 16 different bank groups (word mod 16).
// tw = 8: the MFMA pixel operand is four rows of 8, conflict-free with a
// stride of 8 mod 16.  Wider tiles: odd, so that the staging lanes, which
// write rows-fastest, put 16 consecutive rows in 16 different bank groups
// (the operand reads of tw >= 32 are conflict-free for any stride; tw = 16
// would need 0 mod 16, which makes the staging stores 8-way conflicts and
// measured slower overall).
CONV3X3_HD constexpr int fwd_bf16_rs(int tw) { return tw == 8 ? 24 : tw + 9; }
CONV3X3_HD constexpr int fwd_bf16_plane(int imgs, int th, int tw) {
  return imgs * (th + 2) * fwd_bf16_rs(tw) + ((8 - (imgs * (th + 2) * fwd_bf16_rs(tw)) % 16) + 16) % 16;
}
// Two buffers of the x tile (two 8-channel planes) and of the weight tile.
CONV3X3_HD constexpr int fwd_bf16_lds_bytes(int imgs, int th, int tw, int co_tile) {
  return 2 * 16 * (2 * fwd_bf16_plane(imgs, th, tw) + 9 * 2 * co_tile);
}

// ---- backward-weight, float32 ----
CONV3X3_HD constexpr int wgrad_f32_gstride(int imgs, int th, int tw) { return imgs * th * tw + 1; }
CONV3X3_HD constexpr int wgrad_f32_rs(int tw) { return tw + 2; }
CONV3X3_HD constexpr int wgrad_f32_plane(int imgs, int th, int tw) {
  return (imgs * (th + 2) * wgrad_f32_rs(tw)) | 1;
}
// Two buffers of each tile (chunk i + 1 is staged while chunk i is read).
CONV3X3_HD constexpr int wgrad_f32_lds_bytes(int imgs, int th, int tw) {
  return 2 * 4 * 64 * (wgrad_f32_gstride(imgs, th, tw) + wgrad_f32_plane(imgs, th, tw));
}
// Stride 2 (the chunk's th x tw pixels are output pixels): x holds the
// 2 th + 1 input rows 2 h0 - 1 .. of 2 tw + 1 columns 2 w0 - 1 .. (column t
// at row offset t), about four times the stride-1 tile, so both tiles are
// single-buffered.
CONV3X3_HD constexpr int wgrad_f32_s2_rs(int tw) { return 2 * tw + 2; }
CONV3X3_HD constexpr int wgrad_f32_s2_plane(int imgs, int th, int tw) {
  return (imgs * (2 * th + 1) * wgrad_f32_s2_rs(tw)) | 1;
}
CONV3X3_HD constexpr int wgrad_f32_s2_lds_bytes(int imgs, int th, int tw) {
  return 4 * 64 * (wgrad_f32_gstride(imgs, th, tw) + wgrad_f32_s2_plane(imgs, th, tw));
}

// ---- backward-weight, bfloat16 ----
// g tile : [64 k][P + 8] bf16 (row stride 2P + 16 bytes: eight lanes reading
//          eight k rows at one pixel hit eight different 16-byte bank groups).
// x tile : [64 c][PLX] bf16, PLX = imgs * (th + 2) * (tw + 16) rounded up to
//          8 mod 64 (a plane is 16 mod 128 bytes, for the same reason); image
//          column cc in [-1, tw] sits at row offset 8 + cc, so 8-pixel runs
//          starting at a multiple-of-8 column are 16-byte aligned.
CONV3X3_HD constexpr int wgrad_bf16_gstride(int imgs, int th, int tw) { return imgs * th * tw + 8; }
CONV3X3_HD constexpr int wgrad_bf16_rs(int tw) { return tw + 16; }
CONV3X3_HD constexpr int wgrad_bf16_plane(int imgs, int th, int tw) {
  return imgs * (th + 2) * wgrad_bf16_rs(tw) +
         ((8 - (imgs * (th + 2) * wgrad_bf16_rs(tw)) % 64) + 64) % 64;
}
// Two buffers of each tile (chunk i + 1 is staged while chunk i is read).
CONV3X3_HD constexpr int wgrad_bf16_lds_bytes(int imgs, int th, int tw) {
  return 2 * 2 * 64 * (wgrad_bf16_gstride(imgs, th, tw) + wgrad_bf16_plane(imgs, th, tw));
}

// ---- backward-weight, at most four input channels (packed pairs) ----
// Eight waves per workgroup (two per 32-row k block, taking alternate
// chunks), each with private g rows:
//   g rows : [8 waves][32 k][68] floats (64 pixels; rows 68 floats apart put
//            the 8 lanes of a 128-bit read on all 32 banks).
//   x      : one group of kStemGroup chunks, shared (wave w stages chunk w
//            of the group): [group chunk][cp][XP] floats, a plane = th + 2
//            rows of XR floats, XR = tw + 2 padded to 3 (mod 32) and XP
//            padded to 9 (mod 32), so that (channel, tap) column
//            e = 9 c + 3 r + s reads bank e + const; then a plane of zeros
//            (which also takes the staging items past the planes), a bank
//            shift and a plane of ones.
// Split-K slot: [K][32 NB] floats per slice, NB = 32-column MFMA blocks of
// the 9C pairs and the bias column.
constexpr int kStemWaves = 8;
constexpr int kStemGroup = 8;  // chunks per staged x group
CONV3X3_HD constexpr int stem_xr(int tw) { return tw + 2 + ((3 - (tw + 2)) % 32 + 32) % 32; }
CONV3X3_HD constexpr int stem_xp(int th, int tw) {
  return (th + 2) * stem_xr(tw) + ((9 - (th + 2) * stem_xr(tw)) % 32 + 32) % 32;
}
CONV3X3_HD constexpr int stem_x_items(int th, int tw, int cp) {  // per lane (a chunk per wave)
  return (cp * stem_xp(th, tw) + 63) / 64;
}
CONV3X3_HD constexpr int stem_lds_bytes(int th, int tw, int cp) {
  return 4 * (kStemWaves * 32 * 68 + kStemGroup * cp * stem_xp(th, tw) + stem_xp(th, tw) + 32 +
              stem_xp(th, tw));
}
CONV3X3_HD constexpr int stem_slot_columns(int C) { return 32 * ((9 * C + 1 + 31) / 32); }

// ---- forward, at most four input channels, bfloat16 (packed pairs) ----
// 128-pixel tiles (tw x th); two buffers of the x tile: [c][XP] floats (the
// planes as above, th + 2 rows of XR, bfloat16 widened), then a plane of
// zeros.
// ---- backward-data, at most three output channels ----
// P, the (channel, tap)-row sums of a band of th + 2 image rows, is kept in
// LDS for at most kStemBdPx pixels; w^T for at most kStemBdMaxK channels.
constexpr int kStemBdMaxK = 128;
constexpr int kStemBdPx = 640;
// Output rows per band: 8, fewer for rows wider than 64 pixels (0: a row
// too wide for the band's LDS).
CONV3X3_HD constexpr int stem_bd_rows(int w) {
  return w < 1 || kStemBdPx / w < 3 ? 0 : (kStemBdPx / w - 2 < 8 ? kStemBdPx / w - 2 : 8);
}
CONV3X3_HD constexpr int stem_bd_lds_bytes() { return 4 * (27 * kStemBdPx + kStemBdMaxK * 32); }

constexpr int kStemFwdPix = 128;
constexpr int kStemFwdCo = 64;  // output channels per workgroup
CONV3X3_HD constexpr int stem_fwd_x_floats(int th, int tw, int c) {
  return (c + 1) * stem_xp(th, tw);
}
CONV3X3_HD constexpr int stem_fwd_lds_bytes(int th, int tw, int cp) {
  return 2 * 4 * stem_fwd_x_floats(th, tw, cp);
}

}  // namespace conv3x3
