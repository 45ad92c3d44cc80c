// Forward (+bias) and backward-data 3x3 convolution, bfloat16 inputs with
// float32 accumulation and output, gfx950.
//
// The same implicit GEMM as the float32 kernel (rows: output channels,
// columns: pixels, reduction: 9 taps x input channels), on
// v_mfma_f32_32x32x16_bf16.  That MFMA takes 8 consecutive reduction
// elements per lane, so a reduction step is one tap x 16 input channels:
// lanes 0-31 supply channels 0-7 and lanes 32-63 channels 8-15 of a
// 16-channel LDS fill.  To make the pixel operand a single 128-bit LDS read,
// the x tile is stored channel-interleaved: one 16-byte LDS word holds 8
// channels of one pixel ([group][img][row][col] words).  A lane loads an
// 8 x 8 block (8 pixels of 8 channels, eight 128-bit NCHW row loads) and
// transposes it in registers with byte permutes into eight words.  No global
// memory is transposed.
//
// Weights, as one 16-byte word per (tap, 8-channel group, output channel):
//   forward       : w[co, 16f + 8g .. + 7, 0..8] is one contiguous, 16-byte
//                   aligned 144-byte run; a lane loads it as nine words and
//                   forms the nine tap words with byte permutes;
//   backward-data : the reduction channel is k, the slowest axis of w; a lane
//                   loads the same eight (c, tap) elements of eight rows
//                   w[k, co0.., ..] and transposes them like the x tile, the
//                   180-degree tap rotation applied in the store index.
//
// Workgroup: NW wave64s.  The compute waves (all four of a four-wave
// workgroup; waves 0-3, one per SIMD, of an eight-wave one) split the tile:
// WCO of them the BCO output channels and the rest the pixel block, each
// holding MI x NJ 32x32 accumulators.  The LDS tiles are double-buffered:
// while the MFMAs of fill i read one buffer, fill i + 1 (loaded into
// registers one fill ahead) is written into the other and the global loads
// of fill i + 2 are issued -- by the same waves between their MFMA groups
// (four waves), or by waves 4-7, which do nothing else (eight waves; the
// compute waves then hold 64 x 128 wave tiles, 6 operand reads per 8
// MFMAs).  One barrier per fill.  Forward accumulators start at the bias,
// so the epilogue is stores only.
//
// Either channel axis may be a concatenation of two tensors, as in the
// float32 kernel: source channels [0, cin0) from src and [cin0, Cin) from
// src1, output channels [0, cout0) to dst and [cout0, Cout) to dst1; every
// fill and every channel tile lies inside one tensor.  (The vector path
// needs cin0 % 16 == 0, so its fills are whole, and cout0 % 8 == 0.)
#include <type_traits>

#include "activation.hpp"
#include "common.hpp"
#include "launch.hpp"
#include "lds_layout.hpp"
#include "tile_configs.hpp"

namespace conv3x3 {

namespace {

// Word i of the 8 x 8 transpose of eight 8-element rows r[0..7] (16-bit
// elements): element j of the result is element i of row j.  Dword m packs
// rows 2m and 2m + 1, picked with one byte permute.
template <int I>
__device__ __forceinline__ u32x4 column_word(const u32x4* r) {
  // __builtin_amdgcn_perm(hi, lo, sel): selector bytes 0-3 pick bytes of lo,
  // 4-7 bytes of hi; result byte b is the byte named by selector byte b.
  constexpr uint32_t sel = (I & 1) ? 0x07060302u : 0x05040100u;
  u32x4 v;
  v.x = __builtin_amdgcn_perm(r[1][I >> 1], r[0][I >> 1], sel);
  v.y = __builtin_amdgcn_perm(r[3][I >> 1], r[2][I >> 1], sel);
  v.z = __builtin_amdgcn_perm(r[5][I >> 1], r[4][I >> 1], sel);
  v.w = __builtin_amdgcn_perm(r[7][I >> 1], r[6][I >> 1], sel);
  return v;
}

// Dword m (m = 0..3) of the tap-T word of a 72-element raw weight run
// (element ci * 9 + tap, ci = 0..7): elements (2m) * 9 + T and
// (2m + 1) * 9 + T, picked from their dwords with one byte permute.
template <int T, int M>
__device__ __forceinline__ uint32_t tap_dword(const uint32_t* d) {
  constexpr int E0 = (2 * M) * 9 + T, E1 = (2 * M + 1) * 9 + T;
  // __builtin_amdgcn_perm(hi, lo, sel): selector bytes 0-3 pick bytes of lo,
  // 4-7 bytes of hi; result byte b is the byte named by selector byte b.
  constexpr uint32_t sel = (uint32_t)(2 * (E0 & 1)) | (uint32_t)(2 * (E0 & 1) + 1) << 8 |
                           (uint32_t)(4 + 2 * (E1 & 1)) << 16 |
                           (uint32_t)(5 + 2 * (E1 & 1)) << 24;
  return __builtin_amdgcn_perm(d[E1 >> 1], d[E0 >> 1], sel);
}

template <int T>
__device__ __forceinline__ u32x4 tap_word(const uint32_t* d) {
  u32x4 v;
  v.x = tap_dword<T, 0>(d);
  v.y = tap_dword<T, 1>(d);
  v.z = tap_dword<T, 2>(d);
  v.w = tap_dword<T, 3>(d);
  return v;
}

}  // namespace

// ZG (backward-data): the source is a gradient gy at an activation's output,
// multiplied by act'(zsrc) and rounded to bfloat16 as it is staged.
// PRO: the input prologue -- forward: the staged input is
// a = SiLU(x * pscale[n, c] + pshift[n, c]) rounded to bfloat16;
// backward-data: the output is du = acc * SiLU'(u) with u from px (x, the
// forward's bfloat16 input), pscale and pshift at the output position.
template <int MODE, int TW, int TH, int IMGS, int BCO, int WCO, int NW, bool VEC, bool ZG,
          bool PRO, int XG = kGeoPlain>
__global__ __launch_bounds__(64 * NW) void fwd_bf16_kernel(
    const uint16_t* __restrict__ src, const uint16_t* __restrict__ src1, int cin0,
    const uint16_t* __restrict__ wt, const float* __restrict__ bias, float* __restrict__ dst,
    float* __restrict__ dst1, int cout0, int N, int Cin, int Cout, int H, int W, int tiles_w,
    int tiles_h, uint32_t src_bytes, uint32_t src1_bytes, uint32_t wt_bytes, uint32_t dst_bytes,
    uint32_t dst1_bytes, int act, float* __restrict__ zout, int outb, int per_split,
    float* __restrict__ part, const float* __restrict__ zsrc, const float* __restrict__ pscale,
    const float* __restrict__ pshift, const uint16_t* __restrict__ px, int geo) {
  constexpr int NT = 64 * NW;
  constexpr int CB = 16;
  constexpr int BM = IMGS * TH * TW;
  // XG: the vector path's source is an H/2 x W/2 tensor read at (h/2, w/2)
  // (kGeoUp) or zero-inserted (kGeoZero: only at even h, w); one source
  // tensor, no fusion.  The scalar path takes its geometry from `geo`.
  static_assert(XG == kGeoPlain || (VEC && !ZG && !PRO && (XG == kGeoUp || XG == kGeoZero)),
                "resampled vector staging: plain operands only");
  // Eight-wave workgroups are wave-specialised: waves 0-3 (one per SIMD)
  // only read operands from LDS and run MFMAs, waves 4-7 only stage tiles.
  // Four-wave workgroups do both in every wave.
  constexpr bool WSPEC = NW == 8;
  constexpr int NC = WSPEC ? 4 : NW;        // compute waves
  constexpr int NP = WSPEC ? 256 : NT;      // staging threads
  constexpr int WPX = NC / WCO;
  constexpr int MI = BCO / (32 * WCO);
  constexpr int NJ = BM / (32 * WPX);
  static_assert(MI >= 1 && NJ >= 1 && MI * 32 * WCO == BCO && NJ * 32 * WPX == BM,
                "tile does not split into 32x32 wave tiles");
  constexpr int RS = fwd_bf16_rs(TW);
  constexpr int HR = TH + 2;
  constexpr int PLW = fwd_bf16_plane(IMGS, TH, TW);  // words per 8-channel plane
  constexpr int XW = 2 * PLW;                        // words of one x buffer
  constexpr int WW = 9 * 2 * BCO;                    // words of one weight buffer
  constexpr int EW = BCO * 9 / 8;                    // raw weight words per k row (bwd-data)

  __shared__ u32x4 xs[2 * XW];
  __shared__ u32x4 wa[2 * WW];
  __shared__ float bias_s[MODE == kFwd ? BCO : 1];  // this tile's biases (0 without bias)

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const BlockOrigin o = block_origin<TW, TH, IMGS>(blockIdx.x, tiles_w, tiles_h);
  const long HW = (long)H * W;
  // This workgroup's output channel tile: channels col0 .. col0 + co_n - 1 of
  // output tensor `oseg` (ocs channels), channel co0 of the weight and bias.
  const int nt0 = (cout0 + BCO - 1) / BCO;
  const bool oseg = (int)blockIdx.y >= nt0;
  const int col0 = ((int)blockIdx.y - (oseg ? nt0 : 0)) * BCO;
  const int ocs = oseg ? Cout - cout0 : cout0;
  const int co0 = (oseg ? cout0 : 0) + col0;
  const int co_n = min(BCO, ocs - col0);
  // Reduction fills: nq0 over src's channels, then src1's.  A split
  // reduction (part != null) gives slice blockIdx.z the fills fbase ..
  // fbase + nchunks - 1; `chunk` below counts this workgroup's fills.
  const int nq0 = (cin0 + CB - 1) / CB;
  const int nfills = nq0 + (Cin - cin0 + CB - 1) / CB;
  const int fbase = part ? (int)blockIdx.z * per_split : 0;
  const int nchunks = part ? min(per_split, nfills - fbase) : nfills;
  // staging thread index (-1: this thread stages nothing)
  const int sp = WSPEC ? (wave >= NC ? tid - 64 * NC : -1) : tid;

  // ---- vector staging (W % 8 == 0, Cin % 16 == 0, 16-byte bases) ----
  // A staging thread owns items and holds them in registers from their
  // global loads until it writes them to LDS.  Four-wave workgroups keep two
  // register sets: the loads of fill i + 3 go into the set just written to
  // LDS as fill i + 1, so each load has two fills of MFMA work to arrive.
  // (Their threads stage either x or weights, so the two roles share the
  // registers of a set.)  Eight-wave workgroups keep one set, loaded one
  // fill ahead by their staging waves.  Items:
  //   x item (rr, q, img, g), sp in [0, XI): the 8 x 8 block of channels
  //     8g .. 8g + 7 of the fill x pixels 8q .. 8q + 7 of one staged row,
  //     as eight 128-bit row loads, written as eight channel-interleaved
  //     words;
  //   halo item, sp in [0, XH): 8 channels of one halo-column pixel;
  //   weight items, fill f: forward (co_l, g), co_l fastest: the 144-byte
  //     run w[co0 + co_l, 16f + 8g .. + 7, 0..8] (nine loads, nine tap
  //     words); backward-data (g, eb): word eb of the rows
  //     w[16f + 8g + i, co0.., ..], i = 0..7 (eight loads, transposed into
  //     eight words of 8 k each).
  //     Wave-specialised: items sp and sp + 256; otherwise the last WI
  //     threads, so that x and weight staging sit in different waves.
  constexpr int XI = 2 * IMGS * HR * (TW / 8);
  constexpr int XH = 2 * IMGS * HR * 2;
  constexpr int WI = MODE == kFwd ? 2 * BCO : 2 * EW;
  constexpr int WK = WSPEC ? (WI + NP - 1) / NP : 1;  // weight items per staging thread
  static_assert(XI <= NP && XH <= NP && (WSPEC || XI + WI <= NP), "staging items fit");
  constexpr int NSTG = MODE == kFwd ? 9 : 8;

  auto w_item = [&](int k) -> int {
    if (sp < 0) return -1;
    if constexpr (WSPEC) {
      const int it = sp + NP * k;
      return it < WI ? it : -1;
    } else {
      return sp >= NP - WI ? sp - (NP - WI) : -1;
    }
  };
  const bool xrole = sp >= 0 && sp < XI, hrole = sp >= 0 && sp < XH;
  // With a single tile across the width both halo columns are padding (the
  // tile starts at column 0 and is at least as wide as the image): their LDS
  // words stay zero and nothing is loaded for them.
  const bool halo_loads = tiles_w > 1;

  // (ZG: the source is a gradient gy multiplied by act'(zsrc) as it is
  // staged; its float32 z items take the registers of the second set)
  constexpr bool SPRO = PRO && MODE == kFwd;  // the prologue in the loader
  constexpr int NSET = (WSPEC || ZG || SPRO) ? 1 : 2;
  constexpr int WBASE = WSPEC ? 8 : 0;  // first register word of the weight items
  constexpr int SLOTS = WSPEC ? 8 + WK * NSTG : (NSTG > 8 ? NSTG : 8);
  u32x4 st[NSET][VEC ? SLOTS : 1];
  // halo values as loaded (one channel each); packed into a word when the
  // fill is written, so that issuing the loads never waits for them
  uint32_t hv[NSET][8];
  // ZG: z of the x item (row i's 8 floats in words 2i, 2i + 1) and of the
  // halo item
  f32x4 zx[NSET][ZG && VEC ? 16 : 1];
  float zh[NSET][ZG && VEC ? 8 : 1];
  // SPRO: scale (words 0, 1) and shift (2, 3) of the x item's and of the
  // halo item's 8 channels
  f32x4 psx[NSET][SPRO && VEC ? 4 : 1];
  f32x4 psh[NSET][SPRO && VEC ? 4 : 1];
#pragma unroll
  for (int k = 0; k < NSET; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i) hv[k][i] = 0u;
  // register set of fill f >= 1 (fill 0 is staged through set 0)
  using Set0 = std::integral_constant<int, 0>;
  using SetOdd = std::integral_constant<int, NSET - 1>;

  // Byte offsets, computed once; a fill adds the channel step.  Items
  // outside the tensors hold kOutside and read zero.
  const __amdgpu_buffer_rsrc_t sv0 = buffer_view(src, src_bytes);
  const __amdgpu_buffer_rsrc_t sv1 = buffer_view(src1, src1_bytes);
  const __amdgpu_buffer_rsrc_t wv = buffer_view(wt, wt_bytes);
  // z has the source's shape in float32: twice its byte offsets (below 2^31:
  // the caller keeps every float32 tensor under 2 GiB)
  const __amdgpu_buffer_rsrc_t zv = buffer_view(zsrc, ZG ? 2u * src_bytes : 0u);
  // scale / shift: [N][Cin] float32
  const uint32_t ps_bytes = SPRO ? 4u * (uint32_t)N * (uint32_t)Cin : 0u;
  const __amdgpu_buffer_rsrc_t psv = buffer_view(pscale, ps_bytes);
  const __amdgpu_buffer_rsrc_t ptv = buffer_view(pshift, ps_bytes);
  // bytes of one source channel plane
  const int SH = XG == kGeoPlain ? H : H >> 1, SW = XG == kGeoPlain ? W : W >> 1;
  const uint32_t hw2 = 2u * (uint32_t)(SH * SW);
  // x and halo item offsets in src (channel 8g of image n) and in src1
  uint32_t xoff = kOutside, hoff = kOutside, xoff1 = kOutside, hoff1 = kOutside, woff[WK];
  uint32_t pxo = kOutside, pho = kOutside;  // SPRO: scale / shift of the x and halo items
  int xdst = 0;  // LDS word of the x item's first pixel
#pragma unroll
  for (int k = 0; k < WK; ++k) woff[k] = kOutside;
  if constexpr (VEC) {
    if (xrole) {
      // rows fastest: with the odd row stride, 16 consecutive lanes write
      // 16 different bank groups
      int t = sp;
      const int rr = t % HR;
      t /= HR;
      const int q = t % (TW / 8);
      t /= TW / 8;
      const int img = t % IMGS;
      const int g = t / IMGS;
      const int n = o.n0 + img, h = o.h0 + rr - 1, w = o.w0 + 8 * q;
      if (n < N && h >= 0 && h < H && w < W && (XG != kGeoZero || (h & 1) == 0)) {
        // (resampled: 8 pixels of the row are 4 source elements at w/2)
        const int sh = XG == kGeoPlain ? h : h >> 1, sw = XG == kGeoPlain ? w : w >> 1;
        xoff = 2u * (uint32_t)(((n * cin0 + 8 * g) * SH + sh) * SW + sw);
        xoff1 = 2u * (uint32_t)(((n * (Cin - cin0) + 8 * g) * SH + sh) * SW + sw);
        pxo = 4u * (uint32_t)(n * Cin + 8 * g);
      }
      xdst = g * PLW + (img * HR + rr) * RS + 4 + 8 * q;
    }
    if (hrole) {
      const int side = sp & 1;
      int t = sp >> 1;
      const int rr = t % HR;
      t /= HR;
      const int img = t % IMGS;
      const int g = t / IMGS;
      const int n = o.n0 + img, h = o.h0 + rr - 1, w = o.w0 + (side ? TW : -1);
      if (n < N && h >= 0 && h < H && w >= 0 && w < W &&
          (XG != kGeoZero || ((h | w) & 1) == 0)) {
        const int sh = XG == kGeoPlain ? h : h >> 1, sw = XG == kGeoPlain ? w : w >> 1;
        hoff = 2u * (uint32_t)(((n * cin0 + 8 * g) * SH + sh) * SW + sw);
        hoff1 = 2u * (uint32_t)(((n * (Cin - cin0) + 8 * g) * SH + sh) * SW + sw);
        pho = 4u * (uint32_t)(n * Cin + 8 * g);
      }
    }
#pragma unroll
    for (int k = 0; k < WK; ++k) {
      const int it = w_item(k);
      if (it < 0) continue;
      if constexpr (MODE == kFwd) {
        const int co_l = it % BCO, g = it / BCO;  // consecutive lanes: consecutive co
        if (co_l < co_n) woff[k] = 2u * (uint32_t)(((co0 + co_l) * Cin + 8 * g) * 9);
      } else {
        const int g = it / EW, eb = it % EW;
        if (8 * eb < co_n * 9)
          woff[k] = 2u * (uint32_t)(((8 * g) * Cout + co0) * 9 + 8 * eb);
      }
    }
  }
  // bytes between consecutive fills: 16 channels of the source, and of w;
  // bytes between the rows of a backward-data weight item
  const uint32_t xstep = 16u * hw2;
  const uint32_t wstep = MODE == kFwd ? 2u * 16u * 9u : 2u * 16u * 9u * (uint32_t)Cout;
  const uint32_t wrow = 2u * 9u * (uint32_t)Cout;

  // (fills are whole here, so fill f of src1 starts at weight channel
  // 16 (nq0 + f); items outside the image keep kOutside through the select)
  auto load_tiles = [&](auto set_c, int lchunk) __attribute__((always_inline)) {
    constexpr int S = decltype(set_c)::value;
    const int chunk = fbase + lchunk;  // fill index over the whole reduction
    const uint32_t f = (uint32_t)chunk;
    const bool s1 = chunk >= nq0;
    const __amdgpu_buffer_rsrc_t sv = s1 ? sv1 : sv0;
    const uint32_t fx = (uint32_t)(chunk - (s1 ? nq0 : 0)) * xstep;
    if (xrole) {
      const uint32_t b = (s1 ? xoff1 : xoff) + fx;
      if constexpr (XG == kGeoPlain) {
#pragma unroll
        for (int i = 0; i < 8; ++i) st[S][i] = buffer_load16(sv, b + (uint32_t)i * hw2);
      } else {
        // four source elements per channel row, spread when written
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint64_t u = buffer_load8(sv, b + (uint32_t)i * hw2);
          st[S][i].x = (uint32_t)u;
          st[S][i].y = (uint32_t)(u >> 32);
        }
      }
      if constexpr (SPRO) {
        // (one source tensor: s1 is false) 16 channels per fill
        const uint32_t pb = pxo + 64u * f;
        psx[S][0] = __builtin_bit_cast(f32x4, buffer_load16(psv, pb));
        psx[S][1] = __builtin_bit_cast(f32x4, buffer_load16(psv, pb + 16u));
        psx[S][2] = __builtin_bit_cast(f32x4, buffer_load16(ptv, pb));
        psx[S][3] = __builtin_bit_cast(f32x4, buffer_load16(ptv, pb + 16u));
      }
      if constexpr (ZG) {
        // (one source tensor: s1 is false)
        const uint32_t zb = (xoff == kOutside ? kOutside : 2u * xoff) + 2u * fx;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          zx[S][2 * i] = __builtin_bit_cast(f32x4, buffer_load16(zv, zb + 2u * (uint32_t)i * hw2));
          zx[S][2 * i + 1] =
              __builtin_bit_cast(f32x4, buffer_load16(zv, zb + 2u * (uint32_t)i * hw2 + 16u));
        }
      }
    }
    if (hrole && halo_loads) {
      const uint32_t b = (s1 ? hoff1 : hoff) + fx;
#pragma unroll
      for (int i = 0; i < 8; ++i) hv[S][i] = buffer_load2(sv, b + (uint32_t)i * hw2);
      if constexpr (SPRO) {
        const uint32_t pb = pho + 64u * f;
        psh[S][0] = __builtin_bit_cast(f32x4, buffer_load16(psv, pb));
        psh[S][1] = __builtin_bit_cast(f32x4, buffer_load16(psv, pb + 16u));
        psh[S][2] = __builtin_bit_cast(f32x4, buffer_load16(ptv, pb));
        psh[S][3] = __builtin_bit_cast(f32x4, buffer_load16(ptv, pb + 16u));
      }
      if constexpr (ZG) {
        const uint32_t zb = (hoff == kOutside ? kOutside : 2u * hoff) + 2u * fx;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          zh[S][i] = __builtin_bit_cast(float, buffer_load4(zv, zb + 2u * (uint32_t)i * hw2));
      }
    }
#pragma unroll
    for (int k = 0; k < WK; ++k) {
      if (w_item(k) < 0) continue;
      if constexpr (MODE == kFwd) {
#pragma unroll
        for (int j = 0; j < 9; ++j)
          st[S][WBASE + k * NSTG + j] = buffer_load16(wv, woff[k] + f * wstep + 16u * (uint32_t)j);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          st[S][WBASE + k * NSTG + i] = buffer_load16(wv, woff[k] + f * wstep + (uint32_t)i * wrow);
      }
    }
  };

  auto store_tiles = [&](auto set_c, int buf) __attribute__((always_inline)) {
    constexpr int S = decltype(set_c)::value;
    if constexpr (ZG) {
      // g = gy * act'(z), rounded to bfloat16, before the transposes
      if (xrole) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const f32x4 za = zx[S][2 * i], zb = zx[S][2 * i + 1];
          st[S][i].x = act_grad_bf16x2<false>(st[S][i].x, za.x, za.y, act);
          st[S][i].y = act_grad_bf16x2<false>(st[S][i].y, za.z, za.w, act);
          st[S][i].z = act_grad_bf16x2<false>(st[S][i].z, zb.x, zb.y, act);
          st[S][i].w = act_grad_bf16x2<false>(st[S][i].w, zb.z, zb.w, act);
        }
      }
      if (hrole && halo_loads) {
#pragma unroll
        for (int i = 0; i < 8; ++i) hv[S][i] = act_grad_bf16<false>(hv[S][i], zh[S][i], act);
      }
    }
    if constexpr (SPRO) {
      // a = SiLU(x * scale + shift), rounded to bfloat16, before the
      // transposes (row i is channel 8g + i; items outside the image load
      // x = scale = shift = 0 and stage SiLU(0) = 0, the zero padding of a)
      if (xrole) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float sc = psx[S][i >> 2][i & 3], sh = psx[S][2 + (i >> 2)][i & 3];
          st[S][i].x = silu_affine_bf16x2<false>(st[S][i].x, sc, sh);
          st[S][i].y = silu_affine_bf16x2<false>(st[S][i].y, sc, sh);
          st[S][i].z = silu_affine_bf16x2<false>(st[S][i].z, sc, sh);
          st[S][i].w = silu_affine_bf16x2<false>(st[S][i].w, sc, sh);
        }
      }
      if (hrole && halo_loads) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          hv[S][i] = silu_affine_bf16<false>(hv[S][i], psh[S][i >> 2][i & 3],
                                             psh[S][2 + (i >> 2)][i & 3]);
      }
    }
    if constexpr (XG != kGeoPlain) {
      if (xrole) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          st[S][i] = XG == kGeoUp ? bf16x4_repeat2(st[S][i].x, st[S][i].y)
                                  : bf16x4_zero_insert(st[S][i].x, st[S][i].y);
      }
    }
    if (xrole) {
      u32x4* d = xs + buf * XW + xdst;
      d[0] = column_word<0>(st[S]);
      d[1] = column_word<1>(st[S]);
      d[2] = column_word<2>(st[S]);
      d[3] = column_word<3>(st[S]);
      d[4] = column_word<4>(st[S]);
      d[5] = column_word<5>(st[S]);
      d[6] = column_word<6>(st[S]);
      d[7] = column_word<7>(st[S]);
    }
    if (hrole) {
      const int side = sp & 1;
      const int t = sp >> 1;  // (g * IMGS + img) * HR + rr
      const int g = t / (IMGS * HR);
      const u32x4 h = {hv[S][0] | (hv[S][1] << 16), hv[S][2] | (hv[S][3] << 16),
                       hv[S][4] | (hv[S][5] << 16), hv[S][6] | (hv[S][7] << 16)};
      xs[buf * XW + g * PLW + (t % (IMGS * HR)) * RS + 4 + (side ? TW : -1)] = h;
    }
    u32x4* wb = wa + buf * WW;
#pragma unroll
    for (int k = 0; k < WK; ++k) {
      const int it = w_item(k);
      if (it < 0) continue;
      if constexpr (MODE == kFwd) {
        const int co_l = it % BCO, g = it / BCO;
        const uint32_t* d = reinterpret_cast<const uint32_t*>(&st[S][WBASE + k * NSTG]);
        wb[(0 * 2 + g) * BCO + co_l] = tap_word<0>(d);
        wb[(1 * 2 + g) * BCO + co_l] = tap_word<1>(d);
        wb[(2 * 2 + g) * BCO + co_l] = tap_word<2>(d);
        wb[(3 * 2 + g) * BCO + co_l] = tap_word<3>(d);
        wb[(4 * 2 + g) * BCO + co_l] = tap_word<4>(d);
        wb[(5 * 2 + g) * BCO + co_l] = tap_word<5>(d);
        wb[(6 * 2 + g) * BCO + co_l] = tap_word<6>(d);
        wb[(7 * 2 + g) * BCO + co_l] = tap_word<7>(d);
        wb[(8 * 2 + g) * BCO + co_l] = tap_word<8>(d);
      } else {
        // column i: element e = 8 eb + i (= co_l * 9 + tap of the stored,
        // unrotated weight) of rows 8g .. 8g + 7
        const int g = it / EW, eb = it % EW;
        auto put = [&](int i, u32x4 v) {
          const int e = 8 * eb + i;
          wb[((8 - e % 9) * 2 + g) * BCO + e / 9] = v;
        };
        put(0, column_word<0>(&st[S][WBASE + k * NSTG]));
        put(1, column_word<1>(&st[S][WBASE + k * NSTG]));
        put(2, column_word<2>(&st[S][WBASE + k * NSTG]));
        put(3, column_word<3>(&st[S][WBASE + k * NSTG]));
        put(4, column_word<4>(&st[S][WBASE + k * NSTG]));
        put(5, column_word<5>(&st[S][WBASE + k * NSTG]));
        put(6, column_word<6>(&st[S][WBASE + k * NSTG]));
        put(7, column_word<7>(&st[S][WBASE + k * NSTG]));
      }
    }
  };

  // Scalar path (ragged shapes): 16-bit loads straight into LDS buffer buf,
  // by the staging threads.
  auto fill_scalar = [&](int lchunk, int buf) __attribute__((always_inline)) {
    if (sp < 0) return;
    const int chunk = fbase + lchunk;  // fill index over the whole reduction
    const bool s1 = chunk >= nq0;
    const int cl0 = (chunk - (s1 ? nq0 : 0)) * CB;  // first channel within its tensor
    const int cs = s1 ? Cin - cin0 : cin0;            // channels of that tensor
    const int cg0 = (s1 ? cin0 : 0) + cl0;            // first channel in the weight
    const int cn = min(CB, cs - cl0);                 // valid channels of the fill
    const uint16_t* sx = s1 ? src1 : src;
    uint16_t* xh = reinterpret_cast<uint16_t*>(xs + buf * XW);
    uint16_t* wh = reinterpret_cast<uint16_t*>(wa + buf * WW);
    constexpr int XS = CB * IMGS * HR * (TW + 2);
#pragma unroll 4
    for (int k = 0; k < (XS + NP - 1) / NP; ++k) {
      const int it = sp + NP * k;
      if (XS % NP == 0 || it < XS) {
        const int cc = it % (TW + 2) - 1;
        const int t = it / (TW + 2);  // (ch * IMGS + img) * HR + rr
        const int rr = t % HR;
        const int img = (t / HR) % IMGS;
        const int ch = t / (HR * IMGS);
        const int n = o.n0 + img, h = o.h0 + rr - 1, w = o.w0 + cc;
        uint16_t v = 0;
        // (an upsampled or zero-inserted source is an H/2 x W/2 tensor read
        // at (h / 2, w / 2); zero-inserted: only at even (h, w))
        const bool half = geo == kGeoUp || geo == kGeoZero;
        const int sh = half ? h >> 1 : h, sw = half ? w >> 1 : w;
        const int sW = half ? W >> 1 : W;
        const long sHW = half ? (long)(H >> 1) * sW : HW;
        if (n < N && ch < cn && h >= 0 && h < H && w >= 0 && w < W &&
            (geo != kGeoZero || ((h | w) & 1) == 0)) {
          const long e = ((long)n * cs + cl0 + ch) * sHW + (long)sh * sW + sw;
          v = sx[e];
          if constexpr (ZG) v = (uint16_t)act_grad_bf16<false>(v, zsrc[e], act);
          if constexpr (SPRO) {
            const long pc = (long)n * Cin + cl0 + ch;  // (one source tensor)
            v = (uint16_t)silu_affine_bf16<false>(v, pscale[pc], pshift[pc]);
          }
        }
        xh[((ch >> 3) * PLW + (img * HR + rr) * RS + 4 + cc) * 8 + (ch & 7)] = v;
      }
    }
    constexpr int WSI = CB * 9 * BCO;
#pragma unroll 4
    for (int k = 0; k < (WSI + NP - 1) / NP; ++k) {
      const int it = sp + NP * k;
      if (WSI % NP != 0 && it >= WSI) continue;
      int ci_l, co_l, tap;
      uint16_t v = 0;
      if constexpr (MODE == kFwd) {
        co_l = it / (CB * 9);
        const int e = it % (CB * 9);
        ci_l = e / 9;
        tap = e % 9;
        if (co_l < co_n && ci_l < cn) v = wt[((long)(co0 + co_l) * Cin + cg0 + ci_l) * 9 + tap];
      } else {
        ci_l = it / (BCO * 9);
        const int e = it % (BCO * 9);
        co_l = e / 9;
        const int tg = e % 9;
        tap = 8 - tg;
        if (co_l < co_n && ci_l < cn) v = wt[((long)(cg0 + ci_l) * Cout + co0 + co_l) * 9 + tg];
      }
      wh[((tap * 2 + (ci_l >> 3)) * BCO + co_l) * 8 + (ci_l & 7)] = v;
    }
  };
  // Write fill chunk + 1 (held in set_c) to LDS and load fill
  // chunk + 1 + NSET into the same set.
  auto stage_next = [&](auto set_c, int chunk) __attribute__((always_inline)) {
    if constexpr (VEC) {
      if (chunk + 1 < nchunks) store_tiles(set_c, (chunk + 1) & 1);
      if (chunk + 1 + NSET < nchunks) load_tiles(set_c, chunk + 1 + NSET);
    } else {
      if (chunk + 1 < nchunks) fill_scalar(chunk + 1, (chunk + 1) & 1);
    }
  };

  // ---- prologue: fill 0 in buffer 0, the next NSET fills in registers ----
  if constexpr (MODE == kFwd) {
    for (int i = tid; i < BCO; i += NT)
      bias_s[i] = (bias != nullptr && i < co_n && fbase == 0) ? bias[co0 + i] : 0.f;
  }
  if constexpr (VEC) {
    load_tiles(Set0{}, 0);
    store_tiles(Set0{}, 0);
    if (nchunks > 1) load_tiles(SetOdd{}, 1);
    if (NSET == 2 && nchunks > 2) load_tiles(Set0{}, 2);
  } else {
    fill_scalar(0, 0);
  }
  __syncthreads();

  if constexpr (WSPEC) {
    if (wave >= NC) {
      // Staging waves: between the barrier of fill i - 1 and that of fill i,
      // write fill i + 1 into buffer (i + 1) & 1 (last read by the compute
      // waves before the barrier of fill i - 1) and load fill i + 2.  One
      // barrier per fill, matching the compute waves.
      for (int chunk = 0; chunk + 1 < nchunks; chunk += 2) {
        stage_next(SetOdd{}, chunk);
        __syncthreads();
        if (chunk + 2 < nchunks) {
          stage_next(Set0{}, chunk + 1);
          __syncthreads();
        }
      }
      return;
    }
  }

  // ---- compute ----
  const int wco = wave % WCO, wpx = wave / WCO;
  int boff[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int p = wpx * (BM / WPX) + j * 32 + l32;
    const int img = p / (TH * TW), row = (p / TW) % TH, col = p % TW;
    boff[j] = hi * PLW + (img * HR + row) * RS + 4 + col - 1;
  }
  const int aoff = hi * BCO + wco * (BCO / WCO) + l32;

  // Forward: the accumulators start at the tile's biases (zero without
  // bias), so the epilogue is stores only.
  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    f32x16 init;
#pragma unroll
    for (int v = 0; v < 16; ++v)
      init[v] = MODE == kFwd ? bias_s[wco * (BCO / WCO) + i * 32 + acc_row(v, hi)] : 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = init;
  }

  // Single-block wave tiles (one MFMA per tap) would wait out an LDS read
  // round trip at every tap, so they hold all nine taps of a fill in
  // registers: slot t is refilled with tap t of the next fill as soon as this
  // fill's MFMAs of tap t are issued (from the barrier step on), about a fill
  // ahead of its use.  Larger wave tiles read one tap ahead.
  constexpr bool DEEP = MI * NJ == 1;
  if constexpr (DEEP) {
    // The barrier sits at step kBar: the next fill has been written by then
    // (by the staging waves, or here after tap 0), and every read of the
    // buffer it replaces was issued during the previous fill.
    constexpr int kBar = 2;
    u32x4 ad[9][MI], bd[9][NJ];
    auto read_slot = [&](int cbuf, int t) {
      const u32x4* xb = xs + cbuf * XW;
      const u32x4* wb = wa + cbuf * WW;
      const int r = t / 3, s = t % 3;
#pragma unroll
      for (int i = 0; i < MI; ++i) ad[t][i] = wb[aoff + t * 2 * BCO + i * 32];
#pragma unroll
      for (int j = 0; j < NJ; ++j) bd[t][j] = xb[boff[j] + r * RS + s];
    };
#pragma unroll
    for (int t = 0; t < 9; ++t) read_slot(0, t);
    auto run_fill = [&](auto set_c, int chunk) __attribute__((always_inline)) {
      const int cur = chunk & 1;
      const bool next = chunk + 1 < nchunks;
#pragma unroll
      for (int t = 0; t < 9; ++t) {
        if (t == kBar && next) __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[i][j] = mfma_32x32x16_bf16(ad[t][i], bd[t][j], acc[i][j]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!WSPEC) {
          if (t == 0) stage_next(set_c, chunk);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (next && t >= kBar) {
          if (t == kBar) {
#pragma unroll
            for (int u = 0; u <= kBar; ++u) read_slot(cur ^ 1, u);
          } else {
            read_slot(cur ^ 1, t);
          }
        }
      }
    };
    for (int chunk = 0; chunk < nchunks; chunk += 2) {
      run_fill(SetOdd{}, chunk);
      if (chunk + 1 < nchunks) run_fill(Set0{}, chunk + 1);
    }
  } else {
    // Operands of one tap: a = weights (MI words), b = pixels (NJ words); tap
    // t in register set t & 1.
    u32x4 a[2][MI], b[2][NJ];
    auto read_tap = [&](int cbuf, int rb, int t) {
      const u32x4* xb = xs + cbuf * XW;
      const u32x4* wb = wa + cbuf * WW;
      const int r = t / 3, s = t % 3;
#pragma unroll
      for (int i = 0; i < MI; ++i) a[rb][i] = wb[aoff + t * 2 * BCO + i * 32];
#pragma unroll
      for (int j = 0; j < NJ; ++j) b[rb][j] = xb[boff[j] + r * RS + s];
    };
    // Tap t's operands are read while tap t-1's MFMAs run.  The barrier sits
    // before tap 8's MFMAs: by then the next fill is written (by the staging
    // waves, or here after tap 0) and every lane has read its last operands of
    // this one, so tap 0 of the next fill is read while tap 8 runs.
    // One fill; set_c is the staging register set that holds fill chunk + 1.
    auto run_fill = [&](auto set_c, int chunk) __attribute__((always_inline)) {
      const int cur = chunk & 1;
      const bool next = chunk + 1 < nchunks;
#pragma unroll
      for (int t = 0; t < 9; ++t) {
        const int rb = t & 1;
        if (t + 1 < 9) {
          read_tap(cur, rb ^ 1, t + 1);
        } else if (next) {
          __syncthreads();
          read_tap(cur ^ 1, rb ^ 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[i][j] = mfma_32x32x16_bf16(a[rb][i], b[rb][j], acc[i][j]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!WSPEC) {
          // written after tap 0: the other buffer was last read before the
          // previous fill's barrier
          if (t == 0) stage_next(set_c, chunk);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // tap 0 of the next fill was read into the second operand set
#pragma unroll
      for (int i = 0; i < MI; ++i) a[0][i] = a[1][i];
#pragma unroll
      for (int j = 0; j < NJ; ++j) b[0][j] = b[1][j];
    };
    read_tap(0, 0, 0);
    for (int chunk = 0; chunk < nchunks; chunk += 2) {
      run_fill(SetOdd{}, chunk);
      if (chunk + 1 < nchunks) run_fill(Set0{}, chunk + 1);
    }
  }

  // ---------------- epilogue: NCHW stores ----------------
  // Forward with a fused activation: y = act(z), z = the accumulator (bias
  // included), also written to zout (float32) when it is given.
  // (zout, forward only, has the shape of dst; the output is then one tensor.)
  // outb: dst (and dst1) hold bfloat16, rounded to nearest even.
  // A split reduction writes this slice's partial sums (bias in slice 0),
  // float32, to its slot of the workspace (one tensor of dst's shape per
  // slice); the reduce kernel adds the slices and applies the rest.
  const int cw = col0 + wco * (BCO / WCO);  // first output channel of this wave
  if constexpr (MODE == kBwdData && PRO) {
    // du = acc * SiLU'(u), u = x * scale + shift at the output position (px
    // has dx's shape, one tensor).  Scale and shift of the tile's channels
    // and images go through LDS (the operand tiles are no longer read);
    // then, four elements at a time, x's bfloat16 value, du and its store
    // (elements outside the tensor read zero and store nothing).
    static_assert(2 * IMGS * BCO <= 4 * 2 * XW, "scale/shift fit");
    float* ps_s = reinterpret_cast<float*>(xs);
    float* pt_s = ps_s + IMGS * BCO;
    __syncthreads();
    for (int e = tid; e < IMGS * BCO; e += NT) {
      const int n = o.n0 + e / BCO, co = col0 + e % BCO;
      const bool ok = n < N && co < Cout;
      ps_s[e] = ok ? pscale[(long)n * Cout + co] : 0.f;
      pt_s[e] = ok ? pshift[(long)n * Cout + co] : 0.f;
    }
    __syncthreads();
    if (wave >= NC) return;
    const uint32_t es = outb ? 2u : 4u;
    const __amdgpu_buffer_rsrc_t xv_b =
        buffer_view(px, 2u * (uint32_t)N * (uint32_t)Cout * (uint32_t)HW);
    const __amdgpu_buffer_rsrc_t dv_b = buffer_view(dst, dst_bytes);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int p = wpx * (BM / WPX) + j * 32 + l32;
      const int img = p / (TH * TW), row = (p / TW) % TH, col = p % TW;
      const int n = o.n0 + img, h = o.h0 + row, w = o.w0 + col;
      const bool in = n < N && h < H && w < W;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int v0 = 0; v0 < 16; v0 += 4) {
          float xe[4];
          uint32_t so[4];  // store offsets (kOutside: no store)
#pragma unroll
          for (int v = v0; v < v0 + 4; ++v) {
            const int co = cw + i * 32 + acc_row(v, hi);
            const bool ok = in && co < Cout;
            const uint32_t e = ((uint32_t)n * Cout + co) * (uint32_t)HW + (uint32_t)(h * W + w);
            so[v - v0] = ok ? es * e : kOutside;
            xe[v - v0] =
                __builtin_bit_cast(float, buffer_load2(xv_b, ok ? 2u * e : kOutside) << 16);
          }
#pragma unroll
          for (int v = v0; v < v0 + 4; ++v) {
            const int e = img * BCO + (cw - col0) + i * 32 + acc_row(v, hi);
            const float du =
                acc[i][j][v] * act_slope(kActSilu, __builtin_fmaf(xe[v - v0], ps_s[e], pt_s[e]));
            if (outb)
              buffer_store2(dv_b, so[v - v0], 0u, bf16_rne(du));
            else
              buffer_store4(dv_b, so[v - v0], 0u, du);
          }
        }
      }
    }
    return;
  }
  if (geo == kGeoSub) {
    // stride-2 forward: the stride-1 sums at the even pixels are the
    // strided convolution's outputs, stored to the H/2 x W/2 output (one
    // tensor, float32, no split, no activation)
    const int OH = H >> 1, OW = W >> 1;
    const long OHW = (long)OH * OW;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int p = wpx * (BM / WPX) + j * 32 + l32;
      const int img = p / (TH * TW), row = (p / TW) % TH, col = p % TW;
      const int n = o.n0 + img, h = o.h0 + row, w = o.w0 + col;
      if (n >= N || h >= H || w >= W || ((h | w) & 1)) continue;
      const long base = (long)n * ocs * OHW + (long)(h >> 1) * OW + (w >> 1);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int co = cw + i * 32 + acc_row(v, hi);
          if (co < ocs) dst[base + (long)co * OHW] = acc[i][j][v];
        }
    }
    return;
  }
  const bool plain = part != nullptr || MODE != kFwd || (act == kActNone && zout == nullptr);
  const uint32_t slot_bytes = (uint32_t)N * (uint32_t)Cout * (uint32_t)HW * 4u;
  float* const od = part ? part + (size_t)blockIdx.z * ((size_t)slot_bytes / 4) : oseg ? dst1 : dst;
  const uint32_t od_bytes = part ? slot_bytes : oseg ? dst1_bytes : dst_bytes;
  if (part) outb = 0;
  if (od_bytes != 0 && co_n == BCO) {
    // Whole channel tile in range: one buffer store per accumulator element,
    // the lane's byte offset computed once per pixel column j and the channel
    // step a uniform (scalar) offset.  Pixels outside the image get an offset
    // past the view and the hardware drops their stores.
    const __amdgpu_buffer_rsrc_t dv = buffer_view(od, od_bytes);
    const __amdgpu_buffer_rsrc_t zov =
        buffer_view(zout, plain ? 0u : (outb ? 2u : 1u) * od_bytes);
    const uint32_t es = outb ? 2u : 4u;  // bytes per output element
    // bfloat16 with an even width: lanes 2m and 2m + 1 hold horizontally
    // adjacent pixels, so for each pair of rows (v, v + 1) the two lanes
    // swap one value and lane 2m stores row v's pixel pair, lane 2m + 1 row
    // v + 1's, as one 4-byte store each (half the store instructions; the
    // epilogue is bound by their count, not by bytes).
    const bool pack = outb && (W & 1) == 0;
    const bool odd = l32 & 1;
    if (plain && !outb) {
      // float32 without an activation (also the split slices): a separate,
      // branch-free loop nest.  Inside the general one below the run-time
      // tests of plain / outb stay per element, with a wait on the stores
      // at every merge (measured on 16x16 images, 512 channels: that
      // epilogue took 15 us of a 77 us forward).
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int p = wpx * (BM / WPX) + j * 32 + l32;
        const int img = p / (TH * TW), row = (p / TW) % TH, col = p % TW;
        const int n = o.n0 + img, h = o.h0 + row, w = o.w0 + col;
        const bool in = n < N && h < H && w < W;
        const uint32_t e =
            ((uint32_t)n * ocs + cw + 4 * hi) * (uint32_t)HW + (uint32_t)(h * W + w);
        const uint32_t off = in ? e * 4u : kOutside;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            buffer_store4(dv, off, (uint32_t)(i * 32 + 8 * (v >> 2) + (v & 3)) * (uint32_t)HW * 4u,
                          acc[i][j][v]);
      }
      return;
    }
    if (plain && pack) {
      // bfloat16 pairs without an activation: the same, with the lane-pair
      // exchange below (as a separate loop nest for the same reason)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int p = wpx * (BM / WPX) + j * 32 + l32;
        const int img = p / (TH * TW), row = (p / TW) % TH, col = p % TW;
        const int n = o.n0 + img, h = o.h0 + row, w = o.w0 + col;
        const bool in = n < N && h < H && w < W;
        const uint32_t e =
            ((uint32_t)n * ocs + cw + 4 * hi) * (uint32_t)HW + (uint32_t)(h * W + w);
        const uint32_t poff =
            in ? (e - (odd ? 1u : 0u) + (odd ? (uint32_t)HW : 0u)) * 2u : kOutside;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int v = 0; v < 16; v += 2) {
            const uint32_t rowoff = (uint32_t)(i * 32 + 8 * (v >> 2) + (v & 3)) * (uint32_t)HW;
            const float a0 = acc[i][j][v], a1 = acc[i][j][v + 1];
            const float got = __builtin_bit_cast(
                float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, odd ? a0 : a1), 0xB1,
                                                0xF, 0xF, false));
            const float lo = odd ? got : a0, hi2 = odd ? a1 : got;
            buffer_store4(dv, poff, rowoff * 2u,
                          __builtin_bit_cast(float, bf16_rne(lo) | (bf16_rne(hi2) << 16)));
          }
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int p = wpx * (BM / WPX) + j * 32 + l32;
      const int img = p / (TH * TW), row = (p / TW) % TH, col = p % TW;
      const int n = o.n0 + img, h = o.h0 + row, w = o.w0 + col;
      const bool in = n < N && h < H && w < W;
      const uint32_t e = ((uint32_t)n * ocs + cw + 4 * hi) * (uint32_t)HW + (uint32_t)(h * W + w);
      const uint32_t off = in ? e * es : kOutside, zoff = in ? e * 4u : kOutside;
      if (pack) {
        // pair start (the even lane's pixel); the odd lane's row is one
        // plane further
        const uint32_t poff = in ? (e - (odd ? 1u : 0u) + (odd ? (uint32_t)HW : 0u)) * 2u
                                 : kOutside;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int v = 0; v < 16; v += 2) {
            const uint32_t rowoff = (uint32_t)(i * 32 + 8 * (v >> 2) + (v & 3)) * (uint32_t)HW;
            float a0 = acc[i][j][v], a1 = acc[i][j][v + 1];
            if (!plain) {
              if (zout) {
                buffer_store4(zov, zoff, rowoff * 4u, a0);
                buffer_store4(zov, zoff, (rowoff + (uint32_t)HW) * 4u, a1);
              }
              a0 = act_value(act, a0);
              a1 = act_value(act, a1);
            }
            // quad_perm [1, 0, 3, 2]: each lane reads its neighbour 2m <-> 2m + 1
            const float got = __builtin_bit_cast(
                float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, odd ? a0 : a1), 0xB1,
                                                0xF, 0xF, false));
            const float lo = odd ? got : a0, hi2 = odd ? a1 : got;
            buffer_store4(dv, poff, rowoff * 2u,
                          __builtin_bit_cast(float, bf16_rne(lo) | (bf16_rne(hi2) << 16)));
          }
        continue;
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const uint32_t rowoff = (uint32_t)(i * 32 + 8 * (v >> 2) + (v & 3)) * (uint32_t)HW;
          float val = acc[i][j][v];
          if (!plain) {
            if (zout) buffer_store4(zov, zoff, rowoff * 4u, val);
            val = act_value(act, val);
          }
          if (outb)
            buffer_store2(dv, off, rowoff * 2u, bf16_rne(val));
          else
            buffer_store4(dv, off, rowoff * 4u, val);
        }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int p = wpx * (BM / WPX) + j * 32 + l32;
    const int img = p / (TH * TW), row = (p / TW) % TH, col = p % TW;
    const int n = o.n0 + img, h = o.h0 + row, w = o.w0 + col;
    if (n >= N || h >= H || w >= W) continue;
    const long base = (long)n * ocs * HW + (long)h * W + w;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int co = cw + i * 32 + acc_row(v, hi);
        if (co < ocs) {
          const long ei = base + (long)co * HW;
          float val = acc[i][j][v];
          if (!plain) {
            if (zout) zout[ei] = val;
            val = act_value(act, val);
          }
          if (outb)
            reinterpret_cast<uint16_t*>(od)[ei] = (uint16_t)bf16_rne(val);
          else
            od[ei] = val;
        }
      }
    }
  }
}

// Sum of the S partial-output slots of a split reduction, in slice order,
// then the activation and the store (float32, or bfloat16 when outb; z, the
// sum before the activation, to zout when given).  Four elements per thread.
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part,
                                                           int S, long slot,
                                                           float* __restrict__ dst, int outb,
                                                           int act, float* __restrict__ zout) {
  const long e0 = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e0 >= slot) return;
  if (e0 + 4 <= slot && slot % 4 == 0) {
    f32x4 v = *reinterpret_cast<const f32x4*>(part + e0);
    for (int s = 1; s < S; ++s) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(part + (long)s * slot + e0);
      v.x += q.x;
      v.y += q.y;
      v.z += q.z;
      v.w += q.w;
    }
    if (zout) *reinterpret_cast<f32x4*>(zout + e0) = v;
    v.x = act_value(act, v.x);
    v.y = act_value(act, v.y);
    v.z = act_value(act, v.z);
    v.w = act_value(act, v.w);
    if (outb) {
      uint32_t* d = reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(dst) + e0);
      d[0] = bf16_rne(v.x) | (bf16_rne(v.y) << 16);
      d[1] = bf16_rne(v.z) | (bf16_rne(v.w) << 16);
    } else {
      *reinterpret_cast<f32x4*>(dst + e0) = v;
    }
    return;
  }
  for (long e = e0; e < e0 + 4 && e < slot; ++e) {
    float v = part[e];
    for (int s = 1; s < S; ++s) v += part[(long)s * slot + e];
    if (zout) zout[e] = v;
    v = act_value(act, v);
    if (outb)
      reinterpret_cast<uint16_t*>(dst)[e] = (uint16_t)bf16_rne(v);
    else
      dst[e] = v;
  }
}

// dx = the 2 x 2 block sums of du (see launch.hpp), ((00 + 01) + 10) + 11.
__global__ __launch_bounds__(256) void block_sum2_kernel(const float* __restrict__ du,
                                                         float* __restrict__ dx, long total,
                                                         int H, int W) {
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  const long plane = e / ((long)H * W);
  const int r = (int)(e % ((long)H * W));
  const int i = r / W, j = r % W;
  const float* d = du + plane * 4L * H * W + (long)(2 * i) * (2 * W) + 2 * j;
  dx[e] = ((d[0] + d[1]) + d[2 * W]) + d[2 * W + 1];
}

void launch_block_sum2(const float* du, float* dx, long planes, int H, int W,
                       hipStream_t stream) {
  const long total = planes * H * W;
  dim3 g((unsigned)((total + 255) / 256)), b(256);
  hipLaunchKernelGGL(block_sum2_kernel, g, b, 0, stream, du, dx, total, H, W);
}

void launch_split_reduce(const float* part, int S, long slot, float* dst, hipStream_t stream) {
  dim3 rg((unsigned)((slot + 1023) / 1024)), rb(256);
  hipLaunchKernelGGL(split_reduce_kernel, rg, rb, 0, stream, part, S, slot, dst, 0, (int)kActNone,
                     (float*)nullptr);
}

template <int MODE, int TW, int TH, int IMGS, int BCO, int WCO, int NW, bool ZG, bool PRO>
static void launch_bf16_cfg(const Plan& pl, bool vec, Split<const uint16_t> src,
                            const uint16_t* wt, const float* bias, Split<float> dst, int N,
                            int Cin, int Cout, int H, int W, const ActArgs& a, bool out_bf16,
                            float* ws, hipStream_t stream) {
  if constexpr ((ZG || PRO) && NW != 4) {
    return;  // not instantiated: launch_fwd_bf16 refuses these plans
  } else {
  // split reduction: partial sums into ws, then split_reduce_kernel
  float* const part = pl.split > 1 ? ws : nullptr;
  dim3 grid(pl.grid_x, pl.grid_y, part ? pl.split : 1), block(64 * NW, 1, 1);
  // resampling geometry: the source read at half coordinates (kGeoUp,
  // kGeoZero) or the outputs kept at the even pixels (kGeoSub)
  const int geo = MODE == kFwd ? (a.up2 ? kGeoUp : a.s2 ? kGeoSub : kGeoPlain)
                               : (a.s2 ? kGeoZero : kGeoPlain);
  // Buffer-view stores need each output tensor below 2 GiB (32-bit byte
  // offsets), and a float32 z beside bfloat16 outputs twice that; otherwise
  // the plain-store path runs.
  const long hw = (long)H * W;
  const long es = out_bf16 ? 2 : 4, zf = a.zout ? 4 / es : 1;
  const long ob0 = (long)N * dst.c0 * hw * es, ob1 = (long)N * (Cout - dst.c0) * hw * es;
  const bool small = ob0 * zf < 2147483648L && ob1 * zf < 2147483648L;
  const uint32_t db0 = small ? (uint32_t)ob0 : 0u, db1 = small ? (uint32_t)ob1 : 0u;
  constexpr int XG = MODE == kFwd ? kGeoUp : kGeoZero;  // this pass's resampled source
  if constexpr (!ZG && !PRO) {
    if (vec && geo == XG) {
      // one source tensor of N x Cin x H/2 x W/2
      hipLaunchKernelGGL((fwd_bf16_kernel<MODE, TW, TH, IMGS, BCO, WCO, NW, true, false, false, XG>),
                         grid, block, 0, stream, src.p0, src.p1, src.c0, wt, bias, dst.p0, dst.p1,
                         dst.c0, N, Cin, Cout, H, W, pl.tiles_w, pl.tiles_h,
                         (uint32_t)(N * Cin * (hw / 4) * 2), 0u, (uint32_t)((long)Cin * Cout * 9 * 2),
                         db0, db1, a.act, a.zout, out_bf16 ? 1 : 0, pl.chunks_per_split, part,
                         a.zsrc, a.pscale, a.pshift, (const uint16_t*)a.px, (int)kGeoPlain);
      return;
    }
  }
  if (vec)
    hipLaunchKernelGGL((fwd_bf16_kernel<MODE, TW, TH, IMGS, BCO, WCO, NW, true, ZG, PRO>), grid,
                       block, 0, stream, src.p0, src.p1, src.c0, wt, bias, dst.p0, dst.p1,
                       dst.c0, N, Cin, Cout, H, W, pl.tiles_w, pl.tiles_h,
                       (uint32_t)(N * src.c0 * hw * 2), (uint32_t)(N * (Cin - src.c0) * hw * 2),
                       (uint32_t)((long)Cin * Cout * 9 * 2), db0, db1, a.act, a.zout,
                       out_bf16 ? 1 : 0, pl.chunks_per_split, part, a.zsrc, a.pscale, a.pshift,
                       (const uint16_t*)a.px, geo);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<MODE, TW, TH, IMGS, BCO, WCO, NW, false, ZG, PRO>),
                       grid, block, 0, stream, src.p0, src.p1, src.c0, wt, bias, dst.p0, dst.p1,
                       dst.c0, N, Cin, Cout, H, W, pl.tiles_w, pl.tiles_h, 0u, 0u, 0u, db0, db1,
                       a.act, a.zout, out_bf16 ? 1 : 0, pl.chunks_per_split, part, a.zsrc,
                       a.pscale, a.pshift, (const uint16_t*)a.px, geo);
  if (part) {
    const long slot = (long)N * Cout * hw;
    dim3 rg((unsigned)((slot + 1023) / 1024)), rb(256);
    hipLaunchKernelGGL(split_reduce_kernel, rg, rb, 0, stream, part, pl.split, slot, dst.p0,
                       out_bf16 ? 1 : 0, a.act, a.zout);
  }
  }
}

bool launch_fwd_bf16(const Plan& pl, bool vec, Split<const uint16_t> src, const uint16_t* wt,
                     const float* bias, Split<float> dst, int N, int Cin, int Cout, int H, int W,
                     const ActArgs& a, bool out_bf16, float* ws, hipStream_t stream) {
  if (pl.chunk != 16) return false;
  // a split reduction needs its workspace and one output tensor
  if (pl.split > 1 && (ws == nullptr || dst.c0 != Cout)) return false;
  // A fused activation gradient (a.zsrc, backward-data) or the input
  // prologue (a.pscale) needs one source / output tensor, no split and a
  // four-wave tile (the eight-wave tile's staging waves cannot also hold
  // their float32 operands; the planner keeps to the four-wave tiles for
  // them).  The forward's prologue and a fused gradient do not combine.
  const bool pro = a.pscale != nullptr;
  if ((a.zsrc != nullptr || pro) &&
      (src.c0 != Cin || dst.c0 != Cout || pl.split > 1 || pl.threads != 256))
    return false;
  if (a.zsrc != nullptr && (pl.pass == kFwd || pro)) return false;
  if (pro && pl.pass == kBwdData && a.px == nullptr) return false;
  // Resampling (the stride-1 kernels over the full-resolution grid): one
  // source and one output tensor, float32 output, no split or fusion;
  // backward-data of the upsampling call is composed by the caller (its
  // full-resolution result summed over 2 x 2 blocks).
  if ((a.up2 || a.s2) &&
      (src.c0 != Cin || dst.c0 != Cout || pl.split > 1 || out_bf16 || pro ||
       a.zsrc != nullptr || a.zout != nullptr || a.act != kActNone ||
       (pl.pass == kBwdData && a.up2) || (H & 1) || (W & 1)))
    return false;
#define CONV3X3_X(TW_, TH_, IMGS_, CO_, WCO_, NW_)                                              \
  if (pl.tw == TW_ && pl.th == TH_ && pl.imgs == IMGS_ && pl.tile_co == CO_ &&                  \
      pl.wave_co == WCO_ && pl.threads == 64 * NW_) {                                           \
    if (pl.pass == kFwd && !pro)                                                                \
      launch_bf16_cfg<kFwd, TW_, TH_, IMGS_, CO_, WCO_, NW_, false, false>(                     \
          pl, vec, src, wt, bias, dst, N, Cin, Cout, H, W, a, out_bf16, ws, stream);            \
    else if (pl.pass == kFwd)                                                                   \
      launch_bf16_cfg<kFwd, TW_, TH_, IMGS_, CO_, WCO_, NW_, false, true>(                      \
          pl, vec, src, wt, bias, dst, N, Cin, Cout, H, W, a, out_bf16, ws, stream);            \
    else if (a.zsrc != nullptr)                                                                 \
      launch_bf16_cfg<kBwdData, TW_, TH_, IMGS_, CO_, WCO_, NW_, true, false>(                  \
          pl, vec, src, wt, nullptr, dst, N, Cin, Cout, H, W, a, out_bf16, ws, stream);         \
    else if (pro)                                                                               \
      launch_bf16_cfg<kBwdData, TW_, TH_, IMGS_, CO_, WCO_, NW_, false, true>(                  \
          pl, vec, src, wt, nullptr, dst, N, Cin, Cout, H, W, a, out_bf16, ws, stream);         \
    else                                                                                        \
      launch_bf16_cfg<kBwdData, TW_, TH_, IMGS_, CO_, WCO_, NW_, false, false>(                 \
          pl, vec, src, wt, nullptr, dst, N, Cin, Cout, H, W, a, out_bf16, ws, stream);         \
    return true;                                                                                \
  }
  CONV3X3_FWD_BF16_CONFIGS(CONV3X3_X)
#undef CONV3X3_X
  return false;
}

}  // namespace conv3x3
