// Forward (+bias) and backward-data 3x3 convolution, float32, gfx950.
//
// One implicit-GEMM kernel serves both passes (see the C header for the
// formulas):
//   forward       : out[n,co,p] = bias[co] + sum_{ci,tap} src[n,ci,p+tap] w[co,ci,tap]
//                   with src = x (Cin = C), co over K;
//   backward-data : the same with src = g (Cin = K), co over C and the weight
//                   read as w[ci, co, 8 - tap] -- the transpose and 180-degree
//                   rotation happen in the LDS staging index, never in memory.
//
// Workgroup: 256 threads (4 wave64s) own BCO output channels x a pixel block
// of IMGS x TH x TW pixels.  WCO waves split the channels and 4 / WCO the
// pixels; each wave accumulates MI x NJ 32x32 MFMA tiles.  Per LDS fill the
// block stages CB input channels of the source with their one-pixel halo
// (zero where the halo leaves the image) and the matching CB x 9 x BCO
// weights; the next fill's global loads are issued before the current fill's
// MFMAs so that their latency hides behind the math.  MFMA 32x32x2 f32: the
// two reduction elements of a step are two consecutive input channels at the
// same tap; lanes 0-31 and 32-63 read them from adjacent LDS planes.  The
// operands of step t+1 are read from LDS into a second register set while
// the MFMAs of step t run.
//
// Either channel axis may be a concatenation of two tensors (a UNet's
// up-path input [upsampled ; skip], or the two halves of its gradient):
// source channels [0, cin0) come from src and [cin0, Cin) from src1, output
// channels [0, cout0) go to dst and [cout0, Cout) to dst1.  Every LDS fill
// and every channel tile lies inside one of the two tensors (a tensor's
// ragged last fill or tile is zero-padded like any ragged channel count), so
// the choice of tensor is uniform per fill and per workgroup.
#include "activation.hpp"
#include "common.hpp"
#include "launch.hpp"
#include "lds_layout.hpp"
#include "tile_configs.hpp"

namespace conv3x3 {

// PRO: the input prologue (forward: SiLU(x * scale + shift) in the loader;
// backward-data: du = acc * SiLU'(u) in the epilogue); a separate
// instantiation, so that the plain kernels keep their registers.
// PC (forward, vector path, 3 or 4 input channels, e.g. an RGB image): the
// reduction runs over the 9 * PC (channel, tap) pairs packed two per MFMA
// step -- ceil(9 PC / 2) steps instead of the 36 of an 8-channel fill.  The
// tile's weights w[co0 .. co0 + BCO - 1, 0..PC-1, 0..8] are one contiguous
// run of BCO * 9 PC floats, staged with 16-byte loads.
// UP2 (forward of a convolution of the 2x nearest-upsampled input; H, W are
// the small input's sizes, y is 2H x 2W): output row 2i + ph reads
// upsampled rows 2i + ph - 1 .. 2i + ph + 1, i.e. small rows i - 1 and i
// (ph = 0; kernel rows {0}, {1, 2}) or i and i + 1 (ph = 1; rows {0, 1},
// {2}), and likewise for columns.  So each output parity class (ph, pw) is
// a 2x2-tap convolution of the small input whose weights are sums of the
// 3x3 taps: 16 (class, tap) pairs instead of the 36 that the upsampled
// grid needs per small pixel.  The block tiles the small grid, stages x
// with its halo as a plain forward does, keeps one accumulator set per
// class, sums each pair's taps as it reads them, and stores each set to its
// class's pixels.
// S2B (backward-data of a stride-2 convolution; H, W are g's sizes, dx is
// 2H x 2W): dx[2i + ph, 2j + pw] receives only the taps (r, s) with r = 1
// for ph = 0 and r = 0, 2 for ph = 1 (the same for s and pw), tap r reading
// g row i + (ph + 1 - r) / 2.  The block tiles g's grid, stages g with its
// halo as a plain backward-data does, and runs the nine taps once each: tap
// (r, s) feeds the accumulators of its parity class (ph, pw) = (r != 1,
// s != 1) -- four accumulator sets -- and the epilogue stores each set to
// its class's pixels.  The MFMA work is the useful work, and each staged
// tile serves all four classes.
// S2 (forward of a stride-2 convolution): H, W are the input's sizes and the
// pixel block tiles the H/2 x W/2 output; output pixel (ho, wo) at tap (r, s)
// reads input pixel (2 ho + r - 1, 2 wo + s - 1).  The block's 2 TH + 1 input
// rows are staged with their columns split by parity (odd columns, then even
// ones), so that each tap's operand read is unit-stride across the lanes.
// U2B (backward-data of a convolution of the 2x nearest-upsampled input; H,
// W are g's sizes, dx is H/2 x W/2): dx[i, j] sums the upsampled-grid
// gradient over its 2x2 block, i.e. g rows 2i - 1 .. 2i + 2 and columns
// 2j - 1 .. 2j + 2, row offset d taking kernel rows {2}, {1, 2}, {0, 1},
// {0} for d = -1, 0, 1, 2 (likewise columns): a stride-2 convolution of g
// with a 4 x 4 kernel of summed taps, 16 MFMA steps per pixel and channel
// pair instead of 36 plus a 2x2 block sum.  The block tiles dx's grid and
// stages g like the S2 forward stages x, with one more row and one more
// even column (2 w0 + 2 TW).
template <int MODE, int TW, int TH, int IMGS, int BCO, int WCO, int CB, bool VEC, int NW = 4,
          bool PRO = false, int PC = 0, bool UP2 = false, bool S2B = false, bool S2 = false,
          bool U2B = false, bool SPL = false>
__global__ __launch_bounds__(64 * NW) void fwd_f32_kernel(
    const float* __restrict__ src, const float* __restrict__ src1, int cin0,
    const float* __restrict__ wt, const float* __restrict__ bias, float* __restrict__ dst,
    float* __restrict__ dst1, int cout0, int N, int Cin, int Cout, int H, int W, int tiles_w,
    int tiles_h, uint32_t src_bytes, uint32_t src1_bytes, uint32_t wt_bytes, uint32_t dst_bytes,
    uint32_t dst1_bytes, int act, float* __restrict__ zout, const float* __restrict__ zsrc,
    const float* __restrict__ pscale, const float* __restrict__ pshift,
    const float* __restrict__ px, float* __restrict__ part, int per_split, long slot) {
  constexpr int BM = IMGS * TH * TW;
  constexpr int NT = 64 * NW;  // threads
  constexpr int WPX = NW / WCO;
  constexpr int MI = BCO / (32 * WCO);  // 32x32 tiles per wave along channels
  constexpr int NJ = BM / (32 * WPX);   // 32x32 tiles per wave along pixels
  static_assert(MI >= 1 && NJ >= 1 && MI * 32 * WCO == BCO && NJ * 32 * WPX == BM,
                "tile does not split into 32x32 wave tiles");
  // S2 and U2B stage their source at stride 2 with parity-split columns
  constexpr bool STR2 = S2 || U2B;
  constexpr int RS = S2 ? fwd_f32_s2_rs(TW) : U2B ? fwd_f32_u2b_rs(TW) : fwd_f32_rs(TW);
  constexpr int PL = S2    ? fwd_f32_s2_plane(IMGS, TH, TW)
                     : U2B ? fwd_f32_u2b_plane(IMGS, TH, TW)
                           : fwd_f32_plane(IMGS, TH, TW);
  constexpr int WS = fwd_f32_wstride(BCO);
  // staged rows per image (with halo)
  constexpr int HR = S2 ? 2 * TH + 1 : U2B ? 2 * TH + 2 : TH + 2;
  constexpr int EV = fwd_f32_s2_even(TW);  // S2, U2B: row offset of the even columns
  static_assert(PC == 0 || (MODE == kFwd && VEC && PC < CB), "packed taps: forward only");
  static_assert(!UP2 || (MODE == kFwd && PC == 0 && !PRO), "upsampling: plain forward only");
  static_assert(!S2B || (MODE == kBwdData && !PRO && PC == 0 && !UP2),
                "stride-2 parity classes: plain backward-data only");
  static_assert(!S2 || (MODE == kFwd && PC == 0 && !PRO && !UP2), "stride 2: plain forward only");
  static_assert(!U2B || (MODE == kBwdData && PC == 0 && !PRO && !S2B),
                "upsampling: plain backward-data only");
  // output rows and columns (the pixel grid the blocks tile)
  const int OH = STR2 ? H / 2 : H, OW = STR2 ? W / 2 : W;
  constexpr int NSTEP = PC ? (9 * PC + 1) / 2 : CB / 2 * ((UP2 || U2B) ? 16 : 9);
  constexpr int NACC = (S2B || UP2) ? 4 : 1;  // accumulator sets (one per parity class)
  static_assert(!SPL || (!PRO && PC == 0 && !UP2 && !S2B && !S2 && !U2B),
                "split reduction: plain passes only");
  // SPL: a split reduction (compile-time, so that the unsplit kernels carry
  // none of it)
  const int slice = SPL ? (int)blockIdx.z : 0;

  __shared__ __attribute__((aligned(16))) float xs[CB * PL];
  __shared__ float ws[fwd_f32_w_floats(CB, BCO)];
  __shared__ float bias_s[MODE == kFwd ? BCO : 1];  // this tile's biases (0 without bias)

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int wco = wave % WCO, wpx = wave / WCO;
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
  // Reduction fills: nq0 over src's channels, then src1's.
  const int nq0 = (cin0 + CB - 1) / CB;
  const int nchunks = nq0 + (Cin - cin0 + CB - 1) / CB;
  struct Fill {
    bool s1;  // the fill reads src1
    int cl0;  // first channel of the fill within its tensor
    int cs;   // channels of that tensor
    int cg0;  // first channel of the fill in the weight
    int cn;   // valid channels of the fill
  };
  auto fill_of = [&](int chunk) {
    Fill f;
    f.s1 = chunk >= nq0;
    f.cl0 = (chunk - (f.s1 ? nq0 : 0)) * CB;
    f.cs = f.s1 ? Cin - cin0 : cin0;
    f.cg0 = (f.s1 ? cin0 : 0) + f.cl0;
    f.cn = min(CB, f.cs - f.cl0);
    return f;
  };

  // ---------------- staging: source tile ----------------
  // Vector path: interior columns as float4 (W % 4 == 0 so a float4 never
  // straddles the image edge), the two halo columns as scalars.  S2: an item
  // is 8 input columns (two float4) = 4 output columns, and the only halo
  // column is the left one (input column 2 w0 - 1; the right one, 2 (w0 +
  // TW) - 1, is the last odd column of the last item).
  constexpr int XQ = TW / 4;
  constexpr int XV_ITEMS = CB * IMGS * HR * XQ;
  constexpr int XV_N = (XV_ITEMS + NT - 1) / NT;
  constexpr int XH_ITEMS = CB * IMGS * HR * (S2 ? 1 : 2);  // U2B: left and right
  constexpr int XH_N = (XH_ITEMS + NT - 1) / NT;
  // Scalar path: every column of the staged rows.
  constexpr int XCOLS = S2 ? 2 * TW + 1 : U2B ? 2 * TW + 2 : TW + 2;
  constexpr int XS_ITEMS = CB * IMGS * HR * XCOLS;
  constexpr int XS_N = (XS_ITEMS + NT - 1) / NT;
  f32x4 xv[VEC ? XV_N : 1];
  f32x4 xv2[VEC && STR2 ? XV_N : 1];  // S2, U2B: the item's second float4
  float xf[VEC ? XH_N : 1];
  // Backward-data with a fused activation: z at the same positions as the
  // gradient source; the source is multiplied by act'(z) when it is written
  // to LDS (the loads of both are in flight together until then).
  const bool zs = MODE == kBwdData && zsrc != nullptr;
  f32x4 zv[VEC ? XV_N : 1];
  float zf[VEC ? XH_N : 1];
  // halo values that are not loaded stay zero, and so does their z (a zero
  // gradient times act'(0) is zero; times act'(garbage) might not be)
#pragma unroll
  for (int k = 0; k < (VEC ? XH_N : 1); ++k) zf[k] = 0.f;
  // With a single tile across the width both halo columns are padding: they
  // stay zero and are not loaded.
  const bool halo_loads = tiles_w > 1;
#pragma unroll
  for (int k = 0; k < (VEC ? XH_N : 1); ++k) xf[k] = 0.f;
  // Forward with the input prologue: each staged x value becomes
  // SiLU(x * scale[n, c] + shift[n, c]).  An item outside the image or the
  // channels loads x = scale = shift = 0 (offsets past the views) and so
  // stages SiLU(0) = 0: the padding stays zero after the activation.
  constexpr bool pro = MODE == kFwd && PRO;
  float psv[VEC && pro ? XV_N : 1], ptv[VEC && pro ? XV_N : 1];
  float psh[VEC && pro ? XH_N : 1], pth[VEC && pro ? XH_N : 1];
#pragma unroll
  for (int k = 0; k < (VEC && pro ? XH_N : 1); ++k) psh[k] = pth[k] = 0.f;
  const uint32_t pbytes = pro ? 4u * (uint32_t)(N * Cin) : 0u;
  const __amdgpu_buffer_rsrc_t psview = buffer_view(pscale, pbytes);
  const __amdgpu_buffer_rsrc_t ptview = buffer_view(pshift, pbytes);

  // ---------------- staging: weight tile ----------------
  // Forward: for each co, the CB x 9 weights w[co, cg0.., :] are contiguous.
  // Backward-data: for each ci (= k), the BCO x 9 weights w[ci, co0.., :] are.
  constexpr int RUN = MODE == kFwd ? CB * 9 : BCO * 9;
  constexpr int NRUN = MODE == kFwd ? BCO : CB;
  constexpr int WV_ITEMS = NRUN * RUN / 4;
  constexpr int WV_N = (WV_ITEMS + NT - 1) / NT;
  constexpr int WS_ITEMS = CB * 9 * BCO;
  constexpr int WS_N = (WS_ITEMS + NT - 1) / NT;
  f32x4 wv[VEC ? WV_N : 1];
  // packed taps: float4 items of the tile's contiguous weight run
  constexpr int PW = PC ? BCO * PC * 9 / 4 : 1;
  constexpr int PW_N = (PW + NT - 1) / NT;
  static_assert(PC == 0 || (BCO * PC * 9 % 4 == 0 && PW_N <= WV_N), "packed weight items fit");

  // Vector path: global -> registers here (one fill ahead), registers -> LDS
  // in store_tiles.  Scalar path: everything happens in store_tiles.
  // Vector path: buffer views (32-bit offsets); an item outside the tensors
  // or the image reads zero through an offset past the view.
  const __amdgpu_buffer_rsrc_t sview0 = buffer_view(src, src_bytes);
  const __amdgpu_buffer_rsrc_t sview1 = buffer_view(src1, src1_bytes);
  const __amdgpu_buffer_rsrc_t zview = buffer_view(zsrc, zs ? src_bytes : 0u);
  const __amdgpu_buffer_rsrc_t wview = buffer_view(wt, wt_bytes);
  auto load_tiles = [&](int chunk) {
    if constexpr (VEC) {
      const Fill f = fill_of(chunk);
      const __amdgpu_buffer_rsrc_t sview = f.s1 ? sview1 : sview0;
#pragma unroll
      for (int k = 0; k < XV_N; ++k) {
        const int it = tid + k * NT;
        const int q = it % XQ;
        int t = it / XQ;
        const int rr = t % HR;
        t /= HR;
        const int img = t % IMGS;
        const int ch = t / IMGS;
        if constexpr (STR2) {
          // input row 2 h0 - 1 + rr, columns c .. c + 7
          const int n = o.n0 + img, h = 2 * o.h0 + rr - 1, c = 2 * o.w0 + 8 * q;
          const bool ok = (XV_ITEMS % NT == 0 || it < XV_ITEMS) && n < N && ch < f.cn &&
                          h >= 0 && h < H;
          const uint32_t base = 4u * (uint32_t)(((n * f.cs + f.cl0 + ch) * H + h) * W + c);
          xv[k] = __builtin_bit_cast(f32x4, buffer_load16(sview, ok && c < W ? base : kOutside));
          xv2[k] = __builtin_bit_cast(
              f32x4, buffer_load16(sview, ok && c + 4 < W ? base + 16u : kOutside));
          continue;
        }
        const int n = o.n0 + img, h = o.h0 + rr - 1, w = o.w0 + 4 * q;
        const bool ok = (XV_ITEMS % NT == 0 || it < XV_ITEMS) && n < N && ch < f.cn && h >= 0 &&
                        h < H && w < W;
        const uint32_t off =
            ok ? 4u * (uint32_t)(((n * f.cs + f.cl0 + ch) * H + h) * W + w) : kOutside;
        xv[k] = __builtin_bit_cast(f32x4, buffer_load16(sview, off));
        if (zs) zv[k] = __builtin_bit_cast(f32x4, buffer_load16(zview, off));
        if constexpr (pro) {
          const uint32_t po = ok ? 4u * (uint32_t)(n * Cin + f.cg0 + ch) : kOutside;
          psv[k] = __builtin_bit_cast(float, buffer_load4(psview, po));
          ptv[k] = __builtin_bit_cast(float, buffer_load4(ptview, po));
        }
      }
#pragma unroll
      for (int k = 0; k < XH_N; ++k) {
        if (!halo_loads) break;
        const int it = tid + k * NT;
        const int side = S2 ? 0 : it & 1;
        int t = S2 ? it : it >> 1;
        const int rr = t % HR;
        t /= HR;
        const int img = t % IMGS;
        const int ch = t / IMGS;
        const int n = o.n0 + img, h = STR2 ? 2 * o.h0 + rr - 1 : o.h0 + rr - 1;
        // (U2B: input columns 2 w0 - 1 and 2 w0 + 2 TW)
        const int w = S2 ? 2 * o.w0 - 1
                         : U2B ? 2 * o.w0 + (side ? 2 * TW : -1) : o.w0 + (side ? TW : -1);
        const bool ok = (XH_ITEMS % NT == 0 || it < XH_ITEMS) && n < N && ch < f.cn && h >= 0 &&
                        h < H && w >= 0 && w < W;
        const uint32_t off =
            ok ? 4u * (uint32_t)(((n * f.cs + f.cl0 + ch) * H + h) * W + w) : kOutside;
        xf[k] = __builtin_bit_cast(float, buffer_load4(sview, off));
        if (zs) zf[k] = __builtin_bit_cast(float, buffer_load4(zview, off));
        if constexpr (pro) {
          const uint32_t po = ok ? 4u * (uint32_t)(n * Cin + f.cg0 + ch) : kOutside;
          psh[k] = __builtin_bit_cast(float, buffer_load4(psview, po));
          pth[k] = __builtin_bit_cast(float, buffer_load4(ptview, po));
        }
      }
      if constexpr (PC != 0) {
#pragma unroll
        for (int k = 0; k < PW_N; ++k) {
          const int it = tid + k * NT;
          const bool ok = (PW % NT == 0 || it < PW) && 4 * it < co_n * PC * 9;
          wv[k] = __builtin_bit_cast(
              f32x4, buffer_load16(wview, ok ? 4u * (uint32_t)(co0 * PC * 9 + 4 * it) : kOutside));
        }
      }
#pragma unroll
      for (int k = 0; k < WV_N; ++k) {
        if constexpr (PC != 0) break;  // packed taps: the contiguous run above
        const int it = tid + k * NT;
        const int run = it / (RUN / 4);
        const int e = 4 * (it % (RUN / 4));
        bool ok;
        int idx;
        if constexpr (MODE == kFwd) {
          ok = (WV_ITEMS % NT == 0 || it < WV_ITEMS) && run < co_n && e < f.cn * 9;
          idx = ((co0 + run) * Cin + f.cg0) * 9 + e;
        } else {
          ok = (WV_ITEMS % NT == 0 || it < WV_ITEMS) && run < f.cn && e < co_n * 9;
          idx = ((f.cg0 + run) * Cout + co0) * 9 + e;
        }
        wv[k] = __builtin_bit_cast(f32x4, buffer_load16(wview, ok ? 4u * (uint32_t)idx : kOutside));
      }
    }
  };

  // LDS slot of weight element e (0 <= e < RUN) of run `run`.
  auto w_slot = [&](int run, int e) -> int {
    if constexpr (MODE == kFwd) {
      return e * WS + run;  // e = ci_l * 9 + tap, co_l = run
    } else {
      return (run * 9 + (8 - e % 9)) * WS + e / 9;  // ci_l = run, co_l = e/9, tap = 8 - e%9
    }
  };

  auto store_tiles = [&](int chunk) {
    if constexpr (VEC) {
#pragma unroll
      for (int k = 0; k < XV_N; ++k) {
        const int it = tid + k * NT;
        if (XV_ITEMS % NT == 0 || it < XV_ITEMS) {
          const int q = it % XQ;
          const int t = it / XQ;  // (ch * IMGS + img) * HR + rr
          if constexpr (STR2) {
            // columns c .. c + 7 = even 4q .. 4q + 3 and odd 4q + 1 .. 4q + 4
            const f32x4 u = xv[k], u2 = xv2[k];
            *reinterpret_cast<f32x4*>(&xs[t * RS + EV + 4 * q]) = f32x4{u.x, u.z, u2.x, u2.z};
            *reinterpret_cast<f32x4*>(&xs[t * RS + kS2Odd + 1 + 4 * q]) =
                f32x4{u.y, u.w, u2.y, u2.w};
            continue;
          }
          f32x4 v = xv[k];
          if (zs) {
            v.x *= act_slope(act, zv[k].x);
            v.y *= act_slope(act, zv[k].y);
            v.z *= act_slope(act, zv[k].z);
            v.w *= act_slope(act, zv[k].w);
          }
          if constexpr (pro) {
            v.x = act_value(kActSilu, v.x * psv[k] + ptv[k]);
            v.y = act_value(kActSilu, v.y * psv[k] + ptv[k]);
            v.z = act_value(kActSilu, v.z * psv[k] + ptv[k]);
            v.w = act_value(kActSilu, v.w * psv[k] + ptv[k]);
          }
          *reinterpret_cast<f32x4*>(&xs[t * RS + 4 + 4 * q]) = v;
        }
      }
#pragma unroll
      for (int k = 0; k < XH_N; ++k) {
        const int it = tid + k * NT;
        if (XH_ITEMS % NT == 0 || it < XH_ITEMS) {
          if constexpr (S2) {
            xs[it * RS + kS2Odd] = xf[k];  // odd column 0 = input column 2 w0 - 1
            continue;
          }
          if constexpr (U2B) {
            // odd column 0 and even column TW
            xs[(it >> 1) * RS + ((it & 1) ? EV + TW : kS2Odd)] = xf[k];
            continue;
          }
          const int side = it & 1;
          const int t = it >> 1;
          float v = zs ? xf[k] * act_slope(act, zf[k]) : xf[k];
          if constexpr (pro) v = act_value(kActSilu, v * psh[k] + pth[k]);
          xs[t * RS + 4 + (side ? TW : -1)] = v;
        }
      }
      if constexpr (PC != 0) {
        // packed taps: element q of the run is weight e = q % 9PC of output
        // channel q / 9PC; with 9 PC odd the last step's second element
        // (e = 9 PC) reads a zero slot
        if constexpr (PC * 9 % 2 != 0)
          for (int r = tid; r < BCO; r += NT) ws[w_slot(r, PC * 9)] = 0.f;
#pragma unroll
        for (int k = 0; k < PW_N; ++k) {
          const int it = tid + k * NT;
          if (PW % NT == 0 || it < PW) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int q = 4 * it + u;
              ws[w_slot(q / (PC * 9), q % (PC * 9))] = wv[k][u];
            }
          }
        }
      }
#pragma unroll
      for (int k = 0; k < WV_N; ++k) {
        if constexpr (PC != 0) break;
        const int it = tid + k * NT;
        if (WV_ITEMS % NT == 0 || it < WV_ITEMS) {
          const int run = it / (RUN / 4);
          const int e = 4 * (it % (RUN / 4));
          ws[w_slot(run, e + 0)] = wv[k].x;
          ws[w_slot(run, e + 1)] = wv[k].y;
          ws[w_slot(run, e + 2)] = wv[k].z;
          ws[w_slot(run, e + 3)] = wv[k].w;
        }
      }
    } else {
      // Scalar path (ragged shapes): global loads go straight to LDS.
      const Fill f = fill_of(chunk);
      const float* sp = f.s1 ? src1 : src;
#pragma unroll 4
      for (int k = 0; k < XS_N; ++k) {
        const int it = tid + k * NT;
        if (XS_ITEMS % NT == 0 || it < XS_ITEMS) {
          const int cc = it % XCOLS - 1;
          const int t = it / XCOLS;  // (ch * IMGS + img) * HR + rr
          const int rr = t % HR;
          const int img = (t / HR) % IMGS;
          const int ch = t / (HR * IMGS);
          const int n = o.n0 + img;
          // S2, U2B: input column 2 w0 + cc, cc = -1 .. 2 TW - 1 (U2B: .. 2 TW)
          // (odd column (cc + 1) / 2 for even cc + 1, even column cc / 2
          // otherwise)
          const int h = STR2 ? 2 * o.h0 + rr - 1 : o.h0 + rr - 1;
          const int w = STR2 ? 2 * o.w0 + cc : o.w0 + cc;
          const int slot = STR2 ? ((cc & 1) ? kS2Odd + (cc + 1) / 2 : EV + cc / 2) : 4 + cc;
          float v = 0.f;
          if (n < N && ch < f.cn && h >= 0 && h < H && w >= 0 && w < W) {
            const long e = ((long)n * f.cs + f.cl0 + ch) * HW + (long)h * W + w;
            v = sp[e];
            if (zs) v *= act_slope(act, zsrc[e]);
            if constexpr (pro) {
              const long pc = (long)n * Cin + f.cg0 + ch;
              v = act_value(kActSilu, v * pscale[pc] + pshift[pc]);
            }
          }
          xs[t * RS + slot] = v;
        }
      }
#pragma unroll 4
      for (int k = 0; k < WS_N; ++k) {
        const int it = tid + k * NT;
        if (WS_ITEMS % NT == 0 || it < WS_ITEMS) {
          const int run = it / RUN;
          const int e = it % RUN;
          float v = 0.f;
          if constexpr (MODE == kFwd) {
            if (run < co_n && e / 9 < f.cn)
              v = wt[((long)(co0 + run) * Cin + f.cg0 + e / 9) * 9 + e % 9];
          } else {
            if (run < f.cn && e / 9 < co_n)
              v = wt[((long)(f.cg0 + run) * Cout + co0 + e / 9) * 9 + e % 9];
          }
          ws[w_slot(run, e)] = v;
        }
      }
    }
  };

  // ---------------- per-lane operand offsets ----------------
  int boff[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int p = wpx * (BM / WPX) + j * 32 + l32;
    const int img = p / (TH * TW), row = (p / TW) % TH, col = p % TW;
    boff[j] = STR2 ? hi * PL + (img * HR + 2 * row) * RS + col
                 : (PC ? 0 : hi * PL) + (img * HR + row) * RS + 4 + col - 1;
  }
  const int aoff = (PC ? hi : hi * 9) * WS + wco * (BCO / WCO) + l32;


  // UP2 / U2B: the 3x3 taps summed into the weight of step q (kernel rows
  // rlo..rhi, columns slo..shi) and the tile offset of its pixel operand.
  // UP2: q % 4 = output class (ph, pw) -- consecutive steps feed different
  // accumulator sets -- and q / 4 = small-grid tap (u, v); the kernel rows
  // on small row i + u + ph - 1 = tile row row + u + ph are {0}, {1, 2} for
  // ph = 0 and {0, 1}, {2} for ph = 1 (likewise columns).  U2B: g row offset
  // ri - 1 = q / 4 - 1 and column offset si - 1 = q % 4 - 1 from (2i, 2j);
  // kernel rows {2}, {1, 2}, {0, 1}, {0}; columns 2j - 1 .. 2j + 2 are odd
  // j, even j, odd j + 1, even j + 1 of the staged tile.
  struct TapSet {
    int rlo, rhi, slo, shi, boff;
  };
  auto tap_set = [&](int q) {
    TapSet t;
    if constexpr (UP2) {
      const int ph = (q >> 1) & 1, pw = q & 1, u = q >> 3, v = (q >> 2) & 1;
      t.rlo = ph ? 2 * u : u;
      t.rhi = ph ? 1 + u : 2 * u;
      t.slo = pw ? 2 * v : v;
      t.shi = pw ? 1 + v : 2 * v;
      t.boff = (u + ph) * RS + v + pw;
    } else {
      const int ri = q >> 2, si = q & 3;
      t.rlo = ri < 2 ? 2 - ri : 0;
      t.rhi = ri < 2 ? 2 : 3 - ri;
      t.slo = si < 2 ? 2 - si : 0;
      t.shi = si < 2 ? 2 : 3 - si;
      t.boff = ri * RS + (si & 1 ? EV : kS2Odd) + (si >> 1);
    }
    return t;
  };

  // Operands of one MFMA step st = (cp, r, s), cp the channel pair.
  float a[2][MI], b[2][NJ];
  float araw[(UP2 || U2B) ? 2 : 1][MI][4];  // UP2 / U2B: the step's weight taps
  auto read_step = [&](int buf, int st) {
    if constexpr (PC != 0) {
      // reduction elements e = 2 st (lanes 0-31) and 2 st + 1 (32-63), each
      // a (channel, tap) pair; weight slot e, pixel offset of (c, r, s)
      const int e0 = 2 * st, e1 = 2 * st + 1;
      const int o0 = (e0 / 9) * PL + ((e0 % 9) / 3) * RS + e0 % 3;
      const int o1 = (e1 / 9) * PL + ((e1 % 9) / 3) * RS + e1 % 3;
      const int ob = hi ? o1 : o0;
#pragma unroll
      for (int i = 0; i < MI; ++i) a[buf][i] = ws[aoff + e0 * WS + i * 32];
#pragma unroll
      for (int j = 0; j < NJ; ++j) b[buf][j] = xs[boff[j] + ob];
    } else if constexpr (UP2 || U2B) {
      // the weight taps of step st = 16 cp + q (summed into a just before
      // the step's MFMAs, so that waiting for these reads never holds up the
      // MFMAs of the step before) and its pixel operand
      const int cp = st >> 4;
      const TapSet ts = tap_set(st & 15);
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        int k = 0;
#pragma unroll
        for (int r = ts.rlo; r <= ts.rhi; ++r)
#pragma unroll
          for (int s = ts.slo; s <= ts.shi; ++s, ++k)
            araw[buf][i][k] = ws[aoff + (2 * cp * 9 + (U2B ? 8 - (3 * r + s) : 3 * r + s)) * WS +
                                 i * 32];
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) b[buf][j] = xs[boff[j] + 2 * cp * PL + ts.boff];
    } else if constexpr (S2B) {
      // weight tap (r, s): LDS slot 8 - (3 r + s) (the backward rotation);
      // g at tile offset ((ph + 1 - r) / 2 + 1, (pw + 1 - s) / 2 + 1)
      const int cp = st / 9, r = (st % 9) / 3, s = st % 3;
      const int tr = ((r != 1) + 1 - r) / 2 + 1, ts = ((s != 1) + 1 - s) / 2 + 1;
#pragma unroll
      for (int i = 0; i < MI; ++i)
        a[buf][i] = ws[aoff + (2 * cp * 9 + 8 - (3 * r + s)) * WS + i * 32];
#pragma unroll
      for (int j = 0; j < NJ; ++j) b[buf][j] = xs[boff[j] + 2 * cp * PL + tr * RS + ts];
    } else {
      const int cp = st / 9, r = (st % 9) / 3, s = st % 3;
#pragma unroll
      for (int i = 0; i < MI; ++i) a[buf][i] = ws[aoff + (2 * cp * 9 + r * 3 + s) * WS + i * 32];
      // S2: taps s = 0, 1, 2 read odd column j, even column j, odd column j + 1
      const int so = S2 ? (s == 1 ? EV : kS2Odd + s / 2) : s;
#pragma unroll
      for (int j = 0; j < NJ; ++j) b[buf][j] = xs[boff[j] + 2 * cp * PL + r * RS + so];
    }
  };

  // Forward: the accumulators start at the tile's biases (zero without
  // bias), so the epilogue is stores only.
  if constexpr (MODE == kFwd) {
    for (int i = tid; i < BCO; i += NT)
      bias_s[i] = (bias != nullptr && i < co_n && slice == 0) ? bias[co0 + i] : 0.f;
    __syncthreads();
  }
  // (S2B: parity class c's tiles are acc[c * MI + i])
  f32x16 acc[NACC * MI][NJ];
#pragma unroll
  for (int i = 0; i < NACC * MI; ++i) {
    f32x16 init;
#pragma unroll
    for (int v = 0; v < 16; ++v)
      init[v] = MODE == kFwd ? bias_s[wco * (BCO / WCO) + (i % MI) * 32 + acc_row(v, hi)] : 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = init;
  }

  // A split reduction (SPL) gives slice blockIdx.z the fills fbase ..
  // fbase + per_split - 1 and writes its partial sums (the bias in slice 0
  // only) to slot blockIdx.z of part.
  const int fbase = SPL ? slice * per_split : 0;
  const int fend = SPL ? min(nchunks, fbase + per_split) : nchunks;
  load_tiles(fbase);
  for (int chunk = fbase; chunk < fend; ++chunk) {
    if (chunk != fbase) __syncthreads();
    store_tiles(chunk);
    __syncthreads();
    if (chunk + 1 < fend) load_tiles(chunk + 1);
    read_step(0, 0);
    if constexpr (UP2 || U2B) {
      // 16 (class, tap) steps per channel pair: the channel pairs are a
      // plain loop and the 16 steps are unrolled, so that every step's
      // class, taps and accumulator set are compile-time (a fully unrolled
      // fill of 64 such steps is past the compiler's unroll budget, and a
      // runtime accumulator index turns into selects over all four sets)
#pragma unroll 1
      for (int cp = 0; cp < CB / 2; ++cp) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int cur = q & 1;
          if (q + 1 < 16 || cp + 1 < CB / 2) read_step(cur ^ 1, 16 * cp + q + 1);
          __builtin_amdgcn_sched_barrier(0);
          const TapSet ts = tap_set(q);
          const int nt = (ts.rhi - ts.rlo + 1) * (ts.shi - ts.slo + 1);
#pragma unroll
          for (int i = 0; i < MI; ++i) {
            float sum = araw[cur][i][0];
#pragma unroll
            for (int k = 1; k < nt; ++k) sum += araw[cur][i][k];
            a[cur][i] = sum;
          }
          const int c = UP2 ? q % 4 : 0;  // UP2: the output class of this step
#pragma unroll
          for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
              acc[c * MI + i][j] = mfma_32x32x2_f32(a[cur][i], b[cur][j], acc[c * MI + i][j]);
        }
      }
    } else {
#pragma unroll
      for (int st = 0; st < NSTEP; ++st) {
        const int cur = st & 1;
        if (st + 1 < NSTEP) read_step(cur ^ 1, st + 1);
        // Keep the next step's LDS reads ahead of this step's MFMAs (the
        // scheduler would otherwise sink them next to their use).
        __builtin_amdgcn_sched_barrier(0);
        // S2B: the parity class of this step's tap picks the accumulator set
        const int c = S2B ? 2 * ((st % 9) / 3 != 1) + (st % 3 != 1) : 0;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[c * MI + i][j] = mfma_32x32x2_f32(a[cur][i], b[cur][j], acc[c * MI + i][j]);
      }
    }
  }

  // ---------------- epilogue: NCHW stores ----------------
  // Forward with a fused activation: y = act(z), z = the accumulator (bias
  // included), also written to zout when it is given.
  // (zout, forward only, has the shape of dst; the output is then one tensor.)
  // Backward-data with the input prologue: du = acc * SiLU'(x * scale +
  // shift) at the output position (px has dx's shape, one tensor).
  const int cw = col0 + wco * (BCO / WCO);  // first output channel of this wave
  float* const od = SPL ? part + (long)slice * slot : oseg ? dst1 : dst;
  const uint32_t od_bytes = oseg ? dst1_bytes : dst_bytes;
  if constexpr (MODE == kBwdData && PRO) {
    // scale and shift of the tile's channels and images, through LDS (the
    // operand tiles are no longer read); then, four elements at a time, x at
    // the output position, du = acc * SiLU'(u) and its store (one offset
    // for both; elements outside the tensor read zero and store nothing).
    static_assert(2 * IMGS * BCO <= fwd_f32_x_floats(CB, IMGS, TH, TW), "scale/shift fit");
    float* ps_s = xs;
    float* pt_s = xs + IMGS * BCO;
    __syncthreads();
    for (int e = tid; e < IMGS * BCO; e += NT) {
      const int n = o.n0 + e / BCO, co = col0 + e % BCO;
      const bool ok = n < N && co < ocs;
      ps_s[e] = ok ? pscale[(long)n * Cout + co] : 0.f;
      pt_s[e] = ok ? pshift[(long)n * Cout + co] : 0.f;
    }
    __syncthreads();
    const __amdgpu_buffer_rsrc_t xview_b = buffer_view(px, od_bytes);
    const __amdgpu_buffer_rsrc_t dview_b = buffer_view(od, od_bytes);
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
          uint32_t xo[4];
#pragma unroll
          for (int v = v0; v < v0 + 4; ++v) {
            const int co = cw + i * 32 + acc_row(v, hi);
            xo[v - v0] =
                in && co < ocs
                    ? (((uint32_t)n * ocs + co) * (uint32_t)HW + (uint32_t)(h * W + w)) * 4u
                    : kOutside;
            xe[v - v0] = __builtin_bit_cast(float, buffer_load4(xview_b, xo[v - v0]));
          }
#pragma unroll
          for (int v = v0; v < v0 + 4; ++v) {
            const int e = img * BCO + (cw - col0) + i * 32 + acc_row(v, hi);
            buffer_store4(dview_b, xo[v - v0], 0u,
                          acc[i][j][v] * act_slope(kActSilu, xe[v - v0] * ps_s[e] + pt_s[e]));
          }
        }
      }
    }
    return;
  }
  if constexpr (S2B || UP2) {
    // parity class c = (ph, pw) writes pixel (h, w) of the tiled grid to
    // (2h + ph, 2w + pw) of the 2H x 2W output
    const uint32_t plane2 = 4u * (uint32_t)H * (uint32_t)W;  // output plane, floats
    const bool bufst = od_bytes != 0 && co_n == BCO;
    const __amdgpu_buffer_rsrc_t dv = buffer_view(od, od_bytes);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int p = wpx * (BM / WPX) + j * 32 + l32;
      const int img = p / (TH * TW), row = (p / TW) % TH, col = p % TW;
      const int n = o.n0 + img, h = o.h0 + row, w = o.w0 + col;
      const bool keep = n < N && h < H && w < W;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t pix = (uint32_t)((2 * h + (c >> 1)) * (2 * W) + 2 * w + (c & 1));
        if (bufst) {
          const uint32_t off =
              keep ? (((uint32_t)n * ocs + cw + 4 * hi) * plane2 + pix) * 4u : kOutside;
#pragma unroll
          for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v)
              buffer_store4(dv, off, (uint32_t)(i * 32 + 8 * (v >> 2) + (v & 3)) * plane2 * 4u,
                            acc[c * MI + i][j][v]);
        } else if (keep) {
          float* out = od + (long)n * ocs * plane2 + pix;
#pragma unroll
          for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int co = cw + i * 32 + acc_row(v, hi);
              if (co < ocs) out[(long)co * plane2] = acc[c * MI + i][j][v];
            }
        }
      }
    }
    return;
  }
  const bool plain = MODE != kFwd || (act == kActNone && zout == nullptr);
  const long HWo = (long)OH * OW;
  if (od_bytes != 0 && co_n == BCO) {
    // Whole channel tile in range: one buffer store per accumulator element,
    // the lane's byte offset computed once per pixel column j and the
    // channel step a uniform (scalar) offset.  Pixels outside the image get
    // an offset past the view and the hardware drops their stores.
    const __amdgpu_buffer_rsrc_t dv = buffer_view(od, od_bytes);
    const __amdgpu_buffer_rsrc_t zov = buffer_view(zout, plain ? 0u : od_bytes);
    const uint32_t plane = (uint32_t)HWo * 4u;
    auto lane_offset = [&](int j) -> uint32_t {
      const int p = wpx * (BM / WPX) + j * 32 + l32;
      const int img = p / (TH * TW), row = (p / TW) % TH, col = p % TW;
      const int n = o.n0 + img, h = o.h0 + row, w = o.w0 + col;
      const bool keep = n < N && h < OH && w < OW;
      return keep ? (((uint32_t)n * ocs + cw + 4 * hi) * (uint32_t)HWo + (uint32_t)(h * OW + w)) * 4u
                  : kOutside;
    };
    // The plain stores are a loop nest of their own: with the run-time test
    // inside the loop over j, every merge after it waits on the stores.
    if (plain) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const uint32_t off = lane_offset(j);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            buffer_store4(dv, off, (uint32_t)(i * 32 + 8 * (v >> 2) + (v & 3)) * plane,
                          acc[i][j][v]);
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const uint32_t off = lane_offset(j);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const uint32_t so = (uint32_t)(i * 32 + 8 * (v >> 2) + (v & 3)) * plane;
          if (zout) buffer_store4(zov, off, so, acc[i][j][v]);
          buffer_store4(dv, off, so, act_value(act, acc[i][j][v]));
        }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int p = wpx * (BM / WPX) + j * 32 + l32;
    const int img = p / (TH * TW), row = (p / TW) % TH, col = p % TW;
    const int n = o.n0 + img, h = o.h0 + row, w = o.w0 + col;
    if (n >= N || h >= OH || w >= OW) continue;
    float* out = od + (long)n * ocs * HWo + (long)h * OW + w;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int co = cw + i * 32 + acc_row(v, hi);
        if (co < ocs) {
          if (plain) {
            out[(long)co * HWo] = acc[i][j][v];
          } else {
            if (zout) zout[(out - od) + (long)co * HWo] = acc[i][j][v];
            out[(long)co * HWo] = act_value(act, acc[i][j][v]);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host launcher: dispatch the plan's tile to its instantiation.

template <int MODE, int TW, int TH, int IMGS, int BCO, int WCO>
static bool launch_cfg(const Plan& pl, bool vec, Split<const float> src, const float* wt,
                       const float* bias, Split<float> dst, int N, int Cin, int Cout, int H,
                       int W, const ActArgs& a, float* ws, hipStream_t stream) {
  constexpr int CB = 8;
  const bool s2b = MODE == kBwdData && a.s2;
  // split reduction: partial sums into ws (one output-sized slot per
  // slice), then the slot-order reduce
  float* const part = pl.split > 1 ? ws : nullptr;
  const long slot = (long)N * Cout * H * W;
  dim3 grid(pl.grid_x, pl.grid_y, part ? pl.split : 1), block(256, 1, 1);
  // Buffer-view stores need each output tensor below 2 GiB (32-bit byte
  // offsets); otherwise both take the plain-store path.
  // A stride-2 backward-data and an upsampling forward run their parity
  // classes over the H/2 x W/2 grid of g or x (the kernel's H, W); H, W here
  // are the output's.
  const bool quad = s2b || (MODE == kFwd && a.up2);
  const int kH = quad ? H / 2 : H, kW = quad ? W / 2 : W;
  const long hw4 = (long)H * W * 4;
  // output plane bytes (a stride-2 forward and an upsampling backward-data
  // write an H/2 x W/2 output)
  const long ohw4 = (MODE == kFwd ? a.s2 : a.up2) ? hw4 / 4 : hw4;
  const long ob0 = (long)N * dst.c0 * ohw4, ob1 = (long)N * (Cout - dst.c0) * ohw4;
  const bool small = ob0 < 2147483648L && ob1 < 2147483648L;
  const uint32_t db0 = small ? (uint32_t)ob0 : 0u, db1 = small ? (uint32_t)ob1 : 0u;
  const long shw4 = quad ? hw4 / 4 : hw4;  // source plane bytes
  const uint32_t sb0 = vec ? (uint32_t)(N * src.c0 * shw4) : 0u;
  const uint32_t sb1 = vec ? (uint32_t)(N * (Cin - src.c0) * shw4) : 0u;
  const uint32_t wb = vec ? (uint32_t)((long)Cin * Cout * 9 * 4) : 0u;
#define CONV3X3_LS(VEC_, PRO_, PC_, UP_, S2B_, S2_, U2B_, SPL_)                                  \
  hipLaunchKernelGGL((fwd_f32_kernel<MODE, TW, TH, IMGS, BCO, WCO, CB, VEC_, 4, PRO_, PC_, UP_,   \
                                     S2B_, S2_, U2B_, SPL_>),                                     \
                     grid,                                                                        \
                     block, 0, stream, src.p0, src.p1, src.c0, wt, bias, dst.p0, dst.p1, dst.c0, N, \
                     Cin, Cout, kH, kW, pl.tiles_w, pl.tiles_h, sb0, sb1, wb, db0, db1, a.act,     \
                     a.zout, a.zsrc, a.pscale, a.pshift, a.px, part, pl.chunks_per_split, slot)
#define CONV3X3_L(VEC_, PRO_, PC_, UP_, S2B_, S2_, U2B_) \
  CONV3X3_LS(VEC_, PRO_, PC_, UP_, S2B_, S2_, U2B_, false)
  // packed taps: the forward of a 3- or 4-channel single tensor
  const int pc =
      (MODE == kFwd && vec && !a.pscale && !a.up2 && !a.s2 && src.c0 == Cin) ? Cin : 0;
  constexpr bool kF = MODE == kFwd;
  // one 32 x 32 MFMA tile per wave (64 x 64 workgroup tiles), so that the
  // four accumulator sets of a stride-2 backward-data or an upsampling
  // forward fit
  constexpr bool one_tile = BCO / (32 * WCO) * (IMGS * TH * TW) / (32 * (4 / WCO)) == 1;
  if (a.s2) {
    if constexpr (kF) {
      if (vec)
        CONV3X3_L(true, false, 0, false, false, true, false);
      else
        CONV3X3_L(false, false, 0, false, false, true, false);
    } else if constexpr (one_tile) {
      if (vec)
        CONV3X3_L(true, false, 0, false, true, false, false);
      else
        CONV3X3_L(false, false, 0, false, true, false, false);
    } else {
      return false;  // the planner gives stride-2 backward-data 64 x 64 tiles
    }
  } else if (a.up2) {
    if constexpr (!kF) {
      if (vec)
        CONV3X3_L(true, false, 0, false, false, false, true);
      else
        CONV3X3_L(false, false, 0, false, false, false, true);
    } else if constexpr (one_tile) {
      if (vec)
        CONV3X3_L(true, false, 0, true, false, false, false);
      else
        CONV3X3_L(false, false, 0, true, false, false, false);
    } else {
      return false;  // the planner gives the upsampling forward 64 x 64 tiles
    }
  } else if (a.pscale) {
    if (vec)
      CONV3X3_L(true, true, 0, false, false, false, false);
    else
      CONV3X3_L(false, true, 0, false, false, false, false);
  } else if (pc == 3) {
    CONV3X3_L(true, false, kF ? 3 : 0, false, false, false, false);
  } else if (pc == 4) {
    CONV3X3_L(true, false, kF ? 4 : 0, false, false, false, false);
  } else if (part) {
    // the planner splits only 64-pixel x 64-channel tiles of four waves
    if constexpr (BCO == 64 && WCO == 2 && IMGS * TH * TW == 64) {
      if (vec)
        CONV3X3_LS(true, false, 0, false, false, false, false, true);
      else
        CONV3X3_LS(false, false, 0, false, false, false, false, true);
    } else {
      return false;
    }
  } else {
    if (vec)
      CONV3X3_L(true, false, 0, false, false, false, false);
    else
      CONV3X3_L(false, false, 0, false, false, false, false);
  }
#undef CONV3X3_L
#undef CONV3X3_LS
  if (part) launch_split_reduce(part, pl.split, slot, dst.p0, stream);
  return true;
}

template <int MODE>
static bool launch_mode(const Plan& pl, bool vec, Split<const float> src, const float* wt,
                        const float* bias, Split<float> dst, int N, int Cin, int Cout, int H,
                        int W, const ActArgs& a, float* ws, hipStream_t s) {
  if (pl.chunk != 8) return false;
  // a split reduction: plain passes only, with a workspace and one output
  // tensor
  if (pl.split > 1 && (ws == nullptr || dst.c0 != Cout || a.act != kActNone || a.zout || a.zsrc ||
                       a.pscale || a.up2 || a.s2))
    return false;
#define CONV3X3_X(TW_, TH_, IMGS_, CO_, WCO_)                                               \
  if (pl.tw == TW_ && pl.th == TH_ && pl.imgs == IMGS_ && pl.tile_co == CO_ &&              \
      pl.wave_co == WCO_) {                                                                 \
    return launch_cfg<MODE, TW_, TH_, IMGS_, CO_, WCO_>(pl, vec, src, wt, bias, dst, N, Cin, \
                                                        Cout, H, W, a, ws, s);              \
  }
  CONV3X3_FWD_F32_CONFIGS(CONV3X3_X)
#undef CONV3X3_X
  return false;
}

bool launch_fwd_f32(const Plan& pl, bool vec, Split<const float> src, const float* wt,
                    const float* bias, Split<float> dst, int N, int Cin, int Cout, int H, int W,
                    const ActArgs& a, float* ws, hipStream_t stream) {
  if (pl.pass == kFwd)
    return launch_mode<kFwd>(pl, vec, src, wt, bias, dst, N, Cin, Cout, H, W, a, ws, stream);
  return launch_mode<kBwdData>(pl, vec, src, wt, nullptr, dst, N, Cin, Cout, H, W, a, ws,
                               stream);
}

}  // namespace conv3x3
