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
// channels of one pixel ([group][img][row][col] words).  It is built from
// 128-bit NCHW loads (8 pixels of one channel) by a 4-channel x 8-pixel
// transpose in registers; no global memory is ever transposed.
//
// Weights, as one 16-byte word per (tap, 8-channel group, output channel):
//   forward       : w[co, c0 + 8g .. + 7, 0..8] is 144 contiguous bytes, loaded
//                   with nine 128-bit loads and rearranged in registers;
//   backward-data : the reduction channel is k, the slowest axis of w, so the
//                   raw rows w[k, co0.., 0..8] are first copied to LDS and then
//                   transposed LDS-to-LDS in 8 x 8 blocks, with the 180-degree
//                   tap rotation applied in the store index.
#include "common.hpp"
#include "launch.hpp"
#include "lds_layout.hpp"

namespace conv3x3 {

namespace {

// Low / high 16 bits of two dwords packed into one.
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}
// Element e (bf16) of an array of packed dwords.
template <int E>
__device__ __forceinline__ uint32_t elem(const uint32_t* d) {
  return (E & 1) ? (d[E >> 1] >> 16) : (d[E >> 1] & 0xffffu);
}

}  // namespace

template <int MODE, int TW, int TH, int IMGS, int BCO, bool VEC>
__global__ __launch_bounds__(256) void fwd_bf16_kernel(
    const uint16_t* __restrict__ src, const uint16_t* __restrict__ wt,
    const float* __restrict__ bias, float* __restrict__ dst, int N, int Cin, int Cout, int H,
    int W, int tiles_w, int tiles_h) {
  constexpr int CB = 16;
  constexpr int BM = IMGS * TH * TW;
  static_assert(BM == 128, "pixel block must hold 128 pixels");
  constexpr int RS = fwd_bf16_rs(TW);
  constexpr int HR = TH + 2;
  constexpr int PLW = fwd_bf16_plane(IMGS, TH, TW);  // words per 8-channel plane
  constexpr int MI = BCO / 64;
  constexpr int NJ = BM / 64;
  constexpr int EW = BCO * 9 / 8;  // raw weight words per reduction channel (backward-data)

  __shared__ u32x4 xs[2 * PLW];
  __shared__ u32x4 wa[9 * 2 * BCO];
  __shared__ u32x4 wraw[MODE == kBwdData && VEC ? CB * EW : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int wco = wave & 1, wpx = wave >> 1;
  const BlockOrigin o = block_origin<TW, TH, IMGS>(blockIdx.x, tiles_w, tiles_h);
  const int co0 = blockIdx.y * BCO;
  const long HW = (long)H * W;

  // ---- vector staging (W % 8 == 0, channel counts % 8 == 0, 16-byte bases) ----
  // x: item (c4, img, rr, q8) = 4 channels x 8 pixels.
  constexpr int XI = 4 * IMGS * HR * (TW / 8);
  constexpr int XH = 4 * IMGS * HR * 2;  // halo items: 4 channels x 1 pixel
  static_assert(XI <= 256 && XH <= 256, "one x item per thread");
  // weights: forward item (co_l, g) = 9 words; backward-data raw item = 1 word.
  constexpr int WI = MODE == kFwd ? 2 * BCO : CB * EW;
  constexpr int WN = MODE == kFwd ? 1 : (WI + 255) / 256;
  constexpr int WR = MODE == kFwd ? 9 : WN;
  u32x4 xr[4];
  uint32_t hr[2];
  u32x4 wr[WR];

  auto load_tiles = [&](int c0) {
    if constexpr (VEC) {
      {
        const int it = tid;
        if (it < XI) {
          const int q = it % (TW / 8);
          int t = it / (TW / 8);
          const int rr = t % HR;
          t /= HR;
          const int img = t % IMGS;
          const int c4 = t / IMGS;
          const int n = o.n0 + img, h = o.h0 + rr - 1, w = o.w0 + 8 * q;
          const bool ok = n < N && h >= 0 && h < H && w < W;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int c = c0 + 4 * c4 + i;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (ok && c < Cin)
              v = *reinterpret_cast<const u32x4*>(src + ((long)n * Cin + c) * HW + (long)h * W + w);
            xr[i] = v;
          }
        }
      }
      {
        const int it = tid;
        hr[0] = hr[1] = 0u;
        if (it < XH) {
          const int side = it & 1;
          int t = it >> 1;
          const int rr = t % HR;
          t /= HR;
          const int img = t % IMGS;
          const int c4 = t / IMGS;
          const int n = o.n0 + img, h = o.h0 + rr - 1, w = o.w0 + (side ? TW : -1);
          if (n < N && h >= 0 && h < H && w >= 0 && w < W) {
            uint32_t v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int c = c0 + 4 * c4 + i;
              v[i] = c < Cin ? src[((long)n * Cin + c) * HW + (long)h * W + w] : 0u;
            }
            hr[0] = v[0] | (v[1] << 16);
            hr[1] = v[2] | (v[3] << 16);
          }
        }
      }
      if constexpr (MODE == kFwd) {
        const int co_l = tid >> 1, gq = tid & 1;
        const int co = co0 + co_l;
        const bool ok = tid < WI && co < Cout && c0 + 8 * gq < Cin;
        const uint16_t* p = wt + ((long)co * Cin + c0 + 8 * gq) * 9;
#pragma unroll
        for (int i = 0; i < 9; ++i) {
          u32x4 v = {0u, 0u, 0u, 0u};
          if (ok) v = reinterpret_cast<const u32x4*>(p)[i];
          wr[i] = v;
        }
      } else {
#pragma unroll
        for (int k = 0; k < WN; ++k) {
          const int it = tid + 256 * k;
          u32x4 v = {0u, 0u, 0u, 0u};
          if (WI % 256 == 0 || it < WI) {
            const int kl = it / EW, e8 = it % EW;
            if (c0 + kl < Cin && 8 * e8 < (Cout - co0) * 9)
              v = *reinterpret_cast<const u32x4*>(wt + ((long)(c0 + kl) * Cout + co0) * 9 + 8 * e8);
          }
          wr[k] = v;
        }
      }
    }
  };

  auto store_tiles = [&](int c0) {
    if constexpr (VEC) {
      if (tid < XI) {
        const int q = tid % (TW / 8);
        const int t = tid / (TW / 8);  // (c4 * IMGS + img) * HR + rr
        const int c4 = t / (IMGS * HR);
        const int row = t % (IMGS * HR);
        uint2* d = reinterpret_cast<uint2*>(&xs[(c4 >> 1) * PLW + row * RS + 4 + 8 * q]) + (c4 & 1);
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          const int dw = p >> 1;
          uint2 v;
          if (p & 1) {
            v.x = pack_hi(xr[0][dw], xr[1][dw]);
            v.y = pack_hi(xr[2][dw], xr[3][dw]);
          } else {
            v.x = pack_lo(xr[0][dw], xr[1][dw]);
            v.y = pack_lo(xr[2][dw], xr[3][dw]);
          }
          d[2 * p] = v;  // word stride is two uint2
        }
      }
      if (tid < XH) {
        const int side = tid & 1;
        const int t = tid >> 1;
        const int c4 = t / (IMGS * HR);
        const int row = t % (IMGS * HR);
        uint2* d = reinterpret_cast<uint2*>(&xs[(c4 >> 1) * PLW + row * RS + 4 + (side ? TW : -1)]) +
                   (c4 & 1);
        *d = make_uint2(hr[0], hr[1]);
      }
      if constexpr (MODE == kFwd) {
        if (tid < WI) {
          const int co_l = tid >> 1, gq = tid & 1;
          const uint32_t* d = reinterpret_cast<const uint32_t*>(wr);  // 36 dwords, e = ci * 9 + t
          // word for tap t: channels (2q, 2q+1) -> elements 2q*9+t and (2q+1)*9+t
#define CONV3X3_WWORD(T)                                                                   \
  {                                                                                       \
    u32x4 v;                                                                              \
    v.x = elem<0 * 9 + T>(d) | (elem<1 * 9 + T>(d) << 16);                                \
    v.y = elem<2 * 9 + T>(d) | (elem<3 * 9 + T>(d) << 16);                                \
    v.z = elem<4 * 9 + T>(d) | (elem<5 * 9 + T>(d) << 16);                                \
    v.w = elem<6 * 9 + T>(d) | (elem<7 * 9 + T>(d) << 16);                                \
    wa[((T) * 2 + gq) * BCO + co_l] = v;                                                  \
  }
          CONV3X3_WWORD(0)
          CONV3X3_WWORD(1)
          CONV3X3_WWORD(2)
          CONV3X3_WWORD(3)
          CONV3X3_WWORD(4)
          CONV3X3_WWORD(5)
          CONV3X3_WWORD(6)
          CONV3X3_WWORD(7)
          CONV3X3_WWORD(8)
#undef CONV3X3_WWORD
        }
      } else {
#pragma unroll
        for (int k = 0; k < WN; ++k) {
          const int it = tid + 256 * k;
          if (WI % 256 == 0 || it < WI) wraw[it] = wr[k];
        }
        __syncthreads();
        // 8 x 8 transpose: 8 reduction channels (k) x 8 consecutive (co, tap)
        // elements of the raw rows -> 8 words of 8 k each.
        constexpr int TI = 2 * EW;
#pragma unroll
        for (int k = 0; k < (TI + 255) / 256; ++k) {
          const int it = tid + 256 * k;
          if (TI % 256 == 0 || it < TI) {
            const int g = it / EW, eb = it % EW;
            u32x4 in[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) in[j] = wraw[(8 * g + j) * EW + eb];
#pragma unroll
            for (int ei = 0; ei < 8; ++ei) {
              const int dw = ei >> 1;
              u32x4 v;
              if (ei & 1) {
                v.x = pack_hi(in[0][dw], in[1][dw]);
                v.y = pack_hi(in[2][dw], in[3][dw]);
                v.z = pack_hi(in[4][dw], in[5][dw]);
                v.w = pack_hi(in[6][dw], in[7][dw]);
              } else {
                v.x = pack_lo(in[0][dw], in[1][dw]);
                v.y = pack_lo(in[2][dw], in[3][dw]);
                v.z = pack_lo(in[4][dw], in[5][dw]);
                v.w = pack_lo(in[6][dw], in[7][dw]);
              }
              const int e = 8 * eb + ei;  // co_l * 9 + tap of the stored (unrotated) weight
              wa[((8 - e % 9) * 2 + g) * BCO + e / 9] = v;
            }
          }
        }
      }
    } else {
      // Scalar path (ragged shapes): 16-bit loads straight into LDS.
      uint16_t* xh = reinterpret_cast<uint16_t*>(xs);
      uint16_t* wh = reinterpret_cast<uint16_t*>(wa);
      constexpr int XS = CB * IMGS * HR * (TW + 2);
#pragma unroll 4
      for (int k = 0; k < (XS + 255) / 256; ++k) {
        const int it = tid + 256 * k;
        if (XS % 256 == 0 || it < XS) {
          const int cc = it % (TW + 2) - 1;
          const int t = it / (TW + 2);  // (ch * IMGS + img) * HR + rr
          const int rr = t % HR;
          const int img = (t / HR) % IMGS;
          const int ch = t / (HR * IMGS);
          const int n = o.n0 + img, c = c0 + ch, h = o.h0 + rr - 1, w = o.w0 + cc;
          uint16_t v = 0;
          if (n < N && c < Cin && h >= 0 && h < H && w >= 0 && w < W)
            v = src[((long)n * Cin + c) * HW + (long)h * W + w];
          xh[((ch >> 3) * PLW + (img * HR + rr) * RS + 4 + cc) * 8 + (ch & 7)] = v;
        }
      }
      constexpr int WS = CB * 9 * BCO;
#pragma unroll 4
      for (int k = 0; k < WS / 256; ++k) {
        const int it = tid + 256 * k;
        int ci_l, co_l, tap;
        uint16_t v = 0;
        if constexpr (MODE == kFwd) {
          co_l = it / (CB * 9);
          const int e = it % (CB * 9);
          ci_l = e / 9;
          tap = e % 9;
          const int co = co0 + co_l, ci = c0 + ci_l;
          if (co < Cout && ci < Cin) v = wt[((long)co * Cin + ci) * 9 + tap];
        } else {
          ci_l = it / (BCO * 9);
          const int e = it % (BCO * 9);
          co_l = e / 9;
          const int tg = e % 9;
          tap = 8 - tg;
          const int co = co0 + co_l, ci = c0 + ci_l;
          if (co < Cout && ci < Cin) v = wt[((long)ci * Cout + co) * 9 + tg];
        }
        wh[((tap * 2 + (ci_l >> 3)) * BCO + co_l) * 8 + (ci_l & 7)] = v;
      }
    }
  };

  int boff[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int p = wpx * (BM / 2) + j * 32 + l32;
    const int img = p / (TH * TW), row = (p / TW) % TH, col = p % TW;
    boff[j] = hi * PLW + (img * HR + row) * RS + 4 + col - 1;
  }
  const int aoff = hi * BCO + wco * (BCO / 2) + l32;

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nchunks = (Cin + CB - 1) / CB;
  load_tiles(0);
  for (int chunk = 0; chunk < nchunks; ++chunk) {
    if (chunk) __syncthreads();
    store_tiles(chunk * CB);
    __syncthreads();
    if (chunk + 1 < nchunks) load_tiles((chunk + 1) * CB);
#pragma unroll
    for (int r = 0; r < 3; ++r) {
#pragma unroll
      for (int s = 0; s < 3; ++s) {
        u32x4 a[MI], b[NJ];
#pragma unroll
        for (int i = 0; i < MI; ++i) a[i] = wa[aoff + (r * 3 + s) * 2 * BCO + i * 32];
#pragma unroll
        for (int j = 0; j < NJ; ++j) b[j] = xs[boff[j] + r * RS + s];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j) acc[i][j] = mfma_32x32x16_bf16(a[i], b[j], acc[i][j]);
      }
    }
  }

#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int p = wpx * (BM / 2) + j * 32 + l32;
    const int img = p / (TH * TW), row = (p / TW) % TH, col = p % TW;
    const int n = o.n0 + img, h = o.h0 + row, w = o.w0 + col;
    if (n >= N || h >= H || w >= W) continue;
    float* out = dst + (long)n * Cout * HW + (long)h * W + w;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int co = co0 + wco * (BCO / 2) + i * 32 + acc_row(v, hi);
        if (co < Cout) {
          float val = acc[i][j][v];
          if (MODE == kFwd && bias) val += bias[co];
          out[(long)co * HW] = val;
        }
      }
    }
  }
}

template <int MODE, int TW, int TH, int IMGS, int BCO>
static void launch_bf16_geom(const Plan& pl, bool vec, const uint16_t* src, const uint16_t* wt,
                             const float* bias, float* dst, int N, int Cin, int Cout, int H, int W,
                             hipStream_t stream) {
  dim3 grid(pl.grid_x, pl.grid_y, 1), block(256, 1, 1);
  if (vec)
    hipLaunchKernelGGL((fwd_bf16_kernel<MODE, TW, TH, IMGS, BCO, true>), grid, block, 0, stream,
                       src, wt, bias, dst, N, Cin, Cout, H, W, pl.tiles_w, pl.tiles_h);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<MODE, TW, TH, IMGS, BCO, false>), grid, block, 0, stream,
                       src, wt, bias, dst, N, Cin, Cout, H, W, pl.tiles_w, pl.tiles_h);
}

template <int MODE, int BCO>
static bool launch_bf16_bco(const Plan& pl, bool vec, const uint16_t* src, const uint16_t* wt,
                            const float* bias, float* dst, int N, int Cin, int Cout, int H, int W,
                            hipStream_t s) {
  switch (pl.geom) {
    case kG64x2: launch_bf16_geom<MODE, 64, 2, 1, BCO>(pl, vec, src, wt, bias, dst, N, Cin, Cout, H, W, s); return true;
    case kG32x4: launch_bf16_geom<MODE, 32, 4, 1, BCO>(pl, vec, src, wt, bias, dst, N, Cin, Cout, H, W, s); return true;
    case kG16x8: launch_bf16_geom<MODE, 16, 8, 1, BCO>(pl, vec, src, wt, bias, dst, N, Cin, Cout, H, W, s); return true;
    case kG8x16: launch_bf16_geom<MODE, 8, 16, 1, BCO>(pl, vec, src, wt, bias, dst, N, Cin, Cout, H, W, s); return true;
    case kG8x8x2: launch_bf16_geom<MODE, 8, 8, 2, BCO>(pl, vec, src, wt, bias, dst, N, Cin, Cout, H, W, s); return true;
    default: return false;
  }
}

bool launch_fwd_bf16(const Plan& pl, bool vec, const uint16_t* src, const uint16_t* wt,
                     const float* bias, float* dst, int N, int Cin, int Cout, int H, int W,
                     hipStream_t stream) {
  if (pl.chunk != 16) return false;
  if (pl.pass == kFwd) {
    if (pl.tile_co == 128)
      return launch_bf16_bco<kFwd, 128>(pl, vec, src, wt, bias, dst, N, Cin, Cout, H, W, stream);
    if (pl.tile_co == 64)
      return launch_bf16_bco<kFwd, 64>(pl, vec, src, wt, bias, dst, N, Cin, Cout, H, W, stream);
  } else {
    if (pl.tile_co == 128)
      return launch_bf16_bco<kBwdData, 128>(pl, vec, src, wt, nullptr, dst, N, Cin, Cout, H, W, stream);
    if (pl.tile_co == 64)
      return launch_bf16_bco<kBwdData, 64>(pl, vec, src, wt, nullptr, dst, N, Cin, Cout, H, W, stream);
  }
  return false;
}

}  // namespace conv3x3
