// Backward-weight and bias gradient of the 3x3 convolution, bfloat16 inputs
// with float32 accumulation and output, gfx950.
//
// Same decomposition as the float32 kernel -- a workgroup of 12 wave64s owns
// 64 k x 64 c x 9 taps, wave w the 32 x 32 block (kb, cb) and kernel row
// r = w % 3 -- on v_mfma_f32_32x32x16_bf16, whose lanes each supply 8
// consecutive reduction elements.  The reduction runs over pixels, the
// contiguous axis of NCHW, so both operands come straight from
// pixel-contiguous LDS tiles: g as [k][pixel] and x as [c][img][row][col]
// with its one-pixel halo.  Eight pixels of one row start at an 8-aligned
// column, so the g operand and the centre tap (s = 1) of x are aligned
// 128-bit LDS reads; the left and right taps (s = 0, 2) are the same words
// shifted by one bf16 element, assembled with funnel shifts from the aligned
// word and one dword of its neighbour -- no unaligned LDS access.  A pixel
// chunk is 128 pixels (8 MFMA steps; 64 for 8-wide images), staged through
// buffer views into double-buffered LDS, one barrier per chunk.  Partial
// sums and the split-K reduce are those of the float32 kernel, and so is
// the handling of an x made of two tensors (channels [0, cx0) in x, the rest
// in x1; one tensor per 64-channel tile).
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "lds_layout.hpp"
#include "tile_configs.hpp"

namespace conv3x3 {

namespace {
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
}  // namespace

// ZG: g is a gradient gy at an activation's output, multiplied by act'(zsrc)
// (zsrc float32, g's shape) and rounded to bfloat16 as it is staged.
// PRO: the input prologue -- x is staged as a = SiLU(x * pscale[n, c] +
// pshift[n, c]) rounded to bfloat16 (one x tensor).
template <int TW, int TH, int IMGS, bool VEC, bool ZG, bool PRO, int GEO = kGeoPlain>
__global__ __launch_bounds__(768) void wgrad_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ x1, int cx0,
    const uint16_t* __restrict__ g, float* __restrict__ out, float* __restrict__ out_db, int N,
    int C, int K, int H, int W, int tiles_w, int tiles_h, int nchunks, int per_split,
    long slice_stride, int split, int tiles_c, int tiles_k, uint32_t x_bytes, uint32_t x1_bytes,
    uint32_t g_bytes, int act, const float* __restrict__ zsrc, const float* __restrict__ pscale,
    const float* __restrict__ pshift, int xgeo, int ggeo) {
  constexpr int P = IMGS * TH * TW;
  static_assert(P % 16 == 0, "whole 16-pixel MFMA steps");
  // GEO: the vector path reads x as an H/2 x W/2 tensor at (h/2, w/2)
  // (kGeoUp), or g as an H/2 x W/2 tensor zero-inserted (kGeoZero: only at
  // even h, w); one x tensor, no fusion.  The scalar path takes its geometry
  // from xgeo / ggeo.
  static_assert(GEO == kGeoPlain || (VEC && !ZG && !PRO && (GEO == kGeoUp || GEO == kGeoZero)),
                "resampled vector staging: plain operands only");
  constexpr bool XUP = GEO == kGeoUp, GZI = GEO == kGeoZero;
  static_assert(TW % 8 == 0, "8-pixel operand runs must stay in one row");
  constexpr int GSB = wgrad_bf16_gstride(IMGS, TH, TW);
  constexpr int RSX = wgrad_bf16_rs(TW);
  constexpr int PLX = wgrad_bf16_plane(IMGS, TH, TW);
  constexpr int HR = TH + 2;
  constexpr int NT = 768;

  // Two LDS buffers: chunk i is read from one while chunk i + 1 is written
  // into the other.
  __shared__ __attribute__((aligned(16))) uint16_t gs_buf[2][64 * GSB];
  __shared__ __attribute__((aligned(16))) uint16_t xs_buf[2][64 * PLX];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int r = wave % 3, kb = (wave / 3) & 1, cb = wave / 6;
  // XCD-aware placement: the hardware deals consecutive workgroups to the 8
  // XCDs in turn, so workgroup b takes logical index (b % 8) * (grid / 8) +
  // b / 8.  Each XCD then runs a contiguous range of logical indices -- all
  // channel tiles of the same slices -- and a slice's x / g data is fetched
  // into one L2.  The grid is padded to a multiple of 8; spare workgroups exit.
  const int ntile = tiles_c * tiles_k;
  const int L = (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
  if (L >= split * ntile) return;
  const int slice = L / ntile, tile = L % ntile;
  // channel tile: channels cl0 .. cl0 + cn - 1 of x tensor `xseg` (cs
  // channels; x holds [0, cx0), x1 the rest), channel c0 of dw
  const int ct = tile % tiles_c, nct0 = (cx0 + 63) / 64;
  const bool xseg = ct >= nct0;
  const int cl0 = (ct - (xseg ? nct0 : 0)) * 64;
  const int cs = xseg ? C - cx0 : cx0;
  const int c0 = (xseg ? cx0 : 0) + cl0;
  const int cn = min(64, cs - cl0);
  const uint16_t* const xsrc = xseg ? x1 : x;
  const int k0 = (tile / tiles_c) * 64;
  const long HW = (long)H * W;
  const bool do_db = out_db != nullptr && tile % tiles_c == 0;

  constexpr int XQ = TW / 8;                      // 8-pixel words per row
  constexpr int GI = 64 * IMGS * TH * XQ;         // g words per chunk
  constexpr int GN = (GI + NT - 1) / NT;
  constexpr int XI = 64 * IMGS * HR * XQ;         // x words per chunk
  constexpr int XN = (XI + NT - 1) / NT;
  constexpr int HI_ = 64 * IMGS * HR * 2;         // x halo elements
  constexpr int HN = (HI_ + NT - 1) / NT;
  // Two register sets: the global loads of chunk i + 3 are issued into the
  // set just emptied into LDS for chunk i + 1, so each load has two chunks of
  // MFMA work to arrive.  With ZG the float32 z items take the registers of
  // the second set: one set, loads one chunk ahead.
  constexpr int NSET = (ZG || PRO) ? 1 : 2;
  u32x4 gv[NSET][VEC ? GN : 1];
  u32x4 xv[NSET][VEC ? XN : 1];
  uint16_t xh[NSET][VEC ? HN : 1];
  f32x4 zv[NSET][ZG && VEC ? 2 * GN : 1];
  // PRO: scale and shift of each x item's and halo element's channel
  float pxs[NSET][PRO && VEC ? XN : 1], pxt[NSET][PRO && VEC ? XN : 1];
  float phs[NSET][PRO && VEC ? HN : 1], pht[NSET][PRO && VEC ? HN : 1];
  // With a single tile across the width both halo columns are padding: they
  // stay zero and are not loaded.
  const bool halo_loads = tiles_w > 1;
#pragma unroll
  for (int k = 0; k < (VEC ? HN : 1); ++k)
#pragma unroll
    for (int j = 0; j < NSET; ++j) xh[j][k] = 0;

  // Vector path: buffer views; an item outside the tensors or the image
  // reads zero through an offset past the view (32-bit offset arithmetic).
  const __amdgpu_buffer_rsrc_t gview = buffer_view(g, g_bytes);
  const __amdgpu_buffer_rsrc_t xview = buffer_view(xsrc, xseg ? x1_bytes : x_bytes);
  // z: g's shape in float32, twice g's byte offsets (below 2^31: the caller
  // keeps every float32 tensor under 2 GiB)
  const __amdgpu_buffer_rsrc_t zview = buffer_view(zsrc, ZG ? 2u * g_bytes : 0u);
  // scale / shift: [N][C] float32
  const uint32_t ps_bytes = PRO ? 4u * (uint32_t)N * (uint32_t)C : 0u;
  const __amdgpu_buffer_rsrc_t psview = buffer_view(pscale, ps_bytes);
  const __amdgpu_buffer_rsrc_t ptview = buffer_view(pshift, ps_bytes);
  auto load_tiles = [&](auto set_c, int chunk) __attribute__((always_inline)) {
    constexpr int SET = decltype(set_c)::value;
    if constexpr (VEC) {
      const BlockOrigin o = block_origin<TW, TH, IMGS>(chunk, tiles_w, tiles_h);
#pragma unroll
      for (int k = 0; k < GN; ++k) {
        const int it = tid + k * NT;
        const int q = it % XQ;
        int t = it / XQ;
        const int row = t % TH;
        t /= TH;
        const int img = t % IMGS;
        const int kl = t / IMGS;
        const int n = o.n0 + img, kk = k0 + kl, h = o.h0 + row, w = o.w0 + 8 * q;
        const bool ok = (GI % NT == 0 || it < GI) && n < N && kk < K && h < H && w < W;
        if constexpr (GZI) {
          // 8 pixels of an even row: 4 source elements at (h/2, w/2)
          const uint32_t e = (uint32_t)(((n * K + kk) * (H >> 1) + (h >> 1)) * (W >> 1) + (w >> 1));
          const uint64_t u = buffer_load8(gview, ok && (h & 1) == 0 ? 2u * e : kOutside);
          gv[SET][k].x = (uint32_t)u;
          gv[SET][k].y = (uint32_t)(u >> 32);
          continue;
        }
        const uint32_t e = (uint32_t)(((n * K + kk) * H + h) * W + w);
        gv[SET][k] = buffer_load16(gview, ok ? 2u * e : kOutside);
        if constexpr (ZG) {
          zv[SET][2 * k] = __builtin_bit_cast(f32x4, buffer_load16(zview, ok ? 4u * e : kOutside));
          zv[SET][2 * k + 1] =
              __builtin_bit_cast(f32x4, buffer_load16(zview, ok ? 4u * e + 16u : kOutside));
        }
      }
#pragma unroll
      for (int k = 0; k < XN; ++k) {
        const int it = tid + k * NT;
        const int q = it % XQ;
        int t = it / XQ;
        const int rr = t % HR;
        t /= HR;
        const int img = t % IMGS;
        const int cl = t / IMGS;
        const int n = o.n0 + img, h = o.h0 + rr - 1, w = o.w0 + 8 * q;
        const bool ok = (XI % NT == 0 || it < XI) && n < N && cl < cn && h >= 0 && h < H && w < W;
        if constexpr (XUP) {
          // 8 pixels of the upsampled row: 4 source elements at (h/2, w/2)
          const uint64_t u = buffer_load8(
              xview, ok ? 2u * (uint32_t)(((n * cs + cl0 + cl) * (H >> 1) + (h >> 1)) * (W >> 1) +
                                          (w >> 1))
                        : kOutside);
          xv[SET][k].x = (uint32_t)u;
          xv[SET][k].y = (uint32_t)(u >> 32);
          continue;
        }
        xv[SET][k] = buffer_load16(
            xview, ok ? 2u * (uint32_t)(((n * cs + cl0 + cl) * H + h) * W + w) : kOutside);
        if constexpr (PRO) {
          // (one x tensor: channel c0 + cl)
          const uint32_t po = ok ? 4u * (uint32_t)(n * C + c0 + cl) : kOutside;
          pxs[SET][k] = __builtin_bit_cast(float, buffer_load4(psview, po));
          pxt[SET][k] = __builtin_bit_cast(float, buffer_load4(ptview, po));
        }
      }
#pragma unroll
      for (int k = 0; k < HN; ++k) {
        if (!halo_loads) break;
        const int it = tid + k * NT;
        const int side = it & 1;
        int t = it >> 1;
        const int rr = t % HR;
        t /= HR;
        const int img = t % IMGS;
        const int cl = t / IMGS;
        const int n = o.n0 + img, h = o.h0 + rr - 1;
        const int w = o.w0 + (side ? TW : -1);
        const bool ok = (HI_ % NT == 0 || it < HI_) && n < N && cl < cn && h >= 0 && h < H &&
                        w >= 0 && w < W;
        const uint32_t e = XUP ? (uint32_t)(((n * cs + cl0 + cl) * (H >> 1) + (h >> 1)) * (W >> 1) +
                                            (w >> 1))
                               : (uint32_t)(((n * cs + cl0 + cl) * H + h) * W + w);
        xh[SET][k] = (uint16_t)buffer_load2(xview, ok ? 2u * e : kOutside);
        if constexpr (PRO) {
          const uint32_t po = ok ? 4u * (uint32_t)(n * C + c0 + cl) : kOutside;
          phs[SET][k] = __builtin_bit_cast(float, buffer_load4(psview, po));
          pht[SET][k] = __builtin_bit_cast(float, buffer_load4(ptview, po));
        }
      }
    }
  };

  auto store_tiles = [&](auto set_c, int chunk, int buf) __attribute__((always_inline)) {
    constexpr int SET = decltype(set_c)::value;
    uint16_t* gs = gs_buf[buf];
    uint16_t* xs = xs_buf[buf];
    if constexpr (VEC) {
#pragma unroll
      for (int k = 0; k < XN; ++k) {
        const int it = tid + k * NT;
        if (XI % NT == 0 || it < XI) {
          const int q = it % XQ;
          const int t = it / XQ;  // (cl * IMGS + img) * HR + rr
          const int cl = t / (IMGS * HR);
          u32x4 v = xv[SET][k];
          if constexpr (XUP) v = bf16x4_repeat2(v.x, v.y);
          if constexpr (PRO) {
            // a = SiLU(x * scale + shift), rounded to bfloat16 (items outside
            // the image load x = scale = shift = 0: the zero padding of a)
            v.x = silu_affine_bf16x2<false>(v.x, pxs[SET][k], pxt[SET][k]);
            v.y = silu_affine_bf16x2<false>(v.y, pxs[SET][k], pxt[SET][k]);
            v.z = silu_affine_bf16x2<false>(v.z, pxs[SET][k], pxt[SET][k]);
            v.w = silu_affine_bf16x2<false>(v.w, pxs[SET][k], pxt[SET][k]);
          }
          *reinterpret_cast<u32x4*>(&xs[cl * PLX + (t % (IMGS * HR)) * RSX + 8 + 8 * q]) = v;
        }
      }
#pragma unroll
      for (int k = 0; k < HN; ++k) {
        const int it = tid + k * NT;
        if (HI_ % NT == 0 || it < HI_) {
          const int side = it & 1;
          const int t = it >> 1;
          const int cl = t / (IMGS * HR);
          uint16_t v = xh[SET][k];
          if constexpr (PRO) {
            if (halo_loads) v = (uint16_t)silu_affine_bf16<false>(v, phs[SET][k], pht[SET][k]);
          }
          xs[cl * PLX + (t % (IMGS * HR)) * RSX + 8 + (side ? TW : -1)] = v;
        }
      }
      if constexpr (ZG) {
        // g = gy * act'(z), rounded to bfloat16, in place (after the x
        // stores have freed their registers; constant indices only)
        static_assert(GN <= 2, "ZG staging handles up to two g items per thread");
        auto mul = [&](auto kc) {
          constexpr int k = decltype(kc)::value;
          const f32x4 za = zv[SET][2 * k], zb = zv[SET][2 * k + 1];
          u32x4 v = gv[SET][k];
          v.x = act_grad_bf16x2<false>(v.x, za.x, za.y, act);
          v.y = act_grad_bf16x2<false>(v.y, za.z, za.w, act);
          v.z = act_grad_bf16x2<false>(v.z, zb.x, zb.y, act);
          v.w = act_grad_bf16x2<false>(v.w, zb.z, zb.w, act);
          gv[SET][k] = v;
        };
        mul(std::integral_constant<int, 0>{});
        if constexpr (GN > 1) mul(std::integral_constant<int, 1>{});
      }
#pragma unroll
      for (int k = 0; k < GN; ++k) {
        const int it = tid + k * NT;
        if (GI % NT == 0 || it < GI) {
          const int q = it % XQ;
          const int t = it / XQ;  // (kl * IMGS + img) * TH + row
          const int kl = t / (IMGS * TH);
          const u32x4 v = GZI ? bf16x4_zero_insert(gv[SET][k].x, gv[SET][k].y) : gv[SET][k];
          *reinterpret_cast<u32x4*>(&gs[kl * GSB + (t % (IMGS * TH)) * TW + 8 * q]) = v;
        }
      }
    } else {
      // Scalar path (ragged shapes): 16-bit loads straight into LDS.
      const BlockOrigin o = block_origin<TW, TH, IMGS>(chunk, tiles_w, tiles_h);
      constexpr int GS_ = 64 * P;
#pragma unroll 4
      for (int k = 0; k < (GS_ + NT - 1) / NT; ++k) {
        const int it = tid + k * NT;
        if (GS_ % NT == 0 || it < GS_) {
          const int col = it % TW;
          int t = it / TW;
          const int row = t % TH;
          t /= TH;
          const int img = t % IMGS;
          const int kl = t / IMGS;
          const int n = o.n0 + img, kk = k0 + kl, h = o.h0 + row, w = o.w0 + col;
          uint16_t v = 0;
          // (a zero-inserted g is an H/2 x W/2 tensor read at (h / 2, w / 2)
          // for even (h, w), zero elsewhere)
          const bool zi = ggeo == kGeoZero;
          if (n < N && kk < K && h < H && w < W && (!zi || ((h | w) & 1) == 0)) {
            const long e = zi ? ((long)n * K + kk) * (long)(H >> 1) * (W >> 1) +
                                    (long)(h >> 1) * (W >> 1) + (w >> 1)
                              : ((long)n * K + kk) * HW + (long)h * W + w;
            v = g[e];
            if constexpr (ZG) v = (uint16_t)act_grad_bf16<false>(v, zsrc[e], act);
          }
          gs[kl * GSB + it % P] = v;
        }
      }
      constexpr int XS_ = 64 * IMGS * HR * (TW + 2);
#pragma unroll 4
      for (int k = 0; k < (XS_ + NT - 1) / NT; ++k) {
        const int it = tid + k * NT;
        if (XS_ % NT == 0 || it < XS_) {
          const int cc = it % (TW + 2) - 1;
          int t = it / (TW + 2);
          const int rr = t % HR;
          t /= HR;
          const int img = t % IMGS;
          const int cl = t / IMGS;
          const int n = o.n0 + img, h = o.h0 + rr - 1, w = o.w0 + cc;
          uint16_t v = 0;
          if (n < N && cl < cn && h >= 0 && h < H && w >= 0 && w < W) {
            // (an upsampled x is an H/2 x W/2 tensor read at (h / 2, w / 2))
            v = xgeo == kGeoUp ? xsrc[((long)n * cs + cl0 + cl) * (long)(H >> 1) * (W >> 1) +
                                      (long)(h >> 1) * (W >> 1) + (w >> 1)]
                               : xsrc[((long)n * cs + cl0 + cl) * HW + (long)h * W + w];
            if constexpr (PRO) {
              const long pc = (long)n * C + c0 + cl;
              v = (uint16_t)silu_affine_bf16<false>(v, pscale[pc], pshift[pc]);
            }
          }
          xs[cl * PLX + (img * HR + rr) * RSX + 8 + cc] = v;
        }
      }
    }
  };

  f32x16 acc[3];
#pragma unroll
  for (int t = 0; t < 3; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[t][v] = 0.f;
  float dbsum = 0.f;

  const int chunk_begin = slice * per_split;
  const int chunk_end = min(nchunks, chunk_begin + per_split);
  const int goff = (kb * 32 + l32) * GSB;
  const int xoff = (cb * 32 + l32) * PLX + r * RSX + 8;

  // Operands of one step: g word, x word, and the x dwords on either side.
  u32x4 ga[2], xc[2];
  uint32_t xp[2], xn[2];
  auto read_step = [&](const uint16_t* gs, const uint16_t* xs, int rb, int ks) {
    const int p = ks * 16 + hi * 8;  // first of this lane's 8 pixels (one row)
    const int img = p / (TH * TW), row = (p / TW) % TH, col = p % TW;
    ga[rb] = *reinterpret_cast<const u32x4*>(&gs[goff + p]);
    const int xb = xoff + (img * HR + row) * RSX + col;
    xc[rb] = *reinterpret_cast<const u32x4*>(&xs[xb]);
    xp[rb] = *reinterpret_cast<const uint32_t*>(&xs[xb - 2]);
    xn[rb] = *reinterpret_cast<const uint32_t*>(&xs[xb + 8]);
  };

  // Chunk i is computed from LDS buffer i & 1.  After its second MFMA step
  // the register set holding chunk i + 1 is written to the other buffer (last
  // read in chunk i - 1, before the barrier that ended it) and the global
  // loads of chunk i + 3 are issued into it, so staging runs beside the MFMAs
  // of waves that are still computing.  One barrier per chunk.
  constexpr int kStoreStep = 1;
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, NSET - 1>;
  if (chunk_begin < chunk_end) {
    load_tiles(Set0{}, chunk_begin);
    store_tiles(Set0{}, chunk_begin, 0);
    if (chunk_begin + 1 < chunk_end) load_tiles(Set1{}, chunk_begin + 1);
    if (NSET == 2 && chunk_begin + 2 < chunk_end) load_tiles(Set0{}, chunk_begin + 2);
    __syncthreads();
  }
  // One chunk; SET is the register set that holds chunk + 1.
  auto run_chunk = [&](auto set_c, int chunk) __attribute__((always_inline)) {
    const int cur = (chunk - chunk_begin) & 1;
    const uint16_t* gs = gs_buf[cur];
    const uint16_t* xs = xs_buf[cur];
    // Step ks (16 pixels) reads its operands while step ks-1's MFMAs run.
    read_step(gs, xs, 0, 0);
#pragma unroll
    for (int ks = 0; ks < P / 16; ++ks) {
      const int cb_ = ks & 1;
      if (ks + 1 < P / 16) read_step(gs, xs, cb_ ^ 1, ks + 1);
      __builtin_amdgcn_sched_barrier(0);
      const u32x4 c = xc[cb_];
      u32x4 left, right;  // columns col-1 .. col+6 and col+1 .. col+8
      left.x = __builtin_amdgcn_alignbit(c.x, xp[cb_], 16);
      left.y = __builtin_amdgcn_alignbit(c.y, c.x, 16);
      left.z = __builtin_amdgcn_alignbit(c.z, c.y, 16);
      left.w = __builtin_amdgcn_alignbit(c.w, c.z, 16);
      right.x = left.y;
      right.y = left.z;
      right.z = left.w;
      right.w = __builtin_amdgcn_alignbit(xn[cb_], c.w, 16);
      acc[0] = mfma_32x32x16_bf16(ga[cb_], left, acc[0]);
      acc[1] = mfma_32x32x16_bf16(ga[cb_], c, acc[1]);
      acc[2] = mfma_32x32x16_bf16(ga[cb_], right, acc[2]);
      if (ks == kStoreStep && chunk + 1 < chunk_end) {
        __builtin_amdgcn_sched_barrier(0);
        store_tiles(set_c, chunk + 1, cur ^ 1);
        if (chunk + 1 + NSET < chunk_end) load_tiles(set_c, chunk + 1 + NSET);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (do_db && tid < 256) {
      const int kl = tid >> 2, part = tid & 3;
#pragma unroll
      for (int i = 0; i < P / 4; ++i) dbsum += bf16_to_f32(gs[kl * GSB + part + 4 * i]);
    }
    __syncthreads();
  };
  for (int chunk = chunk_begin; chunk < chunk_end; chunk += 2) {
    run_chunk(Set1{}, chunk);
    if (chunk + 1 < chunk_end) run_chunk(Set0{}, chunk + 1);
  }

  const int c = c0 + cb * 32 + l32;
  const bool c_ok = cb * 32 + l32 < cn;
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    const int t = r * 3 + s;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int k = k0 + kb * 32 + acc_row(v, hi);
      if (k < K && c_ok) {
        if (slice_stride)
          out[(long)slice * slice_stride + ((long)t * K + k) * C + c] = acc[s][v];
        else
          out[((long)k * C + c) * 9 + t] = acc[s][v];
      }
    }
  }
  if (do_db && tid < 256) {
    dbsum += __shfl_xor(dbsum, 1);
    dbsum += __shfl_xor(dbsum, 2);
    const int kl = tid >> 2;
    if ((tid & 3) == 0 && k0 + kl < K) out_db[(long)slice * K + k0 + kl] = dbsum;
  }
}

template <int TW, int TH, int IMGS, bool ZG, bool PRO>
static void launch_wgrad_bf16_geom(const Plan& pl, bool vec, Split<const uint16_t> x,
                                   const uint16_t* g, float* out, float* out_db,
                                   long slice_stride, int N, int C, int K, int H, int W,
                                   const ActArgs& a, hipStream_t stream) {
  dim3 grid(pl.grid_x, 1, 1), block(pl.threads, 1, 1);
  const int tiles_c = (x.c0 + 63) / 64 + (C - x.c0 + 63) / 64;
  const long hw2 = (long)H * W * 2;
  // resampling geometry: x upsampled (read at (h/2, w/2)) or g zero-inserted
  const int xgeo = a.up2 ? kGeoUp : kGeoPlain, ggeo = a.s2 ? kGeoZero : kGeoPlain;
  if constexpr (!ZG && !PRO) {
    if (vec && (a.up2 || a.s2)) {
      // the resampled tensor is N x (C or K) x H/2 x W/2
      const long q2 = hw2 / 4;
      if (a.up2)
        hipLaunchKernelGGL((wgrad_bf16_kernel<TW, TH, IMGS, true, false, false, kGeoUp>), grid,
                           block, 0, stream, x.p0, x.p1, x.c0, g, out, out_db, N, C, K, H, W,
                           pl.tiles_w, pl.tiles_h, pl.nchunks, pl.chunks_per_split, slice_stride,
                           pl.split, tiles_c, (K + 63) / 64, (uint32_t)(N * C * q2), 0u,
                           (uint32_t)(N * K * hw2), a.act, a.zsrc, a.pscale, a.pshift,
                           (int)kGeoPlain, (int)kGeoPlain);
      else
        hipLaunchKernelGGL((wgrad_bf16_kernel<TW, TH, IMGS, true, false, false, kGeoZero>), grid,
                           block, 0, stream, x.p0, x.p1, x.c0, g, out, out_db, N, C, K, H, W,
                           pl.tiles_w, pl.tiles_h, pl.nchunks, pl.chunks_per_split, slice_stride,
                           pl.split, tiles_c, (K + 63) / 64, (uint32_t)(N * C * hw2), 0u,
                           (uint32_t)(N * K * q2), a.act, a.zsrc, a.pscale, a.pshift,
                           (int)kGeoPlain, (int)kGeoPlain);
      return;
    }
  }
  if (vec)
    hipLaunchKernelGGL((wgrad_bf16_kernel<TW, TH, IMGS, true, ZG, PRO>), grid, block, 0, stream,
                       x.p0, x.p1, x.c0, g, out, out_db, N, C, K, H, W, pl.tiles_w, pl.tiles_h,
                       pl.nchunks, pl.chunks_per_split, slice_stride, pl.split, tiles_c,
                       (K + 63) / 64, (uint32_t)(N * x.c0 * hw2),
                       (uint32_t)(N * (C - x.c0) * hw2), (uint32_t)(N * K * hw2), a.act, a.zsrc,
                       a.pscale, a.pshift, (int)kGeoPlain, (int)kGeoPlain);
  else
    hipLaunchKernelGGL((wgrad_bf16_kernel<TW, TH, IMGS, false, ZG, PRO>), grid, block, 0, stream,
                       x.p0, x.p1, x.c0, g, out, out_db, N, C, K, H, W, pl.tiles_w, pl.tiles_h,
                       pl.nchunks, pl.chunks_per_split, slice_stride, pl.split, tiles_c,
                       (K + 63) / 64, 0u, 0u, 0u, a.act, a.zsrc, a.pscale, a.pshift, xgeo, ggeo);
}

bool launch_wgrad_bf16(const Plan& pl, bool vec, Split<const uint16_t> x, const uint16_t* g,
                       float* dw, float* db, float* ws, int N, int C, int K, int H, int W,
                       const ActArgs& a, hipStream_t stream) {
  if (pl.threads != 768) return false;
  // the prologue needs one x tensor and does not combine with a fused
  // activation gradient
  if (a.pscale != nullptr && (a.zsrc != nullptr || x.c0 != C)) return false;
  // resampling (the stride-1 kernel over the full-resolution grid): one x
  // tensor, no fusion, even sizes
  if ((a.up2 || a.s2) && (x.c0 != C || a.zsrc != nullptr || a.pscale != nullptr || (H & 1) ||
                          (W & 1)))
    return false;
  const long n_dw = (long)K * C * 9;
  float* out = pl.split > 1 ? ws : dw;
  float* out_db = db == nullptr ? nullptr : (pl.split > 1 ? ws + (long)pl.split * n_dw : db);
  const long stride = pl.split > 1 ? n_dw : 0;
  bool found = false;
#define CONV3X3_X(TW_, TH_, IMGS_)                                                          \
  if (!found && pl.tw == TW_ && pl.th == TH_ && pl.imgs == IMGS_) {                         \
    if (a.zsrc)                                                                             \
      launch_wgrad_bf16_geom<TW_, TH_, IMGS_, true, false>(pl, vec, x, g, out, out_db, stride, \
                                                           N, C, K, H, W, a, stream);          \
    else if (a.pscale)                                                                        \
      launch_wgrad_bf16_geom<TW_, TH_, IMGS_, false, true>(pl, vec, x, g, out, out_db, stride, \
                                                           N, C, K, H, W, a, stream);          \
    else                                                                                      \
      launch_wgrad_bf16_geom<TW_, TH_, IMGS_, false, false>(pl, vec, x, g, out, out_db,        \
                                                            stride, N, C, K, H, W, a, stream); \
    found = true;                                                                           \
  }
  CONV3X3_WGRAD_BF16_CONFIGS(CONV3X3_X)
#undef CONV3X3_X
  if (!found) return false;
  if (pl.split > 1) launch_wgrad_reduce(ws, dw, db, pl.split, C, K, stream);
  return true;
}

}  // namespace conv3x3
