// Backward-weight and bias gradient of the 3x3 convolution, float32, gfx950.
//
//   dw[k,c,r,s] = sum_{n,h,w} g[n,k,h,w] * x[n,c,h+r-1,w+s-1]
//   db[k]       = sum_{n,h,w} g[n,k,h,w]
//
// A GEMM with rows k, columns (c, tap) and a reduction over pixels -- the
// contiguous axis of both NCHW operands.  A workgroup of 12 wave64s owns
// 64 k x 64 c x 9 taps: wave w takes the 32 x 32 block (kb, cb) and kernel
// row r = w % 3, i.e. three 32x32 accumulators (s = 0, 1, 2) that share the
// g operand.  Three waves per SIMD keep the MFMA pipe fed while others wait
// on LDS.  The workgroup walks one slice of the pixel reduction, 64 pixels
// (an IMGS x TH x TW block) per LDS fill: g for those pixels and x for the
// same block plus its one-pixel halo.  MFMA 32x32x2 f32: the two reduction
// elements of a step are two horizontally adjacent pixels.  Each slice writes
// its partial sums, tap-major ([tap][k][c], so the stores are coalesced),
// and -- in the workgroups of the first channel tile -- the partial db,
// reduced across lanes with fixed-order cross-lane adds, to its own
// workspace slot; wgrad_reduce_kernel adds the slots in a fixed order.  No
// atomics anywhere: results are bitwise reproducible.
//
// x may be the channel concatenation of two tensors (a UNet's up-path input
// [upsampled ; skip]): channels [0, cx0) from x and [cx0, C) from x1.  Each
// 64-channel tile lies inside one of them (a tensor's ragged last tile is
// zero-padded), so the choice is uniform per workgroup.
#include "activation.hpp"
#include "common.hpp"
#include "launch.hpp"
#include "lds_layout.hpp"
#include "tile_configs.hpp"

namespace conv3x3 {

// UP2: x is upsampled 2x by nearest neighbour as it is staged (H, W are the
// upsampled sizes, g's; x is H/2 x W/2).  S2 (a stride-2 convolution): H, W
// are x's, g is H/2 x W/2 and the chunks tile g's pixels; chunk pixel
// (ho, wo) pairs with x at (2 ho + r - 1, 2 wo + s - 1).
template <int TW, int TH, int IMGS, bool VEC, bool UP2 = false, bool S2 = false>
__global__ __launch_bounds__(768) void wgrad_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ x1, int cx0,
    const float* __restrict__ g, float* __restrict__ out, float* __restrict__ out_db, int N,
    int C, int K, int H, int W, int tiles_w, int tiles_h, int nchunks, int per_split,
    long slice_stride, int split, int tiles_c, int tiles_k, uint32_t x_bytes, uint32_t x1_bytes,
    uint32_t g_bytes, int act, const float* __restrict__ zsrc, const float* __restrict__ pscale,
    const float* __restrict__ pshift) {
  constexpr int P = IMGS * TH * TW;
  static_assert(P == 64, "pixel chunk must hold 64 pixels");
  static_assert(!(UP2 && S2), "upsampling or stride 2");
  constexpr int GS = wgrad_f32_gstride(IMGS, TH, TW);
  constexpr int RSW = S2 ? wgrad_f32_s2_rs(TW) : wgrad_f32_rs(TW);
  constexpr int PLW = S2 ? wgrad_f32_s2_plane(IMGS, TH, TW) : wgrad_f32_plane(IMGS, TH, TW);
  constexpr int HR = S2 ? 2 * TH + 1 : TH + 2;  // staged x rows per image

  // Two LDS buffers: chunk i is read from one while chunk i + 1 is written
  // into the other.  S2: one (the next chunk is written after a barrier).
  constexpr int NBUF = S2 ? 1 : 2;
  __shared__ float gs_buf[NBUF][64 * GS];
  __shared__ float xs_buf[NBUF][64 * PLW];

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
  // channels), channel c0 of dw
  const int ct = tile % tiles_c, nct0 = (cx0 + 63) / 64;
  const bool xseg = ct >= nct0;
  const int cl0 = (ct - (xseg ? nct0 : 0)) * 64;
  const int cs = xseg ? C - cx0 : cx0;
  const int c0 = (xseg ? cx0 : 0) + cl0;
  const int cn = min(64, cs - cl0);
  const float* const xp = xseg ? x1 : x;
  const int k0 = (tile / tiles_c) * 64;
  const long HW = (long)H * W;
  const int Hs = UP2 ? H / 2 : H, Ws = UP2 ? W / 2 : W;  // x's rows and columns
  const int Hg = S2 ? H / 2 : H, Wg = S2 ? W / 2 : W;    // g's rows and columns (the chunk grid)
  const bool do_db = out_db != nullptr && tile % tiles_c == 0;

  // g tile: 64 k x P pixels.  x tile: 64 c x IMGS x HR rows x (TW + 2)
  // columns; S2: 2 TW + 1 columns, of which the vector items cover the 2 TW
  // from 2 w0 and the halo item the left one (2 w0 - 1).
  constexpr int XQ = TW / 4;
  constexpr int XQX = S2 ? TW / 2 : TW / 4;  // vector items per staged x row
  constexpr int GV_ITEMS = 64 * IMGS * TH * XQ;
  constexpr int NT = 768;
  constexpr int GV_N = (GV_ITEMS + NT - 1) / NT;
  constexpr int XV_ITEMS = 64 * IMGS * HR * XQX;
  constexpr int XV_N = (XV_ITEMS + NT - 1) / NT;
  constexpr int XH_ITEMS = 64 * IMGS * HR * (S2 ? 1 : 2);
  constexpr int XH_N = (XH_ITEMS + NT - 1) / NT;
  constexpr int GS_ITEMS = 64 * P;
  constexpr int GS_N = (GS_ITEMS + NT - 1) / NT;
  constexpr int XCOLS = S2 ? 2 * TW + 1 : TW + 2;
  constexpr int XS_ITEMS = 64 * IMGS * HR * XCOLS;
  constexpr int XS_N = (XS_ITEMS + NT - 1) / NT;

  f32x4 gv[VEC ? GV_N : 1];
  // Fused activation: z at the positions of g; g is multiplied by act'(z)
  // when it is written to LDS.
  // (neither this nor the prologue below goes with stride 2, whose larger
  // x items need the registers)
  const bool zs = !S2 && zsrc != nullptr;
  f32x4 zv[VEC && !S2 ? GV_N : 1];
  f32x4 xv[VEC ? XV_N : 1];
  float xf[VEC ? XH_N : 1];
  // With a single tile across the width both halo columns are padding: they
  // stay zero and are not loaded.
  const bool halo_loads = tiles_w > 1;
#pragma unroll
  for (int k = 0; k < (VEC ? XH_N : 1); ++k) xf[k] = 0.f;
  // Input prologue: each staged x value becomes SiLU(x * scale[n, c] +
  // shift[n, c]); items outside the image or the channels load x = scale =
  // shift = 0 and stage SiLU(0) = 0, so the padding stays zero.
  const bool pro = !S2 && pscale != nullptr;
  constexpr int PV_N = VEC && !S2 ? XV_N : 1, PH_N = VEC && !S2 ? XH_N : 1;
  float psv[PV_N], ptv[PV_N], psh[PH_N], pth[PH_N];
#pragma unroll
  for (int k = 0; k < PH_N; ++k) psh[k] = pth[k] = 0.f;
  const uint32_t pbytes = pro ? 4u * (uint32_t)(N * C) : 0u;
  const __amdgpu_buffer_rsrc_t psview = buffer_view(pscale, pbytes);
  const __amdgpu_buffer_rsrc_t ptview = buffer_view(pshift, pbytes);

  // Vector path: buffer views; an item outside the tensors or the image
  // reads zero through an offset past the view (32-bit offset arithmetic,
  // no branches).
  const __amdgpu_buffer_rsrc_t gview = buffer_view(g, g_bytes);
  const __amdgpu_buffer_rsrc_t zview = buffer_view(zsrc, zs ? g_bytes : 0u);
  const __amdgpu_buffer_rsrc_t xview = buffer_view(xp, xseg ? x1_bytes : x_bytes);
  auto load_tiles = [&](int chunk) {
    if constexpr (VEC) {
      const BlockOrigin o = block_origin<TW, TH, IMGS>(chunk, tiles_w, tiles_h);
#pragma unroll
      for (int k = 0; k < GV_N; ++k) {
        const int it = tid + k * NT;
        const int q = it % XQ;
        int t = it / XQ;
        const int row = t % TH;
        t /= TH;
        const int img = t % IMGS;
        const int kl = t / IMGS;
        const int n = o.n0 + img, kk = k0 + kl, h = o.h0 + row, w = o.w0 + 4 * q;
        const bool ok =
            (GV_ITEMS % NT == 0 || it < GV_ITEMS) && n < N && kk < K && h < Hg && w < Wg;
        const uint32_t off = ok ? 4u * (uint32_t)(((n * K + kk) * Hg + h) * Wg + w) : kOutside;
        gv[k] = __builtin_bit_cast(f32x4, buffer_load16(gview, off));
        if (zs) zv[k] = __builtin_bit_cast(f32x4, buffer_load16(zview, off));
      }
#pragma unroll
      for (int k = 0; k < XV_N; ++k) {
        const int it = tid + k * NT;
        const int q = it % XQX;
        int t = it / XQX;
        const int rr = t % HR;
        t /= HR;
        const int img = t % IMGS;
        const int cl = t / IMGS;
        // x row and first column of the item (S2: input row 2 h0 - 1 + rr,
        // columns 2 w0 + 4q ..)
        const int n = o.n0 + img;
        const int h = S2 ? 2 * o.h0 + rr - 1 : o.h0 + rr - 1;
        const int w = S2 ? 2 * o.w0 + 4 * q : o.w0 + 4 * q;
        const bool ok = (XV_ITEMS % NT == 0 || it < XV_ITEMS) && n < N && cl < cn && h >= 0 &&
                        h < H && w < W;
        if constexpr (UP2) {
          // four upsampled columns: two x values, each used twice
          float xa, xb;
          buffer_load_2f(xview,
                         ok ? 4u * (uint32_t)(((n * cs + cl0 + cl) * Hs + h / 2) * Ws + w / 2)
                            : kOutside,
                         xa, xb);
          xv[k] = f32x4{xa, xa, xb, xb};
        } else {
          xv[k] = __builtin_bit_cast(
              f32x4, buffer_load16(xview, ok ? 4u * (uint32_t)(((n * cs + cl0 + cl) * H + h) * W + w)
                                              : kOutside));
        }
        if (pro) {
          const uint32_t po = ok ? 4u * (uint32_t)(n * C + c0 + cl) : kOutside;
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
        const int cl = t / IMGS;
        const int n = o.n0 + img, h = S2 ? 2 * o.h0 + rr - 1 : o.h0 + rr - 1;
        const int w = S2 ? 2 * o.w0 - 1 : o.w0 + (side ? TW : -1);
        const bool ok = (XH_ITEMS % NT == 0 || it < XH_ITEMS) && n < N && cl < cn && h >= 0 &&
                        h < H && w >= 0 && w < W;
        xf[k] = __builtin_bit_cast(
            float, buffer_load4(xview, ok ? 4u * (uint32_t)(((n * cs + cl0 + cl) * Hs +
                                                             (UP2 ? h / 2 : h)) * Ws +
                                                            (UP2 ? w / 2 : w))
                                          : kOutside));
        if (pro) {
          const uint32_t po = ok ? 4u * (uint32_t)(n * C + c0 + cl) : kOutside;
          psh[k] = __builtin_bit_cast(float, buffer_load4(psview, po));
          pth[k] = __builtin_bit_cast(float, buffer_load4(ptview, po));
        }
      }
    }
  };

  // Vector path: global -> registers in load_tiles (one chunk ahead),
  // registers -> LDS here.  Scalar path: everything happens here.
  auto store_tiles = [&](int chunk, int buf) {
    float* gs = gs_buf[buf];
    float* xs = xs_buf[buf];
    if constexpr (VEC) {
#pragma unroll
      for (int k = 0; k < GV_N; ++k) {
        const int it = tid + k * NT;
        if (GV_ITEMS % NT != 0 && it >= GV_ITEMS) continue;
        const int q = it % XQ;
        const int t = it / XQ;  // (kl * IMGS + img) * TH + row
        const int kl = t / (IMGS * TH);
        const int p = (t % (IMGS * TH)) * TW + 4 * q;
        float* d = &gs[kl * GS + p];
        f32x4 v = gv[k];
        if (zs) {
          v.x *= act_slope(act, zv[k].x);
          v.y *= act_slope(act, zv[k].y);
          v.z *= act_slope(act, zv[k].z);
          v.w *= act_slope(act, zv[k].w);
        }
        d[0] = v.x;
        d[1] = v.y;
        d[2] = v.z;
        d[3] = v.w;
      }
#pragma unroll
      for (int k = 0; k < XV_N; ++k) {
        const int it = tid + k * NT;
        if (XV_ITEMS % NT == 0 || it < XV_ITEMS) {
          const int q = it % XQX;
          const int t = it / XQX;  // (cl * IMGS + img) * HR + rr
          const int cl = t / (IMGS * HR);
          float* d = &xs[cl * PLW + (t % (IMGS * HR)) * RSW + 1 + 4 * q];
          f32x4 v = xv[k];
          if (pro) {
            v.x = act_value(kActSilu, v.x * psv[k] + ptv[k]);
            v.y = act_value(kActSilu, v.y * psv[k] + ptv[k]);
            v.z = act_value(kActSilu, v.z * psv[k] + ptv[k]);
            v.w = act_value(kActSilu, v.w * psv[k] + ptv[k]);
          }
          d[0] = v.x;
          d[1] = v.y;
          d[2] = v.z;
          d[3] = v.w;
        }
      }
#pragma unroll
      for (int k = 0; k < XH_N; ++k) {
        const int it = tid + k * NT;
        if (XH_ITEMS % NT == 0 || it < XH_ITEMS) {
          const int side = S2 ? 0 : it & 1;
          const int t = S2 ? it : it >> 1;
          const int cl = t / (IMGS * HR);
          xs[cl * PLW + (t % (IMGS * HR)) * RSW + 1 + (side ? TW : -1)] =
              pro ? act_value(kActSilu, xf[k] * psh[k] + pth[k]) : xf[k];
        }
      }
    } else {
      // Scalar path (ragged shapes): global loads go straight to LDS.
      const BlockOrigin o = block_origin<TW, TH, IMGS>(chunk, tiles_w, tiles_h);
#pragma unroll 4
      for (int k = 0; k < GS_N; ++k) {
        const int it = tid + k * NT;
        if (GS_ITEMS % NT != 0 && it >= GS_ITEMS) continue;
        const int col = it % TW;
        int t = it / TW;
        const int row = t % TH;
        t /= TH;
        const int img = t % IMGS;
        const int kl = t / IMGS;
        const int n = o.n0 + img, kk = k0 + kl, h = o.h0 + row, w = o.w0 + col;
        float v = 0.f;
        if (n < N && kk < K && h < Hg && w < Wg) {
          const long e = ((long)n * K + kk) * Hg * Wg + (long)h * Wg + w;
          v = g[e];
          if (zs) v *= act_slope(act, zsrc[e]);
        }
        gs[kl * GS + it % P] = v;
      }
#pragma unroll 4
      for (int k = 0; k < XS_N; ++k) {
        const int it = tid + k * NT;
        if (XS_ITEMS % NT == 0 || it < XS_ITEMS) {
          const int cc = it % XCOLS - 1;
          int t = it / XCOLS;
          const int rr = t % HR;
          t /= HR;
          const int img = t % IMGS;
          const int cl = t / IMGS;
          const int n = o.n0 + img;
          const int h = S2 ? 2 * o.h0 + rr - 1 : o.h0 + rr - 1;
          const int w = S2 ? 2 * o.w0 + cc : o.w0 + cc;
          float v = 0.f;
          if (n < N && cl < cn && h >= 0 && h < H && w >= 0 && w < W) {
            v = UP2 ? xp[((long)n * cs + cl0 + cl) * Hs * Ws + (long)(h / 2) * Ws + w / 2]
                    : xp[((long)n * cs + cl0 + cl) * HW + (long)h * W + w];
            if (pro) {
              const long pc = (long)n * C + c0 + cl;
              v = act_value(kActSilu, v * pscale[pc] + pshift[pc]);
            }
          }
          xs[cl * PLW + (img * HR + rr) * RSW + 1 + cc] = v;
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
  const int goff = (kb * 32 + l32) * GS;
  const int xoff = (cb * 32 + l32) * PLW + r * RSW;

  float a[2], b[2][3];
  auto read_step = [&](const float* gs, const float* xs, int buf, int q2) {
    const int p = 2 * q2 + hi;
    const int img = p / (TH * TW), row = (p / TW) % TH, col = p % TW;
    a[buf] = gs[goff + p];
    // S2: x row 2 row + r and column 2 col + s of the staged tile
    const int xb = S2 ? xoff + (img * HR + 2 * row) * RSW + 2 * col
                      : xoff + (img * HR + row) * RSW + col;
#pragma unroll
    for (int s = 0; s < 3; ++s) b[buf][s] = xs[xb + s];
  };

  // Chunk i is computed from LDS buffer i & 1.  Partway through its MFMA
  // steps the registers holding chunk i + 1 are written to the other buffer
  // (last read in iteration i - 1, before the barrier that ended it) and the
  // global loads of chunk i + 2 are issued into them, so staging runs beside
  // the MFMAs of waves that are still computing.  One barrier per chunk.
  constexpr int kStoreStep = 2;
  if (chunk_begin < chunk_end) {
    load_tiles(chunk_begin);
    store_tiles(chunk_begin, 0);
    if (chunk_begin + 1 < chunk_end) load_tiles(chunk_begin + 1);
    __syncthreads();
  }
  for (int chunk = chunk_begin; chunk < chunk_end; ++chunk) {
    const int cur_buf = S2 ? 0 : (chunk - chunk_begin) & 1;
    const float* gs = gs_buf[cur_buf];
    const float* xs = xs_buf[cur_buf];
    // Step q2 (two pixels) reads its operands while step q2-1's MFMAs run.
    read_step(gs, xs, 0, 0);
#pragma unroll
    for (int q2 = 0; q2 < P / 2; ++q2) {
      const int cur = q2 & 1;
      if (q2 + 1 < P / 2) read_step(gs, xs, cur ^ 1, q2 + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < 3; ++s) acc[s] = mfma_32x32x2_f32(a[cur], b[cur][s], acc[s]);
      if (!S2 && q2 == kStoreStep && chunk + 1 < chunk_end) {
        __builtin_amdgcn_sched_barrier(0);
        store_tiles(chunk + 1, cur_buf ^ 1);
        if (chunk + 2 < chunk_end) load_tiles(chunk + 2);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (do_db && tid < 256) {
      const int kl = tid >> 2, part = tid & 3;
#pragma unroll
      for (int i = 0; i < P / 4; ++i) dbsum += gs[kl * GS + part + 4 * i];
    }
    __syncthreads();
    if (S2 && chunk + 1 < chunk_end) {
      // single buffer: the next chunk is written once every wave is done
      // with this one
      store_tiles(chunk + 1, 0);
      if (chunk + 2 < chunk_end) load_tiles(chunk + 2);
      __syncthreads();
    }
  }

  // Partial dw of this slice.  Split: tap-major [tap][k][c] slot at
  // out + slice * slice_stride (32 consecutive c per store).  No split: dw
  // itself, [k][c][tap].
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
    // Lanes 4j..4j+3 hold four interleaved partial sums of one k: add them
    // pairwise, (p0 + p1) + (p2 + p3), the same way every time.
    dbsum += __shfl_xor(dbsum, 1);
    dbsum += __shfl_xor(dbsum, 2);
    const int kl = tid >> 2;
    if ((tid & 3) == 0 && k0 + kl < K) out_db[(long)slice * K + k0 + kl] = dbsum;
  }
}

// Split-K epilogue.  Workspace: S tap-major partial slots [S][9][K][C],
// then S partial db rows [S][K].  Each workgroup owns 64 consecutive
// elements; wave q of 4 adds the slots of a fixed contiguous quarter of the
// slices in slice order, and wave 0 adds the four quarter sums as
// ((q0 + q1) + q2) + q3.  The order never changes, so the result is bitwise
// reproducible.  dw is written back in [k][c][tap] order.
__global__ __launch_bounds__(256) void wgrad_reduce_kernel(const float* __restrict__ ws,
                                                           float* __restrict__ dw,
                                                           float* __restrict__ db, int S,
                                                           int C, int K) {
  __shared__ float part[4][64];
  const long n_dw = (long)K * C * 9;
  const long total = n_dw + (db != nullptr ? K : 0);
  const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const long e = (long)blockIdx.x * 64 + lane;
  const int per = (S + 3) / 4;
  const int s0 = min(S, q * per), s1 = min(S, s0 + per);
  float sum = 0.f;
  if (e < total) {
    const float* base;
    long stride;
    if (e < n_dw) {
      base = ws + e;
      stride = n_dw;
    } else {
      base = ws + (long)S * n_dw + (e - n_dw);
      stride = K;
    }
    // Loads are issued eight slots at a time; the adds stay in slot order.
    int i = s0;
    for (; i + 8 <= s1; i += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = base[(long)(i + u) * stride];
#pragma unroll
      for (int u = 0; u < 8; ++u) sum += v[u];
    }
    for (; i < s1; ++i) sum += base[(long)i * stride];
  }
  part[q][lane] = sum;
  __syncthreads();
  if (q == 0 && e < total) {
    const float v = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
    if (e < n_dw) {
      const long t = e / ((long)K * C);
      const long kc = e % ((long)K * C);  // k * C + c
      dw[kc * 9 + t] = v;
    } else {
      db[e - n_dw] = v;
    }
  }
}

// The same epilogue with 128-bit loads and stores, for workspaces whose
// slots and db rows are 16-byte aligned ((K * C) % 4 == 0, K % 4 == 0 when
// db is wanted) and 16-byte aligned dw / db.  A workgroup of 9 waves owns 256
// consecutive (k, c) pairs kc0 .. kc0 + 255: wave t adds tap t's slot rows
// of them (4 pairs per lane, the slots in slice order), the 9 x 256 sums go
// through LDS, and the workgroup writes dw[kc0 * 9 .. (kc0 + 256) * 9) --
// one contiguous [k][c][tap] run -- with 128-bit stores.  Workgroups past the
// dw part add the db rows (256 per workgroup, wave 0).  The order never
// changes, so the result is bitwise reproducible.
__global__ __launch_bounds__(576) void wgrad_reduce4_kernel(const float* __restrict__ ws,
                                                            float* __restrict__ dw,
                                                            float* __restrict__ db, int S,
                                                            int C, int K) {
  __shared__ __attribute__((aligned(16))) float tr[9][256];
  const long KC = (long)K * C;
  const long n_dw = KC * 9;
  const long nblk = (KC + 255) / 256;
  const int lane = threadIdx.x & 63, t = threadIdx.x >> 6;
  auto slot_sum = [&](const float* base, long stride) {
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    // loads issued eight slots at a time; the adds stay in slot order
    int i = 0;
    for (; i + 8 <= S; i += 8) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const f32x4*>(base + (long)(i + u) * stride);
#pragma unroll
      for (int u = 0; u < 8; ++u) sum += v[u];
    }
    for (; i < S; ++i) sum += *reinterpret_cast<const f32x4*>(base + (long)i * stride);
    return sum;
  };
  if ((long)blockIdx.x >= nblk) {
    // db rows [S][K] after the dw slots (the whole workgroup takes this branch)
    const long k4 = ((long)blockIdx.x - nblk) * 256 + 4 * (long)threadIdx.x;
    if (t == 0 && k4 < K)
      *reinterpret_cast<f32x4*>(db + k4) = slot_sum(ws + (long)S * n_dw + k4, K);
    return;
  }
  const long kc0 = (long)blockIdx.x * 256;
  const long kc = kc0 + 4 * lane;
  f32x4 sum = {0.f, 0.f, 0.f, 0.f};
  if (kc < KC) sum = slot_sum(ws + (long)t * KC + kc, n_dw);  // (KC % 4 == 0: kc + 3 < KC)
  *reinterpret_cast<f32x4*>(&tr[t][4 * lane]) = sum;
  __syncthreads();
  const long nvalid = (KC - kc0 < 256 ? KC - kc0 : 256) * 9;
  const int o = 4 * threadIdx.x;  // 576 threads x 4 = 2304 = 256 x 9 outputs
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = tr[(o + j) % 9][(o + j) / 9];
  if (o + 3 < nvalid) {
    *reinterpret_cast<f32x4*>(dw + kc0 * 9 + o) = f32x4{v[0], v[1], v[2], v[3]};
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (o + j < nvalid) dw[kc0 * 9 + o + j] = v[j];
  }
}

template <int TW, int TH, int IMGS>
static void launch_wgrad_geom(const Plan& pl, bool vec, Split<const float> x, const float* g,
                              float* out, float* out_db, long slice_stride, int N, int C, int K,
                              int H, int W, const ActArgs& a, hipStream_t stream) {
  dim3 grid(pl.grid_x, 1, 1), block(pl.threads, 1, 1);
  const int tiles_c = (x.c0 + 63) / 64 + (C - x.c0 + 63) / 64;
  const long hw4 = (long)H * W * 4;
  const long xhw4 = a.up2 ? hw4 / 4 : hw4;  // x's plane bytes
  const uint32_t xb0 = vec ? (uint32_t)(N * x.c0 * xhw4) : 0u;
  const uint32_t xb1 = vec ? (uint32_t)(N * (C - x.c0) * xhw4) : 0u;
  const uint32_t gb = vec ? (uint32_t)(N * K * (a.s2 ? hw4 / 4 : hw4)) : 0u;
#define CONV3X3_L(VEC_, UP_, S2_)                                                                 \
  hipLaunchKernelGGL((wgrad_f32_kernel<TW, TH, IMGS, VEC_, UP_, S2_>), grid, block, 0, stream,     \
                     x.p0,                                                                        \
                     x.p1, x.c0, g, out, out_db, N, C, K, H, W, pl.tiles_w, pl.tiles_h,            \
                     pl.nchunks, pl.chunks_per_split, slice_stride, pl.split, tiles_c,             \
                     (K + 63) / 64, xb0, xb1, gb, a.act, a.zsrc, a.pscale, a.pshift)
  if (a.up2) {
    if (vec)
      CONV3X3_L(true, true, false);
    else
      CONV3X3_L(false, true, false);
  } else if (a.s2) {
    if (vec)
      CONV3X3_L(true, false, true);
    else
      CONV3X3_L(false, false, true);
  } else {
    if (vec)
      CONV3X3_L(true, false, false);
    else
      CONV3X3_L(false, false, false);
  }
#undef CONV3X3_L
}

bool launch_wgrad_f32(const Plan& pl, bool vec, Split<const float> x, const float* g, float* dw,
                      float* db, float* ws, int N, int C, int K, int H, int W, const ActArgs& a,
                      hipStream_t stream) {
  if (pl.threads != 768) return false;
  const long n_dw = (long)K * C * 9;
  float* out = pl.split > 1 ? ws : dw;
  float* out_db = db == nullptr ? nullptr : (pl.split > 1 ? ws + (long)pl.split * n_dw : db);
  const long stride = pl.split > 1 ? n_dw : 0;
  bool found = false;
#define CONV3X3_X(TW_, TH_, IMGS_)                                                           \
  if (!found && pl.tw == TW_ && pl.th == TH_ && pl.imgs == IMGS_) {                          \
    launch_wgrad_geom<TW_, TH_, IMGS_>(pl, vec, x, g, out, out_db, stride, N, C, K, H, W, a, \
                                       stream);                                              \
    found = true;                                                                            \
  }
  CONV3X3_WGRAD_F32_CONFIGS(CONV3X3_X)
#undef CONV3X3_X
  if (!found) return false;
  if (pl.split > 1) launch_wgrad_reduce(ws, dw, db, pl.split, C, K, stream);
  return true;
}

void launch_wgrad_reduce(const float* ws, float* dw, float* db, int split, int C, int K,
                         hipStream_t stream) {
  const long total = (long)K * C * 9 + (db ? K : 0);
  const bool vec4 = ((long)K * C) % 4 == 0 && (db == nullptr || K % 4 == 0) &&
                    (reinterpret_cast<uintptr_t>(ws) & 15) == 0 &&
                    (reinterpret_cast<uintptr_t>(dw) & 15) == 0 &&
                    (reinterpret_cast<uintptr_t>(db) & 15) == 0;
  // The 9-wave kernel gives each lane a chain of S slot loads over 256 (k, c)
  // pairs per workgroup: with many slices and few workgroups (64 -> 64
  // channels: 256 slices, 16 workgroups) it is latency-bound (23.8 us
  // against 7.2 us for the 4-wave kernel, which spreads the slices over four
  // waves and 64 outputs per workgroup).
  const long KC = (long)K * C;
  const bool deep = split > 64 && (KC + 255) / 256 < 128;
  if (vec4 && !deep) {
    dim3 grid((unsigned)((KC + 255) / 256 + (db ? (K + 255) / 256 : 0))), block(576);
    hipLaunchKernelGGL(wgrad_reduce4_kernel, grid, block, 0, stream, ws, dw, db, split, C, K);
  } else {
    dim3 grid((unsigned)((total + 63) / 64)), block(256);
    hipLaunchKernelGGL(wgrad_reduce_kernel, grid, block, 0, stream, ws, dw, db, split, C, K);
  }
}

}  // namespace conv3x3
