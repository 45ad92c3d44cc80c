// Backward-weight and bias gradient of the 3x3 convolution, float32, gfx950.
//
//   dw[k,c,r,s] = sum_{n,h,w} g[n,k,h,w] * x[n,c,h+r-1,w+s-1]
//   db[k]       = sum_{n,h,w} g[n,k,h,w]
//
// A GEMM with rows k, columns (c, tap) and a reduction over pixels -- the
// contiguous axis of both NCHW operands.  A workgroup (4 wave64s) owns
// 64 k x 64 c x 9 taps (each wave 32 k x 32 c x 9 taps, nine 32x32
// accumulators that share the g operand) and walks one slice of the pixel
// reduction, 64 pixels (an IMGS x TH x TW block) per LDS fill: g for those
// pixels and x for the same block plus its one-pixel halo.  MFMA 32x32x2
// f32: the two reduction elements of a step are two horizontally adjacent
// pixels.  Each slice writes its partial sums (and, in the workgroups of the
// first channel tile, the partial db, reduced across lanes with fixed-order
// cross-lane adds) to its own workspace slot; wgrad_reduce_kernel then adds
// the slots in slice order.  No atomics anywhere: results are bitwise
// reproducible.
#include "common.hpp"
#include "launch.hpp"
#include "lds_layout.hpp"

namespace conv3x3 {

template <int TW, int TH, int IMGS, bool VEC>
__global__ __launch_bounds__(256, 1) void wgrad_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ g, float* __restrict__ out,
    float* __restrict__ out_db, int N, int C, int K, int H, int W, int tiles_w, int tiles_h,
    int nchunks, int per_split, long slice_stride) {
  constexpr int P = IMGS * TH * TW;
  static_assert(P == 64, "pixel chunk must hold 64 pixels");
  constexpr int GS = wgrad_f32_gstride(IMGS, TH, TW);
  constexpr int RSW = wgrad_f32_rs(TW);
  constexpr int PLW = wgrad_f32_plane(IMGS, TH, TW);
  constexpr int HR = TH + 2;

  __shared__ float gs[64 * GS];
  __shared__ float xs[64 * PLW];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int wk = wave & 1, wc = wave >> 1;
  const int slice = blockIdx.x;
  const int c0 = blockIdx.y * 64;
  const int k0 = blockIdx.z * 64;
  const long HW = (long)H * W;
  const bool do_db = out_db != nullptr && blockIdx.y == 0;

  // g tile: 64 k x P pixels.  x tile: 64 c x IMGS x HR rows x (TW + 2) columns.
  constexpr int XQ = TW / 4;
  constexpr int GV_ITEMS = 64 * IMGS * TH * XQ;
  constexpr int GV_N = GV_ITEMS / 256;
  constexpr int XV_ITEMS = 64 * IMGS * HR * XQ;
  constexpr int XV_N = (XV_ITEMS + 255) / 256;
  constexpr int XH_ITEMS = 64 * IMGS * HR * 2;
  constexpr int XH_N = (XH_ITEMS + 255) / 256;
  constexpr int GS_ITEMS = 64 * P;
  constexpr int GS_N = GS_ITEMS / 256;
  constexpr int XS_ITEMS = 64 * IMGS * HR * (TW + 2);
  constexpr int XS_N = (XS_ITEMS + 255) / 256;
  static_assert(GV_ITEMS % 256 == 0 && GS_ITEMS % 256 == 0, "g tile must split evenly");

  f32x4 gv[VEC ? GV_N : 1];
  f32x4 xv[VEC ? XV_N : 1];
  float xf[VEC ? XH_N : 1];

  auto load_tiles = [&](int chunk) {
    const BlockOrigin o = block_origin<TW, TH, IMGS>(chunk, tiles_w, tiles_h);
    if constexpr (VEC) {
#pragma unroll
      for (int k = 0; k < GV_N; ++k) {
        const int it = tid + k * 256;
        const int q = it % XQ;
        int t = it / XQ;
        const int row = t % TH;
        t /= TH;
        const int img = t % IMGS;
        const int kl = t / IMGS;
        const int n = o.n0 + img, kk = k0 + kl, h = o.h0 + row, w = o.w0 + 4 * q;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (n < N && kk < K && h < H && w < W)
          v = *reinterpret_cast<const f32x4*>(g + ((long)n * K + kk) * HW + (long)h * W + w);
        gv[k] = v;
      }
#pragma unroll
      for (int k = 0; k < XV_N; ++k) {
        const int it = tid + k * 256;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (XV_ITEMS % 256 == 0 || it < XV_ITEMS) {
          const int q = it % XQ;
          int t = it / XQ;
          const int rr = t % HR;
          t /= HR;
          const int img = t % IMGS;
          const int cl = t / IMGS;
          const int n = o.n0 + img, c = c0 + cl, h = o.h0 + rr - 1, w = o.w0 + 4 * q;
          if (n < N && c < C && h >= 0 && h < H && w < W)
            v = *reinterpret_cast<const f32x4*>(x + ((long)n * C + c) * HW + (long)h * W + w);
        }
        xv[k] = v;
      }
#pragma unroll
      for (int k = 0; k < XH_N; ++k) {
        const int it = tid + k * 256;
        float v = 0.f;
        if (XH_ITEMS % 256 == 0 || it < XH_ITEMS) {
          const int side = it & 1;
          int t = it >> 1;
          const int rr = t % HR;
          t /= HR;
          const int img = t % IMGS;
          const int cl = t / IMGS;
          const int n = o.n0 + img, c = c0 + cl, h = o.h0 + rr - 1;
          const int w = o.w0 + (side ? TW : -1);
          if (n < N && c < C && h >= 0 && h < H && w >= 0 && w < W)
            v = x[((long)n * C + c) * HW + (long)h * W + w];
        }
        xf[k] = v;
      }
    }
  };

  // Vector path: global -> registers in load_tiles (one chunk ahead),
  // registers -> LDS here.  Scalar path: everything happens here.
  auto store_tiles = [&](int chunk) {
    if constexpr (VEC) {
#pragma unroll
      for (int k = 0; k < GV_N; ++k) {
        const int it = tid + k * 256;
        const int q = it % XQ;
        const int t = it / XQ;  // (kl * IMGS + img) * TH + row
        const int kl = t / (IMGS * TH);
        const int p = (t % (IMGS * TH)) * TW + 4 * q;
        float* d = &gs[kl * GS + p];
        d[0] = gv[k].x;
        d[1] = gv[k].y;
        d[2] = gv[k].z;
        d[3] = gv[k].w;
      }
#pragma unroll
      for (int k = 0; k < XV_N; ++k) {
        const int it = tid + k * 256;
        if (XV_ITEMS % 256 == 0 || it < XV_ITEMS) {
          const int q = it % XQ;
          const int t = it / XQ;  // (cl * IMGS + img) * HR + rr
          const int cl = t / (IMGS * HR);
          float* d = &xs[cl * PLW + (t % (IMGS * HR)) * RSW + 1 + 4 * q];
          d[0] = xv[k].x;
          d[1] = xv[k].y;
          d[2] = xv[k].z;
          d[3] = xv[k].w;
        }
      }
#pragma unroll
      for (int k = 0; k < XH_N; ++k) {
        const int it = tid + k * 256;
        if (XH_ITEMS % 256 == 0 || it < XH_ITEMS) {
          const int side = it & 1;
          const int t = it >> 1;
          const int cl = t / (IMGS * HR);
          xs[cl * PLW + (t % (IMGS * HR)) * RSW + 1 + (side ? TW : -1)] = xf[k];
        }
      }
    } else {
      // Scalar path (ragged shapes): global loads go straight to LDS.
      const BlockOrigin o = block_origin<TW, TH, IMGS>(chunk, tiles_w, tiles_h);
#pragma unroll 4
      for (int k = 0; k < GS_N; ++k) {
        const int it = tid + k * 256;
        const int col = it % TW;
        int t = it / TW;
        const int row = t % TH;
        t /= TH;
        const int img = t % IMGS;
        const int kl = t / IMGS;
        const int n = o.n0 + img, kk = k0 + kl, h = o.h0 + row, w = o.w0 + col;
        float v = 0.f;
        if (n < N && kk < K && h < H && w < W) v = g[((long)n * K + kk) * HW + (long)h * W + w];
        gs[kl * GS + it % P] = v;
      }
#pragma unroll 4
      for (int k = 0; k < XS_N; ++k) {
        const int it = tid + k * 256;
        if (XS_ITEMS % 256 == 0 || it < XS_ITEMS) {
          const int cc = it % (TW + 2) - 1;
          int t = it / (TW + 2);
          const int rr = t % HR;
          t /= HR;
          const int img = t % IMGS;
          const int cl = t / IMGS;
          const int n = o.n0 + img, c = c0 + cl, h = o.h0 + rr - 1, w = o.w0 + cc;
          float v = 0.f;
          if (n < N && c < C && h >= 0 && h < H && w >= 0 && w < W)
            v = x[((long)n * C + c) * HW + (long)h * W + w];
          xs[cl * PLW + (img * HR + rr) * RSW + 1 + cc] = v;
        }
      }
    }
  };

  f32x16 acc[9];
#pragma unroll
  for (int t = 0; t < 9; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[t][v] = 0.f;
  float dbsum = 0.f;

  const int chunk_begin = slice * per_split;
  const int chunk_end = min(nchunks, chunk_begin + per_split);
  const int goff = (wk * 32 + l32) * GS;
  const int xoff = (wc * 32 + l32) * PLW;

  if (chunk_begin < chunk_end) load_tiles(chunk_begin);
  for (int chunk = chunk_begin; chunk < chunk_end; ++chunk) {
    if (chunk != chunk_begin) __syncthreads();
    store_tiles(chunk);
    __syncthreads();
    if (chunk + 1 < chunk_end) load_tiles(chunk + 1);
#pragma unroll 4
    for (int q2 = 0; q2 < P / 2; ++q2) {
      const int p = 2 * q2 + hi;
      const int img = p / (TH * TW), row = (p / TW) % TH, col = p % TW;
      const float a = gs[goff + p];
      const int xb = xoff + (img * HR + row) * RSW + col;
#pragma unroll
      for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int s = 0; s < 3; ++s)
          acc[r * 3 + s] = mfma_32x32x2_f32(a, xs[xb + r * RSW + s], acc[r * 3 + s]);
    }
    if (do_db) {
      const int kl = tid >> 2, part = tid & 3;
#pragma unroll
      for (int i = 0; i < P / 4; ++i) dbsum += gs[kl * GS + part + 4 * i];
    }
  }

  // Partial dw of this slice: [k][c][tap] at out + slice * slice_stride.
  float* o_dw = out + (long)slice * slice_stride;
#pragma unroll
  for (int t = 0; t < 9; ++t) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int k = k0 + wk * 32 + acc_row(v, hi);
      const int c = c0 + wc * 32 + l32;
      if (k < K && c < C) o_dw[((long)k * C + c) * 9 + t] = acc[t][v];
    }
  }
  if (do_db) {
    // Lanes 4j..4j+3 hold four interleaved partial sums of one k: add them
    // pairwise, (p0 + p1) + (p2 + p3), the same way every time.
    dbsum += __shfl_xor(dbsum, 1);
    dbsum += __shfl_xor(dbsum, 2);
    const int kl = tid >> 2;
    if ((tid & 3) == 0 && k0 + kl < K) out_db[(long)slice * K + k0 + kl] = dbsum;
  }
}

// dw[e] = sum_{s < S} ws[s][e] and db[k] = sum_{s < S} ws_db[s][k], added in
// slice order s = 0, 1, ..., S-1 (one thread per output element).
__global__ __launch_bounds__(256) void wgrad_reduce_kernel(const float* __restrict__ ws,
                                                           float* __restrict__ dw,
                                                           float* __restrict__ db, int S,
                                                           long n_dw, int K) {
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  if (e < n_dw) {
    float s = 0.f;
    for (int i = 0; i < S; ++i) s += ws[(long)i * n_dw + e];
    dw[e] = s;
  } else if (db != nullptr && e < n_dw + K) {
    const long k = e - n_dw;
    const float* wdb = ws + (long)S * n_dw;
    float s = 0.f;
    for (int i = 0; i < S; ++i) s += wdb[(long)i * K + k];
    db[k] = s;
  }
}

template <int TW, int TH, int IMGS>
static void launch_wgrad_geom(const Plan& pl, bool vec, const float* x, const float* g,
                              float* out, float* out_db, long slice_stride, int N, int C, int K,
                              int H, int W, hipStream_t stream) {
  dim3 grid(pl.grid_x, pl.grid_y, pl.grid_z), block(256, 1, 1);
  if (vec)
    hipLaunchKernelGGL((wgrad_f32_kernel<TW, TH, IMGS, true>), grid, block, 0, stream, x, g, out,
                       out_db, N, C, K, H, W, pl.tiles_w, pl.tiles_h, pl.nchunks,
                       pl.chunks_per_split, slice_stride);
  else
    hipLaunchKernelGGL((wgrad_f32_kernel<TW, TH, IMGS, false>), grid, block, 0, stream, x, g,
                       out, out_db, N, C, K, H, W, pl.tiles_w, pl.tiles_h, pl.nchunks,
                       pl.chunks_per_split, slice_stride);
}

bool launch_wgrad_f32(const Plan& pl, bool vec, const float* x, const float* g, float* dw,
                      float* db, float* ws, int N, int C, int K, int H, int W,
                      hipStream_t stream) {
  const long n_dw = (long)K * C * 9;
  float* out = pl.split > 1 ? ws : dw;
  float* out_db = db == nullptr ? nullptr : (pl.split > 1 ? ws + (long)pl.split * n_dw : db);
  const long stride = pl.split > 1 ? n_dw : 0;
  switch (pl.geom) {
    case kG64x1: launch_wgrad_geom<64, 1, 1>(pl, vec, x, g, out, out_db, stride, N, C, K, H, W, stream); break;
    case kG32x2: launch_wgrad_geom<32, 2, 1>(pl, vec, x, g, out, out_db, stride, N, C, K, H, W, stream); break;
    case kG16x4: launch_wgrad_geom<16, 4, 1>(pl, vec, x, g, out, out_db, stride, N, C, K, H, W, stream); break;
    case kG8x8: launch_wgrad_geom<8, 8, 1>(pl, vec, x, g, out, out_db, stride, N, C, K, H, W, stream); break;
    default: return false;
  }
  if (pl.split > 1) {
    const long total = n_dw + (db ? K : 0);
    dim3 grid((unsigned)((total + 255) / 256)), block(256);
    hipLaunchKernelGGL(wgrad_reduce_kernel, grid, block, 0, stream, ws, dw, db, pl.split, n_dw, K);
  }
  return true;
}

}  // namespace conv3x3
