// Backward-weight (+ bias gradient) of a 3x3 convolution whose input has at
// most four channels -- a UNet's first convolution, on the RGB(A) image or a
// latent -- for float32 or bfloat16 inputs, gfx950.
//
// dw[k, c, t] = sum over pixels p of g[k, p] * x[c, p + offset(t)], t = the
// 9 taps: a GEMM with rows k, columns e = (c, t) -- 9C <= 36 of them -- and a
// reduction over pixels.  The general backward-weight kernel tiles 64
// input channels, so with C = 3 it would run 61 of every 64 channel rows on
// zeros.  Here the (channel, tap) pairs are the MFMA's column index instead:
// one 32-column block holds 9C <= 32 pairs (two blocks for C = 4), so the
// MFMA work is 27 useful columns of 32 on an RGB image; the 28th column
// reads ones, so its accumulator is the bias gradient.  The pass streams g
// (the largest tensor, K rows of N*H*W pixels) once from HBM, which is what
// bounds it.
//
// Workgroup: 4 wave64s own 128 k and all pairs; wave w holds rows
// k0 + 32 w .. + 31.  MFMA 32x32x2 f32: step s (0..31) takes pixels s and
// s + 32 of the chunk; lane l supplies A = g[k0 + 32 w + l % 32][p] and
// B = x[c(e)][p + offset(t(e))], p = s + 32 (l / 32), e = 32 b + l % 32.
// A chunk is a 64-pixel block (tw x th); its g rows go through LDS (128-bit
// loads, the rows of NCHW g being pixel-contiguous), x with its one-pixel
// halo.  LDS reads are conflict-free: a lane's A values for four steps are
// adjacent (one 128-bit read; rows 68 floats apart put 8 lanes on all 32
// banks), and the staged x rows and planes are padded to 3 and 9 (mod 32)
// floats, so column e = 9 c + 3 r + s reads bank e + const.
// bfloat16 values are widened to float32 as they are staged: the products
// of bfloat16 values are exact in float32, so the arithmetic is that of the
// bfloat16 MFMA with float32 accumulation.  The chunks are split over
// `split` slices, each slice writing its partial sums tap-major to the
// caller's workspace ([S][9][K][C], then db [S][K]) for the fixed-order
// reduce of the general kernel; no atomics.  (A slice's chunks are every
// S-th chunk rather than a contiguous range; the plan's chunks_per_split is
// the largest count, so the split is the same.)
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace conv3x3 {

namespace {

constexpr int kStemK = 128;  // k rows per workgroup
constexpr int kStemP = 64;   // pixels per chunk

template <typename T>
__device__ __forceinline__ float widen(T v) {
  if constexpr (std::is_same<T, float>::value)
    return v;
  else
    return __builtin_bit_cast(float, (uint32_t)v << 16);
}

// 16 bytes of g: 4 float32 or 8 bfloat16 pixels, widened.
template <typename T>
struct GVec {
  static constexpr int kPix = std::is_same<T, float>::value ? 4 : 8;
};

}  // namespace

template <typename T, int TW, int TH, int CP, bool VEC>
__global__ __launch_bounds__(256) void wgrad_stem_kernel(
    const T* __restrict__ x, const T* __restrict__ g, float* __restrict__ out,
    float* __restrict__ out_db, int N, int C, int K, int H, int W, int tiles_w, int tiles_h,
    int nchunks, int per_split, long slice_stride, int tiles_k, uint32_t x_bytes,
    uint32_t g_bytes) {
  static_assert(TW * TH == kStemP, "64-pixel chunks");
  static_assert(CP >= 1 && CP <= 4, "at most four input channels");
  // 32-column blocks: the 9C (channel, tap) pairs, then one column of ones
  // (its accumulator is the bias gradient sum over pixels of g)
  constexpr int NB = (9 * CP + 1 + 31) / 32;
  constexpr int GS = kStemP + 4;  // g row stride in LDS (floats)
  // x row with its halo columns, padded to 3 (mod 32); a channel's plane
  // of th + 2 rows, padded to 9 (mod 32)
  constexpr int XR = TW + 2 + ((3 - (TW + 2)) % 32 + 32) % 32;
  constexpr int XP = (TH + 2) * XR + ((9 - (TH + 2) * XR) % 32 + 32) % 32;
  static_assert(XR % 32 == 3 && XP % 32 == 9, "bank padding");
  // the lane of a step's second pixel (s + 32) reads this much further
  constexpr int OFF32 = TW >= 64 ? 32 : (32 / TW) * XR;
  constexpr int VP = GVec<T>::kPix;       // pixels per 16-byte g load
  constexpr int GI = kStemK * kStemP / VP;  // g vector items per chunk
  static_assert(GI % 256 == 0, "whole g items per thread");
  constexpr int GN = GI / 256;
  constexpr int XI = CP * XP;              // x elements per chunk (with halo)
  constexpr int XN = (XI + 255) / 256;

  // two LDS buffers: chunk i is read from one while chunk i + 1 is written
  // into the other (one barrier per chunk)
  __shared__ __attribute__((aligned(16))) float gs[2][kStemK * GS];
  // x planes, then a plane of zeros (padding columns read it) and one of
  // ones (the bias-gradient column), shifted so that it falls on the bank
  // of column 9C
  __shared__ float xs[2][(CP + 2) * XP + 32];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int L = blockIdx.x;
  const int slice = L / tiles_k, k0 = (L % tiles_k) * kStemK;
  // Slice s takes chunks s, s + S, s + 2 S, ... (S = split): the workgroups
  // running at one time read neighbouring pixel rows of each g plane, so
  // the memory sees long runs rather than scattered 256-byte pieces.
  const int split = (nchunks + per_split - 1) / per_split;
  const int n = slice < split ? (nchunks - slice + split - 1) / split : 0;
  auto chunk_of = [&](int i) { return slice + i * split; };
  const long HW = (long)H * W;

  const __amdgpu_buffer_rsrc_t gv = buffer_view(g, g_bytes);
  const __amdgpu_buffer_rsrc_t xv = buffer_view(x, x_bytes);

  // Column e = 32 b + l32 of block b: channel c, tap t = 3 r + s; its LDS
  // offset from a pixel's (row, col) in the staged plane, plus this lane's
  // pixel of the step pair (hi).  Column 9C reads the plane of ones, the
  // rest the plane of zeros.
  const int ones = (CP + 1) * XP + ((9 * C - 9 * (CP + 1)) % 32 + 32) % 32;
  int eoff[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int e = 32 * b + l32;
    if (e < 9 * C) {
      const int c = e / 9, t = e % 9;
      eoff[b] = c * XP + (t / 3) * XR + (t % 3) + hi * OFF32;
    } else {
      eoff[b] = (e == 9 * C ? ones : CP * XP) + hi * OFF32;
    }
  }
  for (int i = tid; i < XP; i += 256) {
    xs[0][CP * XP + i] = 0.f;
    xs[1][CP * XP + i] = 0.f;
    xs[0][ones + i] = 1.f;
    xs[1][ones + i] = 1.f;
  }

  // Two register sets: the loads of chunk i + 2 go into chunk i's set once
  // chunk i is in LDS, so each load has a chunk of MFMA work to arrive.
  constexpr int NS = 2;
  u32x4 graw[NS][VEC ? GN : 1];
  T xraw[NS][XN];

  auto load = [&](auto setc, int chunk) __attribute__((always_inline)) {
    constexpr int SET = decltype(setc)::value;
    const BlockOrigin o = block_origin<TW, TH, 1>(chunk, tiles_w, tiles_h);
    if constexpr (VEC) {
#pragma unroll
      for (int i = 0; i < GN; ++i) {
        // item: (k row, pixel vector); consecutive threads take consecutive
        // vectors of one row
        const int it = tid + 256 * i;
        const int kl = it / (kStemP / VP), q = it % (kStemP / VP);
        const int row = (q * VP) / TW, col = (q * VP) % TW;
        const int k = k0 + kl, h = o.h0 + row, w = o.w0 + col;
        const bool ok = o.n0 < N && k < K && h < H && w < W;
        graw[SET][i] = buffer_load16(
            gv, ok ? (uint32_t)(((long)(o.n0 * K + k) * H + h) * W + w) * (uint32_t)sizeof(T)
                   : kOutside);
      }
    }
#pragma unroll
    for (int i = 0; i < XN; ++i) {
      const int it = tid + 256 * i;
      const int c = it / XP, rc = it % XP;
      const int hr = rc / XR, wr = rc % XR;  // (padding: hr >= th + 2 or wr >= tw + 2)
      const int h = o.h0 + hr - 1, w = o.w0 + wr - 1;
      const bool ok = it < XI && c < C && o.n0 < N && hr < TH + 2 && wr < TW + 2 && h >= 0 &&
                      h < H && w >= 0 && w < W;
      if constexpr (std::is_same<T, float>::value)
        xraw[SET][i] = __builtin_bit_cast(
            float, buffer_load4(xv, ok ? (uint32_t)((o.n0 * C + c) * HW + h * W + w) * 4u
                                       : kOutside));
      else
        xraw[SET][i] = (T)buffer_load2(
            xv, ok ? (uint32_t)((o.n0 * C + c) * HW + h * W + w) * 2u : kOutside);
    }
  };

  auto store = [&](auto setc, int chunk, int buf) __attribute__((always_inline)) {
    constexpr int SET = decltype(setc)::value;
    if constexpr (VEC) {
#pragma unroll
      for (int i = 0; i < GN; ++i) {
        const int it = tid + 256 * i;
        const int kl = it / (kStemP / VP), q = it % (kStemP / VP);
        float* d = &gs[buf][kl * GS + q * VP];
        if constexpr (std::is_same<T, float>::value) {
          *reinterpret_cast<u32x4*>(d) = graw[SET][i];
        } else {
          const u32x4 r = graw[SET][i];
          const uint32_t w0 = r.x, w1 = r.y, w2 = r.z, w3 = r.w;
          d[0] = __builtin_bit_cast(float, w0 << 16);
          d[1] = __builtin_bit_cast(float, w0 & 0xffff0000u);
          d[2] = __builtin_bit_cast(float, w1 << 16);
          d[3] = __builtin_bit_cast(float, w1 & 0xffff0000u);
          d[4] = __builtin_bit_cast(float, w2 << 16);
          d[5] = __builtin_bit_cast(float, w2 & 0xffff0000u);
          d[6] = __builtin_bit_cast(float, w3 << 16);
          d[7] = __builtin_bit_cast(float, w3 & 0xffff0000u);
        }
      }
    } else {
      // scalar g (ragged widths or unaligned tensors)
      const BlockOrigin o = block_origin<TW, TH, 1>(chunk, tiles_w, tiles_h);
      for (int it = tid; it < kStemK * kStemP; it += 256) {
        const int kl = it / kStemP, p = it % kStemP;
        const int k = k0 + kl, h = o.h0 + p / TW, w = o.w0 + p % TW;
        float v = 0.f;
        if (o.n0 < N && k < K && h < H && w < W)
          v = widen(g[((long)o.n0 * K + k) * HW + (long)h * W + w]);
        gs[buf][kl * GS + p] = v;
      }
    }
#pragma unroll
    for (int i = 0; i < XN; ++i) {
      const int it = tid + 256 * i;
      if (it < XI) xs[buf][it] = widen(xraw[SET][i]);
    }
  };

  f32x16 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[b][v] = 0.f;
  // step st: pixels st and st + 32; every operand offset is a per-lane
  // base plus a constant of the unrolled step
  const int arow = (32 * wave + l32) * GS + 32 * hi;
  auto compute = [&](int buf) __attribute__((always_inline)) {
    const float* g_l = gs[buf];
    const float* x_l = xs[buf];
#pragma unroll
    for (int j = 0; j < kStemP / 8; ++j) {
      const f32x4 a4 = *reinterpret_cast<const f32x4*>(&g_l[arow + 4 * j]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int st = 4 * j + u;
        const int pb = (st / TW) * XR + (st % TW);
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = mfma_32x32x2_f32(a4[u], x_l[eoff[b] + pb], acc[b]);
      }
    }
  };

  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;
  if (n > 0) load(Set0{}, chunk_of(0));
  if (n > 1) load(Set1{}, chunk_of(1));
  // Chunk i: its set (i & 1) is written to LDS buffer i & 1 -- last read by
  // chunk i - 2, before the barrier that ended chunk i - 1 -- the set is
  // refilled with chunk i + 2, one barrier, then chunk i's MFMAs.
  auto step = [&](auto setc, int i) __attribute__((always_inline)) {
    store(setc, chunk_of(i), i & 1);
    if (i + NS < n) load(setc, chunk_of(i + NS));
    __syncthreads();
    compute(i & 1);
  };
  for (int i = 0; i < n; i += 2) {
    step(Set0{}, i);
    if (i + 1 < n) step(Set1{}, i + 1);
  }

  // Partial dw of this slice: tap-major [t][k][c] slot at out + slice *
  // slice_stride (the reduce adds the slots); without a split, dw itself,
  // [k][c][t].
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int e = 32 * b + l32;
    if (e == 9 * C && out_db != nullptr) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int k = k0 + 32 * wave + acc_row(v, hi);
        if (k < K) out_db[(long)slice * K + k] = acc[b][v];
      }
    }
    if (e >= 9 * C) continue;
    const int c = e / 9, t = e % 9;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int k = k0 + 32 * wave + acc_row(v, hi);
      if (k < K) {
        if (slice_stride)
          out[(long)slice * slice_stride + ((long)t * K + k) * C + c] = acc[b][v];
        else
          out[((long)k * C + c) * 9 + t] = acc[b][v];
      }
    }
  }
}

// The split-K reduce for the many slots of this kernel (up to 512): a
// workgroup of 16 waves owns 64 outputs; wave q adds the slots of a fixed
// sixteenth of them, all of its loads in flight at once, in slot order, and
// wave 0 adds the sixteen partial sums in wave order -- one fixed order for
// every output, bitwise reproducible.  Layouts as the general reduce: dw
// slots tap-major [S][9][K][C], then db rows [S][K]; dw written [k][c][tap].
constexpr int kStemSlotsPerWave = 32;  // slots <= 16 * 32

__global__ __launch_bounds__(1024) void stem_reduce_kernel(const float* __restrict__ ws,
                                                           float* __restrict__ dw,
                                                           float* __restrict__ db, int S,
                                                           int C, int K) {
  __shared__ float part[16][64];
  const long n_dw = (long)K * C * 9;
  const long total = n_dw + (db != nullptr ? K : 0);
  const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const long e = (long)blockIdx.x * 64 + lane;
  const int per = (S + 15) / 16;
  const int s0 = min(S, q * per), s1 = min(S, s0 + per);
  float sum = 0.f;
  if (e < total) {
    const bool dwe = e < n_dw;
    const float* base = dwe ? ws + e : ws + (long)S * n_dw + (e - n_dw);
    const long stride = dwe ? n_dw : K;
    float v[kStemSlotsPerWave];
#pragma unroll
    for (int u = 0; u < kStemSlotsPerWave; ++u)
      v[u] = s0 + u < s1 ? base[(long)(s0 + u) * stride] : 0.f;
#pragma unroll
    for (int u = 0; u < kStemSlotsPerWave; ++u) sum += v[u];
  }
  part[q][lane] = sum;
  __syncthreads();
  if (q == 0 && e < total) {
    float v = part[0][lane];
#pragma unroll
    for (int i = 1; i < 16; ++i) v += part[i][lane];
    if (e < n_dw) {
      const long t = e / ((long)K * C);
      const long kc = e % ((long)K * C);  // k * C + c
      dw[kc * 9 + t] = v;
    } else {
      db[e - n_dw] = v;
    }
  }
}

template <typename T, int TW, int TH>
static void launch_stem_geom(const Plan& pl, bool vec, const T* x, const T* g, float* out,
                             float* out_db, long slice_stride, int N, int C, int K, int H, int W,
                             hipStream_t stream) {
  dim3 grid(pl.grid_x, 1, 1), block(256, 1, 1);
  const int tiles_k = (K + kStemK - 1) / kStemK;
  const long hw = (long)H * W;
  const uint32_t xb = (uint32_t)(N * C * hw * (long)sizeof(T));
  const uint32_t gb = (uint32_t)(N * K * hw * (long)sizeof(T));
#define CONV3X3_S(CP_, VEC_)                                                                     \
  hipLaunchKernelGGL((wgrad_stem_kernel<T, TW, TH, CP_, VEC_>), grid, block, 0, stream, x, g, out, \
                     out_db, N, C, K, H, W, pl.tiles_w, pl.tiles_h, pl.nchunks,                  \
                     pl.chunks_per_split, slice_stride, tiles_k, xb, gb)
  if (C <= 3) {
    if (vec)
      CONV3X3_S(3, true);
    else
      CONV3X3_S(3, false);
  } else {
    if (vec)
      CONV3X3_S(4, true);
    else
      CONV3X3_S(4, false);
  }
#undef CONV3X3_S
}

template <typename T>
static bool launch_stem(const Plan& pl, bool vec, const T* x, const T* g, float* dw, float* db,
                        float* ws, int N, int C, int K, int H, int W, hipStream_t stream) {
  if (C > 4 || pl.threads != 256 || pl.split > 16 * kStemSlotsPerWave) return false;
  const long n_dw = (long)K * C * 9;
  float* out = pl.split > 1 ? ws : dw;
  float* out_db = db == nullptr ? nullptr : (pl.split > 1 ? ws + (long)pl.split * n_dw : db);
  const long stride = pl.split > 1 ? n_dw : 0;
  if (pl.tw == 64 && pl.th == 1)
    launch_stem_geom<T, 64, 1>(pl, vec, x, g, out, out_db, stride, N, C, K, H, W, stream);
  else if (pl.tw == 32 && pl.th == 2)
    launch_stem_geom<T, 32, 2>(pl, vec, x, g, out, out_db, stride, N, C, K, H, W, stream);
  else if (pl.tw == 16 && pl.th == 4)
    launch_stem_geom<T, 16, 4>(pl, vec, x, g, out, out_db, stride, N, C, K, H, W, stream);
  else if (pl.tw == 8 && pl.th == 8)
    launch_stem_geom<T, 8, 8>(pl, vec, x, g, out, out_db, stride, N, C, K, H, W, stream);
  else
    return false;
  if (pl.split > 1) {
    const long total = n_dw + (db ? K : 0);
    dim3 rg((unsigned)((total + 63) / 64)), rb(1024);
    hipLaunchKernelGGL(stem_reduce_kernel, rg, rb, 0, stream, ws, dw, db, pl.split, C, K);
  }
  return true;
}

bool launch_wgrad_stem_f32(const Plan& pl, bool vec, const float* x, const float* g, float* dw,
                           float* db, float* ws, int N, int C, int K, int H, int W,
                           hipStream_t stream) {
  return launch_stem<float>(pl, vec, x, g, dw, db, ws, N, C, K, H, W, stream);
}

bool launch_wgrad_stem_bf16(const Plan& pl, bool vec, const uint16_t* x, const uint16_t* g,
                            float* dw, float* db, float* ws, int N, int C, int K, int H, int W,
                            hipStream_t stream) {
  return launch_stem<uint16_t>(pl, vec, x, g, dw, db, ws, N, C, K, H, W, stream);
}

}  // namespace conv3x3
