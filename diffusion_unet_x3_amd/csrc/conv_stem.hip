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
// MFMA work is 27 useful columns of 32 on an RGB image; column 9C reads
// ones, so its accumulator is the bias gradient.  The pass streams g (the
// largest tensor, K rows of N*H*W pixels) once from HBM, which is what
// bounds it.
//
// Wave w of a workgroup owns the 32 rows k0 + 32 w .. + 31 (128 per
// workgroup) and works alone: it stages its own rows of g and its own copy
// of the small x tile in a private LDS region, so no workgroup barrier ever
// couples one wave's memory wait to another's.  MFMA 32x32x2 f32: step s
// (0..31) takes pixels s and s + 32 of a 64-pixel chunk (tw x th); lane l
// supplies A = g[k][p] (k = its row l % 32) and B = x[c(e)][p + offset(t(e))],
// p = s + 32 (l / 32), e = 32 b + l % 32.  g rows are loaded 16 bytes per
// lane (16 lanes per 256-byte pixel row of a plane) and transposed through
// LDS; a lane's A values for four steps are then one 128-bit LDS read (rows
// 68 floats apart put 8 lanes on all 32 banks), and the staged x rows and
// planes are padded to 3 and 9 (mod 32) floats, so column e = 9 c + 3 r + s
// reads bank e + const.  bfloat16 values are widened to float32 as they are
// staged: products of bfloat16 values are exact in float32, so the
// arithmetic is that of the bfloat16 MFMA with float32 accumulation.
//
// The chunks are split over `split` slices (slice s: chunks s, s + S, ... --
// the workgroups running at one time read neighbouring pixel rows of each g
// plane).  Each slice writes its partial sums as a slot [K][32 NB] -- row k,
// column e, the bias gradient in column 9C -- so that a wave's stores are
// two 128-byte runs per instruction; stem_reduce_kernel adds the slots in a
// fixed order.  No atomics.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "lds_layout.hpp"

namespace conv3x3 {

namespace {

constexpr int kStemK = 128;     // k rows per workgroup
constexpr int kStemWaveK = 32;  // k rows per wave
constexpr int kStemP = 64;      // pixels per chunk
static_assert(kStemWaves == 2 * kStemK / kStemWaveK, "two waves per 32-row block");

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

// A wave's g rows are private to it: its LDS operations execute in order,
// so its stores are seen by its later loads; the fence keeps the compiler
// from moving LDS accesses across this point.
__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
}

template <typename T, int TW, int TH, int CP, bool VEC>
__global__ __launch_bounds__(512) void wgrad_stem_kernel(
    const T* __restrict__ x, const T* __restrict__ g, float* __restrict__ out,
    float* __restrict__ out_db, int N, int C, int K, int H, int W, int tiles_w, int tiles_h,
    int nchunks, int per_split, int tiles_k, int slots, uint32_t x_bytes, uint32_t g_bytes) {
  static_assert(TW * TH == kStemP, "64-pixel chunks");
  static_assert(CP >= 1 && CP <= 4, "at most four input channels");
  // 32-column blocks: the 9C (channel, tap) pairs, then one column of ones
  constexpr int NB = (9 * CP + 1 + 31) / 32;
  constexpr int EP = 32 * NB;      // columns of a slot row
  static_assert(EP == stem_slot_columns(CP), "slot layout");
  constexpr int GS = kStemP + 4;   // g row stride in LDS (floats)
  // x row with its halo columns, padded to 3 (mod 32); a channel's plane
  // of th + 2 rows, padded to 9 (mod 32)
  constexpr int XR = stem_xr(TW);
  constexpr int XP = stem_xp(TH, TW);
  static_assert(XR % 32 == 3 && XP % 32 == 9, "bank padding");
  // the lane of a step's second pixel (s + 32) reads this much further
  constexpr int OFF32 = TW >= 64 ? 32 : (32 / TW) * XR;
  constexpr int VP = GVec<T>::kPix;             // pixels per 16-byte g load
  constexpr int GI = kStemWaveK * kStemP / VP;  // g vector items per wave and chunk
  static_assert(GI % 64 == 0, "whole g items per lane");
  constexpr int GN = GI / 64;
  constexpr int XI = CP * XP;                   // one chunk's x planes
  constexpr int XGI = kStemGroup * XI;          // a group's
  constexpr int XN = stem_x_items(TH, TW, CP);  // x items per lane (one chunk per wave)
  constexpr int ZP = XP;                        // the plane of zeros
  constexpr int GREG = kStemWaveK * GS;         // a wave's g rows
  static_assert(XN * 64 >= XI && GREG == 32 * 68 && kStemGroup == kStemWaves, "layout");
  __shared__ __attribute__((aligned(16))) float lds[stem_lds_bytes(TH, TW, CP) / 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int par = wave >> 2;  // this wave takes the slice's chunks of this parity
  const int L = blockIdx.x;
  const int slice = L / tiles_k;
  const int kw = (L % tiles_k) * kStemK + kStemWaveK * (wave & 3);
  const int split = (nchunks + per_split - 1) / per_split;
  if (slice >= split) return;  // (the plan launches split * tiles_k workgroups)
  const int n = (nchunks - slice + split - 1) / split;
  auto chunk_of = [&](int i) { return slice + i * split; };
  const long HW = (long)H * W;
  float* gsw = lds + wave * GREG;
  float* xs = lds + kStemWaves * GREG;

  const __amdgpu_buffer_rsrc_t gv = buffer_view(g, g_bytes);
  const __amdgpu_buffer_rsrc_t xv = buffer_view(x, x_bytes);

  // Column e = 32 b + l32 of block b: channel c, tap t = 3 r + s; its LDS
  // offset from a pixel's (row, col) in a chunk's staged planes, plus this
  // lane's pixel of the step (hi).  Column 9C reads the plane of ones,
  // shifted to that column's bank; the rest the plane of zeros.
  const int ones = XGI + ZP + ((9 * C - XGI - ZP) % 32 + 32) % 32;
  int eoff[NB];
  bool edata[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int e = 32 * b + l32;
    edata[b] = e < 9 * C;
    if (e < 9 * C) {
      const int c = e / 9, t = e % 9;
      eoff[b] = c * XP + (t / 3) * XR + (t % 3) + hi * OFF32;
    } else {
      eoff[b] = (e == 9 * C ? ones : XGI) + hi * OFF32;
    }
  }
  for (int i = tid; i < ZP; i += 512) xs[XGI + i] = 0.f;
  for (int i = tid; i < XP; i += 512) xs[ones + i] = 1.f;

  // x of a group of kStemGroup chunks (slice chunks 8 q .. 8 q + 7): wave
  // w stages chunk 8 q + w (its origin is uniform across the wave) at
  // xs + w * XI.  Items of chunks past the slice's last read zero (out of
  // range, no memory access); items past the planes go to the plane of
  // zeros.
  T xraw[XN];
  auto load_x = [&](int q) __attribute__((always_inline)) {
    const int i = kStemGroup * q + wave;
    const bool live = i < n;
    const BlockOrigin o = block_origin<TW, TH, 1>(live ? chunk_of(i) : 0, tiles_w, tiles_h);
#pragma unroll
    for (int j = 0; j < XN; ++j) {
      const int it = lane + 64 * j;
      const int c = it / XP, rc = it % XP;
      const int hr = rc / XR, wr = rc % XR;  // (padding: hr >= th + 2 or wr >= tw + 2)
      const int h = o.h0 + hr - 1, w = o.w0 + wr - 1;
      // (& rather than &&: a select, not a branch)
      const bool ok = live & (it < XI) & (c < C) & (o.n0 < N) & (hr < TH + 2) & (wr < TW + 2) &
                      (h >= 0) & (h < H) & (w >= 0) & (w < W);
      if constexpr (std::is_same<T, float>::value)
        xraw[j] = __builtin_bit_cast(
            float, buffer_load4(xv, ok ? (uint32_t)((o.n0 * C + c) * HW + h * W + w) * 4u
                                       : kOutside));
      else
        xraw[j] = (T)buffer_load2(
            xv, ok ? (uint32_t)((o.n0 * C + c) * HW + h * W + w) * 2u : kOutside);
    }
  };
  auto store_x = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < XN; ++j) {
      const int it = lane + 64 * j;
      xs[it < XI ? wave * XI + it : XGI + lane] = widen(xraw[j]);
    }
  };

  // g: wave-chunk j is the slice's chunk 2 j + par.  Two register sets:
  // wave-chunk j + 2 is loaded into j's set once j is in LDS, so each load
  // has a chunk of MFMA work to arrive.  Past the slice's last chunk every
  // offset is out of range (zeros, no memory access): loads are issued on
  // every path, so the compiler's count of loads in flight is exact.
  constexpr int NS = 2;
  u32x4 graw[NS][VEC ? GN : 1];
  auto load_g = [&](auto setc, int j) __attribute__((always_inline)) {
    if constexpr (VEC) {
      constexpr int SET = decltype(setc)::value;
      const int i = 2 * j + par;
      const bool live = i < n;
      const BlockOrigin o = block_origin<TW, TH, 1>(live ? chunk_of(i) : 0, tiles_w, tiles_h);
#pragma unroll
      for (int u = 0; u < GN; ++u) {
        // item: (k row, pixel vector); 64 / VP consecutive lanes take one
        // row's 256 bytes (float32)
        const int it = lane + 64 * u;
        const int kl = it / (kStemP / VP), q = it % (kStemP / VP);
        const int row = (q * VP) / TW, col = (q * VP) % TW;
        const int k = kw + kl, h = o.h0 + row, w = o.w0 + col;
        const bool ok = live & (o.n0 < N) & (k < K) & (h < H) & (w < W);
        graw[SET][u] = buffer_load16(
            gv, ok ? (uint32_t)(((long)(o.n0 * K + k) * H + h) * W + w) * (uint32_t)sizeof(T)
                   : kOutside);
      }
    }
  };
  auto store_g = [&](auto setc, int j) __attribute__((always_inline)) {
    constexpr int SET = decltype(setc)::value;
    if constexpr (VEC) {
#pragma unroll
      for (int u = 0; u < GN; ++u) {
        const int it = lane + 64 * u;
        const int kl = it / (kStemP / VP), q = it % (kStemP / VP);
        float* d = &gsw[kl * GS + q * VP];
        if constexpr (std::is_same<T, float>::value) {
          *reinterpret_cast<u32x4*>(d) = graw[SET][u];
        } else {
          const u32x4 r = graw[SET][u];
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
      const int i = 2 * j + par;
      const bool live = i < n;
      const BlockOrigin o = block_origin<TW, TH, 1>(live ? chunk_of(i) : 0, tiles_w, tiles_h);
      for (int it = lane; it < kStemWaveK * kStemP; it += 64) {
        const int kl = it / kStemP, p = it % kStemP;
        const int k = kw + kl, h = o.h0 + p / TW, w = o.w0 + p % TW;
        float v = 0.f;
        if (live && o.n0 < N && k < K && h < H && w < W)
          v = widen(g[((long)o.n0 * K + k) * HW + (long)h * W + w]);
        gsw[kl * GS + p] = v;
      }
    }
  };

  // Consecutive MFMAs do not wait for each other's results: with one
  // column block, two accumulator chains (even and odd steps, added at the
  // end); with two, the blocks alternate.
  constexpr int CH = NB == 1 ? 2 : 1;
  f32x16 acc[NB][CH];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int h = 0; h < CH; ++h)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[b][h][v] = 0.f;
  // step st: pixels st and st + 32; every operand offset is a per-lane
  // base plus a constant of the unrolled step.  The steps go in groups (8
  // steps; 4 with two column blocks) whose operands are read from LDS one
  // group ahead (two register sets), so the MFMAs never wait for an LDS
  // read just issued.
  constexpr int GSZ = NB == 1 ? 8 : 4;
  const int arow = l32 * GS + 32 * hi;
  auto compute = [&](int xb) __attribute__((always_inline)) {
    int eo[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) eo[b] = eoff[b] + (edata[b] ? xb : 0);
    f32x4 av[2][GSZ / 4];
    float bv[2][NB][GSZ];
    auto read = [&](int grp, int set) __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < GSZ / 4; ++q)
        av[set][q] = *reinterpret_cast<const f32x4*>(&gsw[arow + GSZ * grp + 4 * q]);
#pragma unroll
      for (int u = 0; u < GSZ; ++u) {
        const int st = GSZ * grp + u;
        const int pb = (st / TW) * XR + (st % TW);
#pragma unroll
        for (int b = 0; b < NB; ++b) bv[set][b][u] = xs[eo[b] + pb];
      }
    };
    read(0, 0);
#pragma unroll
    for (int grp = 0; grp < kStemP / 2 / GSZ; ++grp) {
      if (grp + 1 < kStemP / 2 / GSZ) read(grp + 1, (grp + 1) & 1);
      // (keeps the compiler from sinking those reads below the MFMAs)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < GSZ; ++u)
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[b][u % CH] =
              mfma_32x32x2_f32(av[grp & 1][u / 4][u % 4], bv[grp & 1][b][u], acc[b][u % CH]);
    }
  };

  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;
  // Wave-chunk j: the MFMAs of j - 1 have read the wave's rows; j's set
  // goes to LDS, the set is refilled with j + 2, then j's MFMAs on x slot
  // 2 (j % 4) + par of the group.
  auto step = [&](auto setc, int j) __attribute__((always_inline)) {
    wave_lds_order();
    store_g(setc, j);
    load_g(setc, j + NS);
    wave_lds_order();
    compute((2 * (j % (kStemGroup / 2)) + par) * XI);
  };
  // The first group's x loads go out before the g loads, so that staging
  // them waits for nothing else; a later group's are issued at its start
  // (behind the g loads in flight -- once per kStemGroup chunks).
  load_x(0);
  load_g(Set0{}, 0);
  load_g(Set1{}, 1);
  const int ngroups = (n + kStemGroup - 1) / kStemGroup;
  for (int q = 0; q < ngroups; ++q) {
    if (q > 0) {
      __syncthreads();  // every wave is done with group q - 1's x
      load_x(q);
    }
    store_x();
    __syncthreads();
#pragma unroll
    for (int jj = 0; jj < kStemGroup / 2; jj += 2) {
      step(Set0{}, (kStemGroup / 2) * q + jj);
      step(Set1{}, (kStemGroup / 2) * q + jj + 1);
    }
  }

  if constexpr (CH == 2) {
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b][0] += acc[b][CH - 1];
  }
  // The odd-chunk waves hand their sums to the even-chunk waves of the same
  // rows through their own (now idle) g regions; the sum is even + odd.
  __syncthreads();
  if (par == 1) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) gsw[(b * 16 + v) * 64 + lane] = acc[b][0][v];
  }
  __syncthreads();
  if (par == 1) return;
  {
    const float* pr = lds + (wave + 4) * GREG;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[b][0][v] += pr[(b * 16 + v) * 64 + lane];
  }

  // This slice's partial sums: slot row k, column e (two 128-byte runs per
  // store); without a split, dw itself ([k][c][tap] = [k][e]) and db.
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int e = 32 * b + l32;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int k = kw + acc_row(v, hi);
      if (k >= K) continue;
      if (slots) {
        out[((long)slice * K + k) * EP + e] = acc[b][0][v];
      } else if (e < 9 * C) {
        out[(long)k * 9 * C + e] = acc[b][0][v];
      } else if (e == 9 * C && out_db != nullptr) {
        out_db[k] = acc[b][0][v];
      }
    }
  }
}

// The split-K reduce of the slots [S][K][EP] (S <= 256): a workgroup owns
// 16 consecutive (k, e) positions; thread t loads the 16 bytes of slot
// t / 4 at positions 4 (t % 4) .. + 3 -- every load of the workgroup in
// flight at once -- and the slots are added by a pairwise tree in LDS
// (slot s + h into slot s, h = 128, 64, .., 1): one fixed order for every
// output, bitwise reproducible.  dw[k][e] for e < 9C ([k][c][tap]), db[k]
// from column 9C.
constexpr int kStemMaxSlots = 256;

__global__ __launch_bounds__(1024) void stem_reduce_kernel(const float* __restrict__ ws,
                                                           float* __restrict__ dw,
                                                           float* __restrict__ db, int S,
                                                           int C, int K, int EP) {
  __shared__ __attribute__((aligned(16))) float part[kStemMaxSlots][16];
  const long total = (long)K * EP;  // a multiple of 32: 16-position groups never straddle it
  const int t = threadIdx.x, sl = t >> 2, q = t & 3;
  const long p0 = (long)blockIdx.x * 16;
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  if (sl < S) v = *reinterpret_cast<const f32x4*>(ws + (long)sl * total + p0 + 4 * q);
  *reinterpret_cast<f32x4*>(&part[sl][4 * q]) = v;
  __syncthreads();
#pragma unroll
  for (int h = kStemMaxSlots / 2; h >= 1; h /= 2) {
    if (sl < h) {
      f32x4 a = *reinterpret_cast<const f32x4*>(&part[sl][4 * q]);
      const f32x4 b = *reinterpret_cast<const f32x4*>(&part[sl + h][4 * q]);
      a += b;
      *reinterpret_cast<f32x4*>(&part[sl][4 * q]) = a;
    }
    __syncthreads();
  }
  if (t < 16) {
    const long pos = p0 + t;
    const long k = pos / EP;
    const int e = (int)(pos % EP);
    const float r = part[0][t];
    if (e < 9 * C)
      dw[k * 9 * C + e] = r;
    else if (e == 9 * C && db != nullptr)
      db[k] = r;
  }
}

template <typename T, int TW, int TH>
static void launch_stem_geom(const Plan& pl, bool vec, const T* x, const T* g, float* out,
                             float* out_db, int N, int C, int K, int H, int W,
                             hipStream_t stream) {
  dim3 grid(pl.grid_x, 1, 1), block(64 * kStemWaves, 1, 1);
  const int tiles_k = (K + kStemK - 1) / kStemK;
  const long hw = (long)H * W;
  const uint32_t xb = (uint32_t)(N * C * hw * (long)sizeof(T));
  const uint32_t gb = (uint32_t)(N * K * hw * (long)sizeof(T));
  const int slots = pl.split > 1 ? 1 : 0;
#define CONV3X3_S(CP_, VEC_)                                                                     \
  hipLaunchKernelGGL((wgrad_stem_kernel<T, TW, TH, CP_, VEC_>), grid, block, 0, stream, x, g, out, \
                     out_db, N, C, K, H, W, pl.tiles_w, pl.tiles_h, pl.nchunks,                  \
                     pl.chunks_per_split, tiles_k, slots, xb, gb)
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
  if (C > 4 || !pl.stem || pl.threads != 64 * kStemWaves || pl.split > kStemMaxSlots)
    return false;
  const int EP = stem_slot_columns(C);
  float* out = pl.split > 1 ? ws : dw;
  float* out_db = pl.split > 1 ? nullptr : db;
  if (pl.tw == 64 && pl.th == 1)
    launch_stem_geom<T, 64, 1>(pl, vec, x, g, out, out_db, N, C, K, H, W, stream);
  else if (pl.tw == 32 && pl.th == 2)
    launch_stem_geom<T, 32, 2>(pl, vec, x, g, out, out_db, N, C, K, H, W, stream);
  else if (pl.tw == 16 && pl.th == 4)
    launch_stem_geom<T, 16, 4>(pl, vec, x, g, out, out_db, N, C, K, H, W, stream);
  else if (pl.tw == 8 && pl.th == 8)
    launch_stem_geom<T, 8, 8>(pl, vec, x, g, out, out_db, N, C, K, H, W, stream);
  else
    return false;
  if (pl.split > 1) {
    const long total = (long)K * EP;
    dim3 rg((unsigned)(total / 16)), rb(1024);
    hipLaunchKernelGGL(stem_reduce_kernel, rg, rb, 0, stream, ws, dw, db, pl.split, C, K, EP);
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
