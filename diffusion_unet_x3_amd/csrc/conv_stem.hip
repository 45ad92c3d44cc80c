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
// staged and run v_mfma_f32_32x32x16_bf16 on their (exact) high halves:
// step s covers 16 pixels, lane l the eight pixels 16 s + 8 (l / 32) + j,
// so a chunk takes 4 MFMA steps instead of 32 (the same LDS reads).
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
  // bfloat16 runs v_mfma_f32_32x32x16_bf16 (see compute): lanes 32-63 take
  // pixels 8 further; float32 the step's second pixel, 32 further.  The
  // lane's x offset for that pixel:
  constexpr bool BF = !std::is_same<T, float>::value;
  constexpr int OFF32 = TW >= 64 ? 32 : (32 / TW) * XR;
  constexpr int OFF8 = TW >= 16 ? 8 : XR;
  constexpr int OFFH = BF ? OFF8 : OFF32;
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
      eoff[b] = c * XP + (t / 3) * XR + (t % 3) + hi * OFFH;
    } else {
      eoff[b] = (e == 9 * C ? ones : XGI) + hi * OFFH;
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
    if constexpr (BF) {
      // bfloat16: step s takes pixels 16 s .. 16 s + 15, lane (l32, hi) the
      // eight pixels 16 s + 8 hi + j -- A from its g row, B from column e's
      // staged x (eight consecutive pixels of one row: 8 | TW), each value
      // bfloat16 widened to float32, so its high half is exact.  All the
      // chunk's operands are read before its four MFMA steps.
      u32x4 aw[kStemP / 16];
      u32x4 bw[kStemP / 16][NB];
      auto pack = [](float lo, float hi2) __attribute__((always_inline)) {
        return (__builtin_bit_cast(uint32_t, lo) >> 16) |
               (__builtin_bit_cast(uint32_t, hi2) & 0xffff0000u);
      };
#pragma unroll
      for (int st = 0; st < kStemP / 16; ++st) {
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(&gsw[l32 * GS + 16 * st + 8 * hi]);
        const f32x4 a1 = *reinterpret_cast<const f32x4*>(&gsw[l32 * GS + 16 * st + 8 * hi + 4]);
        aw[st] = u32x4{pack(a0[0], a0[1]), pack(a0[2], a0[3]), pack(a1[0], a1[1]),
                       pack(a1[2], a1[3])};
        const int pb = ((16 * st) / TW) * XR + (16 * st) % TW;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          float xv8[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) xv8[j] = xs[eo[b] + pb + j];
          bw[st][b] = u32x4{pack(xv8[0], xv8[1]), pack(xv8[2], xv8[3]), pack(xv8[4], xv8[5]),
                            pack(xv8[6], xv8[7])};
        }
      }
#pragma unroll
      for (int st = 0; st < kStemP / 16; ++st)
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[b][st % CH] = mfma_32x32x16_bf16(aw[st], bw[st][b], acc[b][st % CH]);
      return;
    }
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

// ---------------------------------------------------------------------------
// Forward (+ bias) of a convolution whose input has at most four channels,
// bfloat16 inputs, float32 output: y[n, k, p] = b[k] + sum over e = (c, tap)
// of w[k, e] x[n, c, p + offset(e)].  A GEMM with rows k, columns pixels and
// a reduction of only 9C (channel, tap) pairs, so the pass is bound by its
// output (K float32 per pixel).  MFMA 32x32x16 (products exact in float32):
// step s takes the pairs e = 16 s + 8 (l / 32) + 0..7, pairs past 9C are
// zero (two steps for C = 3); the bias (float32, from LDS) is added to the
// sums as they are stored.  Each wave keeps its weights in registers for the
// whole launch, and the workgroups loop over 128-pixel tiles (persistent),
// so that a wave's stores of one tile drain while it computes the next.
// Workgroup: 4 waves, kStemFwdCo = 64 output channels (2 blocks of 32,
// masked past K) x one tile; wave w computes the tile's pixels 32 w .. 32 w +
// 31 for all 64 channels.  The tile's x (with its halo, zero outside the
// image, widened to float32) is staged by the workgroup into one of two LDS
// buffers; one barrier per tile.  Stores: the lane's offset is one
// register, each channel's plane offset the store's scalar offset.  (A
// fused activation or z output takes the general kernel.  The float32
// forward keeps the packed-tap path of the general kernel, which measured
// faster than this structure with 32x32x2 MFMAs.)
template <int TW, int C>
__global__ __launch_bounds__(256) void fwd_stem_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const float* __restrict__ bias, float* __restrict__ y, int N, int K, int H, int W,
    int tiles_w, int tiles_h, int ntiles, uint32_t x_bytes, uint32_t y_bytes) {
  constexpr int TH = kStemFwdPix / TW;
  constexpr int XR = stem_xr(TW);
  constexpr int XP = stem_xp(TH, TW);
  constexpr int XI = C * XP;                     // x floats per tile (with padding)
  constexpr int XN = (XI + 255) / 256;           // x items per thread
  constexpr int XF = stem_fwd_x_floats(TH, TW, C);
  static_assert(XN * 256 - XI <= XP, "items past the planes land in the plane of zeros");
  constexpr int NS = (9 * C + 15) / 16;           // MFMA steps of 16 pairs
  constexpr int NB = kStemFwdCo / 32;            // channel blocks per wave
  __shared__ __attribute__((aligned(16))) float xs[2][XF];
  __shared__ float bias_s[kStemFwdCo];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int k0 = blockIdx.y * kStemFwdCo;
  const long HW = (long)H * W;

  // the plane of zeros (pairs past 9C read it), in both buffers
  for (int i = tid; i < XP; i += 256) {
    xs[0][XI + i] = 0.f;
    xs[1][XI + i] = 0.f;
  }
  if (tid < kStemFwdCo) bias_s[tid] = bias != nullptr && k0 + tid < K ? bias[k0 + tid] : 0.f;

  // This lane's pixel of the tile: p = 32 wave + l32 -> (row, col), and
  // its LDS base in a staged plane.
  const int p = 32 * wave + l32;
  const int prow = p / TW, pcol = p % TW;
  const int pbase = prow * XR + pcol;
  // LDS offset of pair e at this lane's pixel (a constant of e; the zero
  // plane is read at its first element by every lane)
  auto e_off = [&](int e) -> int {
    if (e < 9 * C) return pbase + (e / 9) * XP + ((e % 9) / 3) * XR + (e % 9) % 3;
    return XI;
  };

  // Weights (A) for the NB channel blocks, held for the whole launch: lane
  // (l32, hi) packs w[k, e], e = 16 s + 8 hi + 0..7, two per 32-bit word.
  uint32_t aw[NB][4 * NS];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int k = k0 + 32 * b + l32;
    auto wval = [&](int e) -> uint32_t {
      return k < K && e < 9 * C ? (uint32_t)w[(long)k * 9 * C + e] : 0u;
    };
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int e = 16 * s + 8 * hi + 2 * m;
        aw[b][4 * s + m] = wval(e) | wval(e + 1) << 16;
      }
  }

  const __amdgpu_buffer_rsrc_t xv = buffer_view(x, x_bytes);
  const __amdgpu_buffer_rsrc_t yv = buffer_view(y, y_bytes);
  uint16_t xraw[XN];
  auto load_x = [&](int tile) __attribute__((always_inline)) {
    const bool live = tile < ntiles;
    const BlockOrigin o = block_origin<TW, TH, 1>(live ? tile : 0, tiles_w, tiles_h);
#pragma unroll
    for (int j = 0; j < XN; ++j) {
      const int it = tid + 256 * j;
      const int c = it / XP, rc = it % XP;
      const int hr = rc / XR, wr = rc % XR;  // (padding: hr >= th + 2 or wr >= tw + 2)
      const int h = o.h0 + hr - 1, ww = o.w0 + wr - 1;
      // (& rather than &&: a select, not a branch)
      const bool ok = live & (it < XI) & (o.n0 < N) & (hr < TH + 2) & (wr < TW + 2) & (h >= 0) &
                      (h < H) & (ww >= 0) & (ww < W);
      const uint32_t off = ok ? (uint32_t)((o.n0 * C + c) * HW + h * W + ww) * 2u : kOutside;
      xraw[j] = (uint16_t)buffer_load2(xv, off);
    }
  };
  auto store_x = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < XN; ++j) xs[buf][tid + 256 * j] = widen(xraw[j]);
  };

  const uint32_t plane4 = (uint32_t)(HW * 4);
  // The tile loop, for a whole channel tile or the partial last one (the
  // choice made once, outside the loop).  Iteration i: barrier, tile i's
  // MFMAs from buffer i & 1, tile i + 1's x loads, tile i's stores, then
  // tile i + 1's x into the other buffer (last read in iteration i - 1,
  // before this iteration's barrier).  Every wait for memory sits in
  // straight-line code after the stores, so the compiler counts them
  // exactly and waits for the x loads only -- the stores drain while the
  // next tile computes.
  auto tiles = [&](auto whole_c) __attribute__((always_inline)) {
    constexpr bool WHOLE = decltype(whole_c)::value;
    int tile = blockIdx.x;
    load_x(tile);
    store_x(0);
    for (int i = 0; tile < ntiles; ++i, tile += gridDim.x) {
      const int buf = i & 1;
      __syncthreads();
      const float* xb = xs[buf];
      f32x16 acc[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[b][v] = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        u32x4 bw;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int e0 = 16 * s + 2 * m, e1 = e0 + 8;  // (lanes 0-31 / 32-63)
          const float v0 = xb[hi ? e_off(e1) : e_off(e0)];
          const float v1 = xb[hi ? e_off(e1 + 1) : e_off(e0 + 1)];
          // (staged values are bfloat16 widened: the high halves are exact)
          bw[m] = (__builtin_bit_cast(uint32_t, v0) >> 16) |
                  (__builtin_bit_cast(uint32_t, v1) & 0xffff0000u);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const u32x4 a4 = {aw[b][4 * s], aw[b][4 * s + 1], aw[b][4 * s + 2], aw[b][4 * s + 3]};
          acc[b] = mfma_32x32x16_bf16(a4, bw, acc[b]);
        }
      }
      load_x(tile + gridDim.x);  // (past the last tile: zeros, no memory access)
      // y of this lane's pixel for its channels: lane offset of channel
      // k0 + 4 hi, plus channel 32 b + 8 (v / 4) + v % 4's plane as the
      // scalar offset; out-of-range elements store nothing (the range check)
      const BlockOrigin o = block_origin<TW, TH, 1>(tile, tiles_w, tiles_h);
      const int h = o.h0 + prow, ww = o.w0 + pcol;
      const bool pix_ok = (o.n0 < N) & (h < H) & (ww < W);
      const uint32_t lane_off =
          (uint32_t)((((long)o.n0 * K + k0 + 4 * hi) * H + h) * W + ww) * 4u;
      const uint32_t pix_off = pix_ok ? lane_off : kOutside;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kr = 32 * b + 8 * (v / 4) + v % 4;  // channel row less 4 hi
          const uint32_t voff = WHOLE || k0 + kr + 4 * hi < K ? pix_off : kOutside;
          buffer_store4(yv, voff, (uint32_t)kr * plane4, acc[b][v] + bias_s[kr + 4 * hi]);
        }
      store_x(buf ^ 1);
    }
  };
  if (k0 + kStemFwdCo <= K)
    tiles(std::true_type{});
  else
    tiles(std::false_type{});
}

template <int TW>
static void launch_fwd_stem_geom(const Plan& pl, const uint16_t* x, const uint16_t* w,
                                 const float* bias, float* y, int N, int C, int K, int H, int W,
                                 hipStream_t stream) {
  dim3 grid(pl.grid_x, pl.grid_y, 1), block(256, 1, 1);
  const long hw = (long)H * W;
  const uint32_t xb = (uint32_t)(N * C * hw * 2L);
  const uint32_t yb = (uint32_t)(N * K * hw * 4L);
#define CONV3X3_F(C_)                                                                          \
  hipLaunchKernelGGL((fwd_stem_bf16_kernel<TW, C_>), grid, block, 0, stream, x, w, bias, y, N, K, \
                     H, W, pl.tiles_w, pl.tiles_h, pl.nchunks, xb, yb)
  switch (C) {
    case 1: CONV3X3_F(1); break;
    case 2: CONV3X3_F(2); break;
    case 3: CONV3X3_F(3); break;
    default: CONV3X3_F(4); break;
  }
#undef CONV3X3_F
}

bool launch_fwd_stem_bf16(const Plan& pl, const uint16_t* x, const uint16_t* w,
                          const float* bias, float* y, int N, int C, int K, int H, int W,
                          hipStream_t stream) {
  if (C > 4 || !pl.stem || pl.threads != 256 || pl.tw * pl.th != kStemFwdPix) return false;
  switch (pl.tw) {
    case 64: launch_fwd_stem_geom<64>(pl, x, w, bias, y, N, C, K, H, W, stream); break;
    case 32: launch_fwd_stem_geom<32>(pl, x, w, bias, y, N, C, K, H, W, stream); break;
    case 16: launch_fwd_stem_geom<16>(pl, x, w, bias, y, N, C, K, H, W, stream); break;
    case 8: launch_fwd_stem_geom<8>(pl, x, w, bias, y, N, C, K, H, W, stream); break;
    default: return false;
  }
  return true;
}

// ---------------------------------------------------------------------------
// Backward-data of a 3x3 convolution whose input has at most three channels
// (a UNet's first convolution on an RGB image):
//   dx[c, i, j] = sum over k, (r, s) of g[k, i + 1 - r, j + 1 - s] w[k, c, r, s].
// The general backward-data kernel tiles 64 output channels, 61 of them
// zero here.  Instead the (channel, tap) pairs m = 9 c + 3 r + s are the
// rows of a GEMM: P[m, p] = sum_k w[k, m] g[k, p] for every pixel p of a
// band of th + 2 image rows (the band's th output rows and one row above
// and below), 27 of 32 MFMA rows, 32-pixel columns, the reduction over k.
// Lane l supplies B = g[k][p] for p = l % 32 of a 32-pixel block, one
// element per load, so a wave's load reads two 32-pixel runs of two g
// planes and g streams from HBM once with no transpose; A = w[k][m] comes
// from w^T staged in LDS and is held in registers.  float32 runs
// v_mfma_f32_32x32x2_f32, bfloat16 v_mfma_f32_32x32x16_bf16 (eight times
// fewer MFMA cycles for the same loads).  P goes to LDS, and each thread then adds the nine shifted taps of an
// output pixel per channel, in a fixed order.  Eight waves take the bands'
// 32-pixel blocks in turn, each loading its next block's operands while the
// MFMAs of the current one run.
// KS: g values a lane loads per 32-pixel block, K <= 2 KS.  FULL: K == 2 KS
// (no load of a block reads past the last channel).
template <typename T, int KS, bool FULL>
__global__ __launch_bounds__(512) void bwd_data_stem_kernel(
    const T* __restrict__ g, const T* __restrict__ w, float* __restrict__ dx, int N, int C,
    int K, int H, int W, int th, int bands, uint32_t g_bytes, int outb) {
  static_assert(2 * KS <= kStemBdMaxK, "w^T fits its LDS rows");
  __shared__ float ps[27 * kStemBdPx];  // P[m][band pixel]
  __shared__ float wt[kStemBdMaxK * 32];  // w^T: row k, column m (zero past 9C and K)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int n = blockIdx.x / bands, h0 = (blockIdx.x % bands) * th;
  const int nc = 9 * C;
  for (int e = tid; e < 2 * KS * 32; e += 512) {
    const int k = e >> 5, m = e & 31;
    wt[e] = (k < K && m < nc) ? widen(w[(long)k * nc + m]) : 0.f;
  }
  __syncthreads();
  const int px = (th + 2) * W;  // band pixels, rows h0 - 1 .. h0 + th
  const int nblk = (px + 31) / 32;
  const long hw = (long)H * W;
  const __amdgpu_buffer_rsrc_t gv = buffer_view(g, g_bytes);
  // bfloat16 runs v_mfma_f32_32x32x16_bf16 (products exact in float32, so
  // the same sums as float32 operands up to the order of additions): lane
  // (l32, hi) of step s supplies k = 16 s + 8 hi + j, j = 0..7, packed in
  // pairs.  float32 runs v_mfma_f32_32x32x2_f32: step i supplies
  // k = 2 i + hi.  Either way a lane loads KS values of g per block.
  constexpr bool BF = std::is_same<T, uint16_t>::value;
  constexpr int NS = BF ? KS / 8 : KS;  // MFMA steps per block
  using E = typename std::conditional<BF, uint32_t, float>::type;
  // A operands: this lane's column of w^T, the same for every block (the
  // staged w^T holds rows 0 .. 2 KS - 1, zero from K on)
  float wa[BF ? 1 : KS];
  u32x4 wb[BF ? NS : 1];
  if constexpr (BF) {
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int k = 16 * st + 8 * hi + 2 * d;
        // (staged values are bfloat16 widened: the high halves are exact)
        wb[st][d] = (__builtin_bit_cast(uint32_t, wt[k * 32 + l32]) >> 16) |
                    (__builtin_bit_cast(uint32_t, wt[(k + 1) * 32 + l32]) & 0xffff0000u);
      }
  } else {
#pragma unroll
    for (int i = 0; i < KS; ++i) wa[i] = wt[(2 * i + hi) * 32 + l32];
  }
  // B operands, two register sets that take the wave's blocks in turn.  A
  // block's KS loads form four quarters; loads run three quarters ahead of
  // the MFMAs (into the other set across a block boundary), so each wait
  // names loads issued three quarters earlier and leaves at most 3 KS / 4
  // younger ones in flight, within what a wait counter can name.  Rows
  // outside the image, pixels past the band (also blocks past the last)
  // and k >= K read zero.
  constexpr int QS = KS / 4;
  static_assert(!BF || QS % 8 == 0, "a quarter holds whole bf16 steps");
  E ba[KS], bb[KS];
  // Load i reads channel k(i) = k0 + dk(i), k0 = hi (float32) or 8 hi
  // (bfloat16), dk a compile-time step.  With FULL every k < K, so a lane's
  // offsets are one base (kOutside for a pixel outside the band or the
  // image: kOutside plus any in-range offset stays past the view) plus a
  // wave-uniform dk(i) planes -- one add per load; otherwise each load also
  // checks k < K.
  const uint32_t hwb = (uint32_t)hw * (uint32_t)sizeof(T);
  auto load_q = [&](E(&dst)[KS], int blk, int qi) __attribute__((always_inline)) {
    const int q = blk * 32 + l32;
    const int row = h0 - 1 + q / W, col = q % W;
    const bool in = q < px && row >= 0 && row < H;
    const int k0 = BF ? 8 * hi : hi;
    const uint32_t e0 = in ? (uint32_t)((long)n * K * hw + (long)row * W + col) : 0u;
    const uint32_t base = in ? (e0 + (uint32_t)k0 * (uint32_t)hw) * (uint32_t)sizeof(T) : kOutside;
#pragma unroll
    for (int i = qi * QS; i < (qi + 1) * QS; ++i) {
      const int dk = BF ? 16 * (i >> 3) + (i & 7) : 2 * i;
      const int k = k0 + dk;
      const uint32_t off = FULL ? base + (uint32_t)dk * hwb
                                : (in & (k < K) ? (e0 + (uint32_t)k * (uint32_t)hw) *
                                                      (uint32_t)sizeof(T)
                                                : kOutside);
      if constexpr (BF)
        dst[i] = buffer_load2(gv, off);
      else
        dst[i] = __builtin_bit_cast(float, buffer_load4(gv, off));
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto mfma_q = [&](f32x16& acc, const E(&src)[KS], int qi) __attribute__((always_inline)) {
    if constexpr (BF) {
#pragma unroll
      for (int st = qi * QS / 8; st < (qi + 1) * QS / 8; ++st) {
        u32x4 bw;
#pragma unroll
        for (int d = 0; d < 4; ++d) bw[d] = src[8 * st + 2 * d] | (src[8 * st + 2 * d + 1] << 16);
        acc = mfma_32x32x16_bf16(wb[st], bw, acc);
      }
    } else {
#pragma unroll
      for (int i = qi * QS; i < (qi + 1) * QS; ++i) acc = mfma_32x32x2_f32(wa[i], src[i], acc);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // one block (its first three quarters already requested), then P to LDS
  auto step = [&](int blk, E(&cur)[KS], E(&nxt)[KS]) __attribute__((always_inline)) {
    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
    load_q(cur, blk, 3);
    mfma_q(acc, cur, 0);
    load_q(nxt, blk + 8, 0);
    mfma_q(acc, cur, 1);
    load_q(nxt, blk + 8, 1);
    mfma_q(acc, cur, 2);
    load_q(nxt, blk + 8, 2);
    mfma_q(acc, cur, 3);
    const int q = blk * 32 + l32;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = acc_row(v, hi);
      if (m < 27) ps[m * kStemBdPx + q] = acc[v];
    }
  };
  // (the block index is wave-uniform, so the loop carries no exec masks)
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  load_q(ba, wv, 0);
  load_q(ba, wv, 1);
  load_q(ba, wv, 2);
  for (int blk = wv; blk < nblk; blk += 16) {
    step(blk, ba, bb);
    if (blk + 8 >= nblk) break;
    step(blk + 8, bb, ba);
  }
  __syncthreads();
  for (int o = tid; o < th * W; o += 512) {
    const int lr = o / W, j = o % W, i = h0 + lr;
    if (i >= H) continue;
    for (int c = 0; c < C; ++c) {
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int t = 0; t < 3; ++t) {
          // g pixel (i + 1 - r, j + 1 - t): band row lr + 2 - r; columns
          // outside the image add nothing
          const int pc = j + 1 - t;
          const bool ok = pc >= 0 && pc < W;
          const float v = ps[(c * 9 + r * 3 + t) * kStemBdPx + (lr + 2 - r) * W + (ok ? pc : j)];
          sum += ok ? v : 0.f;
        }
      const long e = (((long)n * C + c) * H + i) * W + j;
      if (outb)
        reinterpret_cast<uint16_t*>(dx)[e] = (uint16_t)bf16_rne(sum);
      else
        dx[e] = sum;
    }
  }
}

template <typename T>
static bool launch_bd_stem(const Plan& pl, const T* g, const T* w, float* dx, int N, int C,
                           int K, int H, int W, bool outb, hipStream_t stream) {
  if (!pl.stem || C > 3 || K > kStemBdMaxK || pl.th != stem_bd_rows(W) || pl.th < 1 ||
      pl.threads != 512)
    return false;
  const int bands = (H + pl.th - 1) / pl.th;
  const uint32_t gb = (uint32_t)((long)N * K * H * W * (long)sizeof(T));
  dim3 grid((unsigned)(N * bands)), block(512);
#define CONV3X3_BD(KS_, FULL_)                                                            \
  hipLaunchKernelGGL((bwd_data_stem_kernel<T, KS_, FULL_>), grid, block, 0, stream, g, w, dx, N, \
                     C, K, H, W, pl.th, bands, gb, outb ? 1 : 0)
  if (K == 64)
    CONV3X3_BD(32, true);
  else if (K < 64)
    CONV3X3_BD(32, false);
  else if (K == 128)
    CONV3X3_BD(64, true);
  else
    CONV3X3_BD(64, false);
#undef CONV3X3_BD
  return true;
}

bool launch_bwd_data_stem_f32(const Plan& pl, const float* g, const float* w, float* dx, int N,
                              int C, int K, int H, int W, hipStream_t stream) {
  return launch_bd_stem<float>(pl, g, w, dx, N, C, K, H, W, false, stream);
}

bool launch_bwd_data_stem_bf16(const Plan& pl, const uint16_t* g, const uint16_t* w, float* dx,
                               int N, int C, int K, int H, int W, bool outb,
                               hipStream_t stream) {
  return launch_bd_stem<uint16_t>(pl, g, w, dx, N, C, K, H, W, outb, stream);
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
