/*
 * conv3x3 reference oracle -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  It shares no code, header, table or helper with the
 * HIP library: it is plain C that accumulates every sum in IEEE double, one
 * output element at a time, in a fixed order.
 *
 * What it computes (the plainest reading of the sources):
 *   The sourcepulse summary of the C++/CUDA UNet project ("How It Works",
 *   "Highlighted Details") describes hand-written 3x3 convolution kernels,
 *   forward and backward, for a diffusion UNet whose parameters are created by
 *   a PyTorch script ("Quick Start & Requirements") and whose speed is
 *   compared with PyTorch's.  We therefore read the operation as PyTorch's
 *   Conv2d with kernel 3x3, stride 1, zero padding 1, dilation 1, groups 1,
 *   on NCHW activations and OIHW ([K][C][3][3]) weights, i.e. a
 *   cross-correlation:
 *
 *     y [n,k,h,w] = b[k] + sum_{c,r,s} x[n,c,h+r-1,w+s-1] * wt[k,c,r,s]
 *     dx[n,c,h,w] = sum_{k,r,s} g[n,k,h-r+1,w-s+1] * wt[k,c,r,s]
 *     dw[k,c,r,s] = sum_{n,h,w} g[n,k,h,w] * x[n,c,h+r-1,w+s-1]
 *     db[k]       = sum_{n,h,w} g[n,k,h,w]
 *
 *   where any x or g index outside the H x W image reads as zero.  dx, dw and
 *   db are the gradients of L = <y, g> with respect to x, wt and b (the
 *   "backward pass" of "Highlighted Details" / "Limitations & Caveats").
 *
 * Every function takes double arrays; callers widen float32 / bfloat16 inputs
 * to double, which is exact.  Outputs are overwritten.  Each output element's
 * sum runs in the order written below, so results are bitwise reproducible
 * for any number of OpenMP threads.
 *
 * Pins (tests/test_oracle_*.py): hand-computed 3x3 cases (tests/golden),
 * delta / shift / identity invariants, bilinearity, the adjoint identities,
 * central finite differences of L, and torch.nn.functional.conv2d in float64.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define IDX4(a, b, c, d, B, C, D) ((((int64_t)(a) * (B) + (b)) * (C) + (c)) * (D) + (d))

/* One forward output element: bias first, then channels, then taps r, s. */
static double fwd_one(const double* x, const double* wt, const double* b,
                      int C, int K, int H, int W, int n, int k, int h, int w) {
  double acc = b ? b[k] : 0.0;
  (void)K;
  for (int c = 0; c < C; ++c) {
    for (int r = 0; r < 3; ++r) {
      int ih = h + r - 1;
      if (ih < 0 || ih >= H) continue;
      for (int s = 0; s < 3; ++s) {
        int iw = w + s - 1;
        if (iw < 0 || iw >= W) continue;
        acc += x[IDX4(n, c, ih, iw, C, H, W)] * wt[IDX4(k, c, r, s, C, 3, 3)];
      }
    }
  }
  return acc;
}

/* One input-gradient element: output channels, then taps r, s. */
static double bwd_data_one(const double* g, const double* wt,
                           int C, int K, int H, int W, int n, int c, int h, int w) {
  double acc = 0.0;
  for (int k = 0; k < K; ++k) {
    for (int r = 0; r < 3; ++r) {
      int oh = h - r + 1;
      if (oh < 0 || oh >= H) continue;
      for (int s = 0; s < 3; ++s) {
        int ow = w - s + 1;
        if (ow < 0 || ow >= W) continue;
        acc += g[IDX4(n, k, oh, ow, K, H, W)] * wt[IDX4(k, c, r, s, C, 3, 3)];
      }
    }
  }
  return acc;
}

/* One weight-gradient element: images, then rows, then columns. */
static double bwd_weight_one(const double* x, const double* g,
                             int N, int C, int K, int H, int W, int k, int c, int r, int s) {
  double acc = 0.0;
  for (int n = 0; n < N; ++n) {
    for (int h = 0; h < H; ++h) {
      int ih = h + r - 1;
      if (ih < 0 || ih >= H) continue;
      for (int w = 0; w < W; ++w) {
        int iw = w + s - 1;
        if (iw < 0 || iw >= W) continue;
        acc += g[IDX4(n, k, h, w, K, H, W)] * x[IDX4(n, c, ih, iw, C, H, W)];
      }
    }
  }
  return acc;
}

/* One bias-gradient element: images, then rows, then columns. */
static double bias_grad_one(const double* g, int N, int K, int H, int W, int k) {
  double acc = 0.0;
  for (int n = 0; n < N; ++n)
    for (int h = 0; h < H; ++h)
      for (int w = 0; w < W; ++w) acc += g[IDX4(n, k, h, w, K, H, W)];
  return acc;
}

static int bad_dims(int N, int C, int K, int H, int W) {
  return N < 1 || C < 1 || K < 1 || H < 1 || W < 1;
}

/* ---- whole-tensor entry points ------------------------------------------ */

int oracle_conv3x3_fwd(const double* x, const double* wt, const double* b, double* y,
                       int N, int C, int K, int H, int W) {
  if (!x || !wt || !y || bad_dims(N, C, K, H, W)) return 1;
  int64_t total = (int64_t)N * K * H * W;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < total; ++i) {
    int w = (int)(i % W);
    int h = (int)((i / W) % H);
    int k = (int)((i / ((int64_t)W * H)) % K);
    int n = (int)(i / ((int64_t)W * H * K));
    y[i] = fwd_one(x, wt, b, C, K, H, W, n, k, h, w);
  }
  return 0;
}

int oracle_conv3x3_bwd_data(const double* g, const double* wt, double* dx,
                            int N, int C, int K, int H, int W) {
  if (!g || !wt || !dx || bad_dims(N, C, K, H, W)) return 1;
  int64_t total = (int64_t)N * C * H * W;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < total; ++i) {
    int w = (int)(i % W);
    int h = (int)((i / W) % H);
    int c = (int)((i / ((int64_t)W * H)) % C);
    int n = (int)(i / ((int64_t)W * H * C));
    dx[i] = bwd_data_one(g, wt, C, K, H, W, n, c, h, w);
  }
  return 0;
}

int oracle_conv3x3_bwd_weight(const double* x, const double* g, double* dw, double* db,
                              int N, int C, int K, int H, int W) {
  if (!x || !g || !dw || bad_dims(N, C, K, H, W)) return 1;
  int64_t total = (int64_t)K * C * 9;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < total; ++i) {
    int s = (int)(i % 3);
    int r = (int)((i / 3) % 3);
    int c = (int)((i / 9) % C);
    int k = (int)(i / ((int64_t)9 * C));
    dw[i] = bwd_weight_one(x, g, N, C, K, H, W, k, c, r, s);
  }
  if (db) {
#pragma omp parallel for schedule(static)
    for (int k = 0; k < K; ++k) db[k] = bias_grad_one(g, N, K, H, W, k);
  }
  return 0;
}

/* ---- sampled entry points: out[i] = the full result at flat index idx[i] --
 * Each output element is an independent sum, so a sample of elements of a
 * large problem is computed exactly as the whole-tensor call would.          */

int oracle_conv3x3_fwd_at(const double* x, const double* wt, const double* b,
                          int N, int C, int K, int H, int W,
                          const int64_t* idx, int64_t count, double* out) {
  if (!x || !wt || !out || (count > 0 && !idx) || bad_dims(N, C, K, H, W)) return 1;
  int64_t total = (int64_t)N * K * H * W;
  for (int64_t j = 0; j < count; ++j)
    if (idx[j] < 0 || idx[j] >= total) return 2;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t j = 0; j < count; ++j) {
    int64_t i = idx[j];
    int w = (int)(i % W);
    int h = (int)((i / W) % H);
    int k = (int)((i / ((int64_t)W * H)) % K);
    int n = (int)(i / ((int64_t)W * H * K));
    out[j] = fwd_one(x, wt, b, C, K, H, W, n, k, h, w);
  }
  return 0;
}

int oracle_conv3x3_bwd_data_at(const double* g, const double* wt,
                               int N, int C, int K, int H, int W,
                               const int64_t* idx, int64_t count, double* out) {
  if (!g || !wt || !out || (count > 0 && !idx) || bad_dims(N, C, K, H, W)) return 1;
  int64_t total = (int64_t)N * C * H * W;
  for (int64_t j = 0; j < count; ++j)
    if (idx[j] < 0 || idx[j] >= total) return 2;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t j = 0; j < count; ++j) {
    int64_t i = idx[j];
    int w = (int)(i % W);
    int h = (int)((i / W) % H);
    int c = (int)((i / ((int64_t)W * H)) % C);
    int n = (int)(i / ((int64_t)W * H * C));
    out[j] = bwd_data_one(g, wt, C, K, H, W, n, c, h, w);
  }
  return 0;
}

int oracle_conv3x3_bwd_weight_at(const double* x, const double* g,
                                 int N, int C, int K, int H, int W,
                                 const int64_t* idx, int64_t count, double* out) {
  if (!x || !g || !out || (count > 0 && !idx) || bad_dims(N, C, K, H, W)) return 1;
  int64_t total = (int64_t)K * C * 9;
  for (int64_t j = 0; j < count; ++j)
    if (idx[j] < 0 || idx[j] >= total) return 2;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t j = 0; j < count; ++j) {
    int64_t i = idx[j];
    int s = (int)(i % 3);
    int r = (int)((i / 3) % 3);
    int c = (int)((i / 9) % C);
    int k = (int)(i / ((int64_t)9 * C));
    out[j] = bwd_weight_one(x, g, N, C, K, H, W, k, c, r, s);
  }
  return 0;
}

int oracle_conv3x3_bias_grad_at(const double* g, int N, int K, int H, int W,
                                const int64_t* idx, int64_t count, double* out) {
  if (!g || !out || (count > 0 && !idx) || bad_dims(N, 1, K, H, W)) return 1;
  for (int64_t j = 0; j < count; ++j)
    if (idx[j] < 0 || idx[j] >= K) return 2;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t j = 0; j < count; ++j) out[j] = bias_grad_one(g, N, K, H, W, (int)idx[j]);
  return 0;
}

/* ---- fused activation ------------------------------------------------------
 * The project-guide page on StyleGAN2's custom CUDA kernels describes fusing a
 * bias and an activation (a leaky ReLU that comes with a bias term) into one
 * operation, to save memory traffic; the diffusion UNet's activation is SiLU.
 * Read as: the forward convolution's output with its bias, z, goes through
 *   act 0: identity     act(z) = z
 *   act 1: SiLU         act(z) = z * sigmoid(z)
 *   act 2: leaky ReLU   act(z) = z (z >= 0), 0.2 z (z < 0)   (no gain)
 * and the backward pass multiplies the gradient arriving at act's output, gy,
 * by act'(z) to get the convolution's output gradient g = gy * act'(z).  The
 * derivatives, written out from the definitions:
 *   SiLU:        act'(z) = s (1 + z (1 - s)),  s = sigmoid(z) = 1 / (1 + e^-z)
 *   leaky ReLU:  act'(z) = 1 for z > 0, 0.2 otherwise (z = 0 takes the slope)
 */
static double act_value(int act, double z) {
  if (act == 1) return z / (1.0 + exp(-z));
  if (act == 2) return z >= 0.0 ? z : 0.2 * z;
  return z;
}

static double act_slope(int act, double z) {
  if (act == 1) {
    double sg = 1.0 / (1.0 + exp(-z));
    return sg * (1.0 + z * (1.0 - sg));
  }
  if (act == 2) return z > 0.0 ? 1.0 : 0.2;
  return 1.0;
}

static int bad_act(int act) { return act < 0 || act > 2; }

int oracle_act_forward(const double* z, double* y, int64_t n, int act) {
  if (!z || !y || n < 0 || bad_act(act)) return 1;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) y[i] = act_value(act, z[i]);
  return 0;
}

int oracle_act_grad(const double* gy, const double* z, double* g, int64_t n, int act) {
  if (!gy || !z || !g || n < 0 || bad_act(act)) return 1;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) g[i] = gy[i] * act_slope(act, z[i]);
  return 0;
}

/* Number of OpenMP threads the whole-tensor calls use (for reporting). */
int oracle_num_threads(void) {
  int n = 1;
#ifdef _OPENMP
#pragma omp parallel
  {
#pragma omp single
    n = omp_get_num_threads();
  }
#endif
  return n;
}
