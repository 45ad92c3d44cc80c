/*
 * conv3x3.h -- C ABI of the gfx950 (MI355X) 3x3 convolution library.
 *
 * The operation is the stride-1, zero-padding-1 3x3 convolution that the
 * sourcepulse summary of the C++/CUDA diffusion-UNet project singles out as
 * the layer worth hand-written kernels ("How It Works"; forward timings and
 * the forward/backward comparison with PyTorch in "Highlighted Details";
 * the lagging backward pass in "Limitations & Caveats").  The model is built
 * by a PyTorch script ("Quick Start & Requirements"), so the operation is read
 * as PyTorch's Conv2d(kernel 3, stride 1, padding 1) -- a cross-correlation:
 *
 *   y [n,k,h,w] = bias[k] + sum_{c,r,s} x[n,c,h+r-1,w+s-1] * w[k,c,r,s]
 *   dx[n,c,h,w] = sum_{k,r,s} g[n,k,h-r+1,w-s+1] * w[k,c,r,s]
 *   dw[k,c,r,s] = sum_{n,h,w} g[n,k,h,w] * x[n,c,h+r-1,w+s-1]
 *   db[k]       = sum_{n,h,w} g[n,k,h,w]
 *
 * with x, g read as zero outside the H x W image.  dx, dw, db are the
 * gradients of <y, g> with respect to x, w and bias.
 *
 * Layouts (all dense, row-major, no strides):
 *   x, dx : [N][C][H][W]      g, y : [N][K][H][W]
 *   w, dw : [K][C][3][3]      bias, db : [K]
 *
 * dtype (the `dtype` argument):
 *   CONV3X3_F32  : x, w, g are float32.
 *   CONV3X3_BF16 : x, w, g are bfloat16 (raw 16-bit patterns); products are
 *                  exact and accumulate in float32.
 *   In both modes bias is float32 and every output (y, dx, dw, db) is float32.
 *   CONV3X3_BF16_IO : as CONV3X3_BF16, but y and dx (the activations and
 *                  input gradients that the next layer reads) are written
 *                  as bfloat16, rounded to nearest even from the float32
 *                  accumulators; dw, db (and a fused activation's z) stay
 *                  float32.  Halves the bytes of the two largest stores.
 *
 * Memory and ownership: every pointer is a device pointer (hipMalloc'd or
 * torch-allocated) owned by the caller.  The library allocates nothing and
 * is safe to call from several host threads; its only global state is the
 * scratch array of conv3x3_bwd_weight_noalloc (see there).  Outputs are overwritten, never accumulated into.  Outputs must
 * not alias inputs (identical base pointers are rejected; partial overlap is
 * undefined).  No alignment is required: 128-bit paths are used when the
 * base address and row length allow it.
 *
 * Streams and errors: work is enqueued on `stream` (NULL = the null stream)
 * and the call returns without synchronising.  Argument errors return a
 * nonzero status BEFORE anything is enqueued.  A failed launch returns
 * CONV3X3_ERR_HIP.  Faults inside a kernel surface at the caller's next
 * synchronisation, as usual for HIP.
 *
 * Graph capture: a call enqueues only kernel launches on `stream` -- no
 * allocation, memset, copy, event or synchronisation -- so a caller may
 * capture calls into a HIP graph (hipStreamBeginCapture on a non-null
 * stream) and replay it; each replay recomputes every output from the
 * pointers captured, bit for bit as the eager call (the kernels are
 * deterministic).  Workspaces must stay allocated while the graph lives.
 *
 * Size limits: N, C, K, H, W >= 1; every tensor holds fewer than 2^31
 * elements (else CONV3X3_ERR_BAD_SHAPE).  The compute entry points also
 * need every tensor they touch below 2 GiB counted as float32 -- N*C*H*W,
 * N*K*H*W and 9*K*C each below 2^29, H x W being the call's largest grid --
 * because the kernels address tensors through 32-bit buffer offsets; larger
 * problems return CONV3X3_ERR_UNSUPPORTED before anything is enqueued
 * (the plan and workspace-size queries still answer for them).
 */
#ifndef CONV3X3_H
#define CONV3X3_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t, declared here so that C callers need no HIP
 * headers.  NULL selects the null stream. */
typedef struct ihipStream_t* conv3x3_stream_t;

typedef enum {
  CONV3X3_F32 = 0,
  CONV3X3_BF16 = 1,
  CONV3X3_BF16_IO = 2
} conv3x3_dtype_t;

typedef enum {
  CONV3X3_OK = 0,
  CONV3X3_ERR_NULL_POINTER = 1, /* a required pointer is NULL */
  CONV3X3_ERR_BAD_SHAPE = 2,    /* a dimension < 1, or a tensor >= 2^31 elements */
  CONV3X3_ERR_BAD_DTYPE = 3,    /* dtype is not a conv3x3_dtype_t value */
  CONV3X3_ERR_WORKSPACE = 4,    /* workspace NULL or smaller than required */
  CONV3X3_ERR_ALIAS = 5,        /* an output shares its base pointer with an input */
  CONV3X3_ERR_HIP = 6,          /* the HIP runtime rejected a launch */
  CONV3X3_ERR_BAD_PASS = 7,     /* conv3x3_plan: unknown pass */
  CONV3X3_ERR_BAD_ACT = 8,      /* act is not a conv3x3_act_t value */
  CONV3X3_ERR_UNSUPPORTED = 9,  /* a fusion this dtype (or size) does not provide */
  CONV3X3_ERR_NOALLOC = 10      /* conv3x3_bwd_weight_noalloc: the problem needs more than
                                   CONV3X3_NOALLOC_SCRATCH_BYTES of scratch, or the stream
                                   is not on the current device */
} conv3x3_status_t;

/*
 * Activation fused into the convolution (the *_act entry points).  The
 * project-guide page on StyleGAN2's custom CUDA kernels fuses a bias and an
 * activation -- a leaky ReLU with a bias term -- into one kernel to save a
 * round trip through memory; here the activation is applied to the biased
 * convolution output z = conv(x; w) + bias:
 *   CONV3X3_ACT_NONE  : act(z) = z
 *   CONV3X3_ACT_SILU  : act(z) = z * sigmoid(z)            (the UNet's)
 *   CONV3X3_ACT_LRELU : act(z) = z (z >= 0), 0.2 z (z < 0)  (no gain)
 * The backward entry points take gy, the gradient at the activation's
 * output, and z, and run the convolution backward on g = gy * act'(z), with
 * act'(z) = s (1 + z (1 - s)), s = sigmoid(z), for SiLU and 1 (z > 0) or
 * 0.2 (z <= 0) for the leaky ReLU.
 */
typedef enum {
  CONV3X3_ACT_NONE = 0,
  CONV3X3_ACT_SILU = 1,
  CONV3X3_ACT_LRELU = 2
} conv3x3_act_t;

typedef enum {
  CONV3X3_PASS_FWD = 0,
  CONV3X3_PASS_BWD_DATA = 1,
  CONV3X3_PASS_BWD_WEIGHT = 2
} conv3x3_pass_t;

/*
 * Forward with fused bias:  y = conv(x; w) + bias.
 *   x    : [N][C][H][W], dtype          w : [K][C][3][3], dtype
 *   bias : [K] float32, or NULL for no bias
 *   y    : [N][K][H][W] float32 (overwritten); for CONV3X3_BF16_IO bfloat16,
 *          the pointer then addressing 16-bit values
 * Implicit GEMM with M = N*H*W pixels, N = K output channels and a
 * reduction of length 9*C; input tiles and their one-pixel halo are staged
 * in LDS, the products run on MFMA.
 */
int conv3x3_fwd(const void* x, const void* w, const float* bias, float* y,
                int N, int C, int K, int H, int W, int dtype,
                conv3x3_stream_t stream);

/*
 * Backward-data:  dx = gradient of <conv(x; w), g> with respect to x.
 *   g  : [N][K][H][W], dtype      w : [K][C][3][3], dtype
 *   dx : [N][C][H][W] float32 (overwritten); bfloat16 for CONV3X3_BF16_IO
 * The same implicit GEMM as the forward pass over g, with the weight tile
 * transposed (k <-> c) and rotated by 180 degrees while it is staged in LDS.
 * dx with at most 3 channels (an image's gradient), K <= 128 and W <= 213
 * (plain call, no fusion, g under 2 GiB) takes a kernel of its own: the
 * 9*C (channel, tap) pairs are the rows of P = w^T g over bands of image
 * rows, and each dx element is the sum of its nine shifted taps of P.
 */
int conv3x3_bwd_data(const void* g, const void* w, float* dx,
                     int N, int C, int K, int H, int W, int dtype,
                     conv3x3_stream_t stream);

/*
 * Bytes of device workspace conv3x3_bwd_weight needs for this problem
 * (0 if it needs none).  Returns (size_t)-1 for invalid arguments.
 */
size_t conv3x3_bwd_weight_workspace_size(int N, int C, int K, int H, int W, int dtype);

/*
 * Backward-weight and bias gradient:
 *   x  : [N][C][H][W], dtype      g : [N][K][H][W], dtype
 *   dw : [K][C][3][3] float32 (overwritten)
 *   db : [K] float32 (overwritten), or NULL to skip the bias gradient
 *   workspace : device buffer of at least
 *               conv3x3_bwd_weight_workspace_size(...) bytes (may be NULL
 *               when that size is 0); its contents are scratch.
 * The pixel reduction (length N*H*W) is split into slices whose partial sums
 * are written to the workspace and then added in a fixed order by a second
 * kernel on the same stream: no atomics, bitwise-reproducible results.
 */
int conv3x3_bwd_weight(const void* x, const void* g, float* dw, float* db,
                       void* workspace, size_t workspace_bytes,
                       int N, int C, int K, int H, int W, int dtype,
                       conv3x3_stream_t stream);

/*
 * Backward-weight without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same operation, arguments, kernels
 * and results as conv3x3_bwd_weight (bitwise), but the split-K partial sums
 * go to a device array the library holds: CONV3X3_NOALLOC_SCRATCH_BYTES per
 * GPU, reserved when the library's code is loaded on that GPU and held
 * until the process ends.  The call allocates nothing.  Its device address
 * is looked up once per device, on the first call that needs it (with the
 * stream's device current).
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (two streams, or two host threads) race and give undefined results.
 *   Calls in one stream are ordered and safe.  Each call writes every
 *   scratch byte it later reads, so nothing needs clearing between calls.
 * Errors: as conv3x3_bwd_weight, plus CONV3X3_ERR_NOALLOC when the problem's
 * workspace size (conv3x3_bwd_weight_workspace_size) exceeds the array or
 * the stream belongs to another device than the current one, and
 * CONV3X3_ERR_HIP when the array's address cannot be found.  The planner
 * never splits beyond 256 slice-tiles of 64 x 64 x 9 floats, so every
 * valid problem fits (the largest needs about 36.1 MiB).
 */
#define CONV3X3_NOALLOC_SCRATCH_BYTES ((size_t)40 << 20)

int conv3x3_bwd_weight_noalloc(const void* x, const void* g, float* dw, float* db,
                               int N, int C, int K, int H, int W, int dtype,
                               conv3x3_stream_t stream);

/*
 * Forward with fused bias and activation:  z = conv(x; w) + bias,  y = act(z).
 *   x, w, bias, y : as conv3x3_fwd (y now holds act(z))
 *   z   : [N][K][H][W] float32 (overwritten), or NULL when not needed; the
 *         backward entry points below take it
 *   act : conv3x3_act_t
 * The activation is applied to the accumulators as they are stored (no
 * extra pass over y).  Errors as conv3x3_fwd, plus CONV3X3_ERR_BAD_ACT.
 */
int conv3x3_fwd_act(const void* x, const void* w, const float* bias, float* y, float* z,
                    int N, int C, int K, int H, int W, int dtype, int act,
                    conv3x3_stream_t stream);

/*
 * Backward-data through the activation:  dx = conv3x3_bwd_data(g = gy * act'(z), w).
 *   gy : [N][K][H][W], dtype (the gradient at the activation's output)
 *   z  : [N][K][H][W] float32, the forward's pre-activation (may be NULL
 *        only when act is CONV3X3_ACT_NONE)
 *   w, dx : as conv3x3_bwd_data
 * g is formed as gy and z are staged into LDS; it never exists in memory.
 * bfloat16 modes: gy is bfloat16 and z float32; the contraction's operand g
 * is bfloat16, formed in float32 as gy * act'(z) and rounded to nearest
 * even (so it can differ from the exact product's rounding by one bfloat16
 * step in rare elements).
 */
int conv3x3_bwd_data_act(const void* gy, const float* z, const void* w, float* dx,
                         int N, int C, int K, int H, int W, int dtype, int act,
                         conv3x3_stream_t stream);

/*
 * Backward-weight and bias gradient through the activation:
 *   dw, db = conv3x3_bwd_weight(x, g = gy * act'(z)); arguments as
 *   conv3x3_bwd_weight, plus gy / z / act as conv3x3_bwd_data_act (same
 *   workspace size and the same bfloat16 rounding of g; db is the sum of
 *   that g).
 */
int conv3x3_bwd_weight_act(const void* x, const void* gy, const float* z, float* dw, float* db,
                           void* workspace, size_t workspace_bytes,
                           int N, int C, int K, int H, int W, int dtype, int act,
                           conv3x3_stream_t stream);

/*
 * Concatenated input (a UNet's up-path blocks take the channel
 * concatenation [x0 ; x1] of the upsampled features and the skip tensor --
 * the standard UNet that the sourcepulse summary's "How It Works" builds).
 * These entry points run the convolution of that concatenation with C0 + C1
 * input channels, reading x0 ([N][C0][H][W]) and x1 ([N][C1][H][W]) where
 * they are: the concatenated tensor is never formed.  w is
 * [K][C0 + C1][3][3] (channels 0..C0-1 act on x0).  Backward-data writes the
 * input gradient's two halves, dx0 [N][C0][H][W] and dx1 [N][C1][H][W].
 * C0 >= 0, C1 >= 0, C0 + C1 >= 1; a half with no channels is not read or
 * written and its pointer may be NULL (the call is then the plain one).
 * Otherwise arguments, dtypes, limits (on C = C0 + C1), ownership and errors
 * are those of the plain entry points.  Every workgroup reads (or writes)
 * one half, so there is no per-element selection; a half whose channel count
 * is not a multiple of the channel tile costs one partly filled tile.
 */
int conv3x3_fwd_cat(const void* x0, const void* x1, int C0, int C1, const void* w,
                    const float* bias, float* y, int N, int K, int H, int W, int dtype,
                    conv3x3_stream_t stream);

int conv3x3_bwd_data_cat(const void* g, const void* w, float* dx0, float* dx1, int C0, int C1,
                         int N, int K, int H, int W, int dtype, conv3x3_stream_t stream);

/* Workspace bytes of conv3x3_bwd_weight_cat ((size_t)-1 for invalid
 * arguments); it can differ from the plain size for C0 + C1 channels. */
size_t conv3x3_bwd_weight_cat_workspace_size(int N, int C0, int C1, int K, int H, int W,
                                             int dtype);

int conv3x3_bwd_weight_cat(const void* x0, const void* x1, int C0, int C1, const void* g,
                           float* dw, float* db, void* workspace, size_t workspace_bytes, int N,
                           int K, int H, int W, int dtype, conv3x3_stream_t stream);

/*
 * Input prologue: GroupNorm-apply + SiLU fused into the convolution's input
 * loader -- the input-side counterpart of the fused bias + activation of the
 * project-guide page on StyleGAN2's custom kernels, as a UNet residual block
 * uses it before its convolution.  The convolution's input is
 *   a = SiLU(u),  u = x * scale[n, c] + shift[n, c],
 * zero-padded after the activation; scale and shift ([N][C] float32) fold a
 * GroupNorm's statistics and affine parameters into one multiplier and one
 * offset per sample and channel (computing them is the caller's).  a is
 * formed as x is staged and never exists in memory.
 *
 *   conv3x3_fwd_gnsilu        : y = conv(a; w) + bias (as conv3x3_fwd)
 *   conv3x3_bwd_data_gnsilu   : du = conv3x3_bwd_data(g, w) * SiLU'(u), the
 *                               gradient with respect to u (what a GroupNorm
 *                               backward takes); x, scale, shift are the
 *                               forward's and du is [N][C][H][W] float32
 *                               (bfloat16 for CONV3X3_BF16_IO)
 *   conv3x3_bwd_weight_gnsilu : dw, db of the convolution on a (as
 *                               conv3x3_bwd_weight, same workspace size)
 *
 * bfloat16 modes: x is bfloat16 and the contraction's operand a is
 * bfloat16, rounded to the nearest bfloat16 value (ties to even) as the
 * exact SiLU(x * scale + shift) rounds; du is not rounded (float32, unless
 * CONV3X3_BF16_IO).  scale and shift must not be NULL.  Other arguments,
 * limits and errors as the plain passes.
 */
int conv3x3_fwd_gnsilu(const void* x, const float* scale, const float* shift, const void* w,
                       const float* bias, float* y, int N, int C, int K, int H, int W, int dtype,
                       conv3x3_stream_t stream);

int conv3x3_bwd_data_gnsilu(const void* g, const void* w, const void* x, const float* scale,
                            const float* shift, float* du, int N, int C, int K, int H, int W,
                            int dtype, conv3x3_stream_t stream);

int conv3x3_bwd_weight_gnsilu(const void* x, const float* scale, const float* shift,
                              const void* g, float* dw, float* db, void* workspace,
                              size_t workspace_bytes, int N, int C, int K, int H, int W,
                              int dtype, conv3x3_stream_t stream);

/*
 * Forward / backward-data with a caller-provided workspace.  Same operation,
 * arguments and results as conv3x3_fwd / conv3x3_bwd_data, plus
 *   workspace : device buffer of at least conv3x3_workspace_size(pass, ...)
 *               bytes (may be NULL when that size is 0); its contents are
 *               scratch, it must not overlap an input or output.
 * With a workspace, a problem whose output tiles are too few to fill the
 * device splits its channel reduction over several workgroups per tile:
 *   - bfloat16, largest tile (256 pixels x 128 channels) short of a round of
 *     256 workgroups and at least 24 fills of 16 channels: 2 to 8 slices of
 *     at least 4 fills (only 2 slices below 32 fills), as long as the split
 *     grid reaches 192 workgroups;
 *   - either dtype, smallest tile (64 x 64) whose grid is 128 to 256
 *     workgroups, with at least 32 fills (16 channels bfloat16, 8 float32):
 *     2 slices (bfloat16) or 4 (float32);
 *   - float32, smallest tile with at most 64 workgroups and at least 4
 *     fills of 8 channels: up to 4 slices of at least 2 fills, no more than
 *     256 / workgroups.
 * Plain passes only (no activation, prologue, resampling or concatenation).
 * Each slice writes its partial sums (float32, one output-sized slot per
 * slice) to the workspace and a second kernel on the same stream adds the
 * slots in slice order -- no atomics, bitwise-reproducible results (which
 * can differ in the last bits from the unsplit entry points: another
 * summation order).  The plan's `split` field reports the slices.
 */
size_t conv3x3_workspace_size(int pass, int N, int C, int K, int H, int W, int dtype);

int conv3x3_fwd_ws(const void* x, const void* w, const float* bias, float* y, void* workspace,
                   size_t workspace_bytes, int N, int C, int K, int H, int W, int dtype,
                   conv3x3_stream_t stream);

int conv3x3_bwd_data_ws(const void* g, const void* w, float* dx, void* workspace,
                        size_t workspace_bytes, int N, int C, int K, int H, int W, int dtype,
                        conv3x3_stream_t stream);

/*
 * Nearest-neighbour 2x upsampling fused into the convolution's loader (a
 * UNet up block).  The project-guide page on StyleGAN2's custom kernels
 * describes upsampling as zero insertion followed by an FIR filter;
 * nearest-neighbour is its 2x2 box-filter case.  Here H, W are x's sizes:
 *   x  : [N][C][H][W]                the small input
 *   y  : [N][K][2H][2W]              y = conv(upsample2(x); w) + bias,
 *                                    upsample2(x)[n,c,i,j] = x[n,c,i/2,j/2]
 *   g  : [N][K][2H][2W]              the gradient at y
 *   dx : [N][C][H][W]                the sum of the input gradient over each
 *                                    2x2 block of the upsampled grid
 * The upsampled tensor never exists.  Forward: each output pixel parity
 * class (2i + ph, 2j + pw) is a 2x2-tap convolution of x whose weights are
 * sums of the 3x3 taps (kernel rows {0}, {1, 2} on x rows i - 1, i for
 * ph = 0; {0, 1}, {2} on rows i, i + 1 for ph = 1; likewise columns).
 * Backward-data: dx[i, j] gathers g rows and columns 2i - 1 .. 2i + 2 at
 * stride 2 with a 4 x 4 kernel of summed taps.  Backward-weight's loader
 * reads x at (h/2, w/2) as it stages the upsampled tile.  The summed taps
 * round differently from the upsampled-grid sums (within the float32 bar).
 * CONV3X3_BF16 (bfloat16 x, w, g; float32 y, dx, dw, db) runs the stride-1
 * bfloat16 kernels over the 2H x 2W grid instead: the forward and
 * backward-weight stage x read at (h/2, w/2) (no summed taps, so every
 * product is one of the upsampled grid's); backward-data writes the
 * upsampled grid's float32 input gradient into the workspace and then sums
 * each 2 x 2 block into dx.  Workspace bytes:
 * conv3x3_up2_workspace_size(pass, ...) -- 0 for the forward (whose
 * workspace arguments may be NULL, 0); for backward-data 0 for float32 and
 * N * C * 2H * 2W * 4 for bfloat16; the split-K size of the 2H x 2W
 * problem for backward-weight.  A bfloat16 backward-data workspace that
 * overlaps g, w or dx is CONV3X3_ERR_ALIAS.  CONV3X3_BF16_IO is
 * CONV3X3_ERR_UNSUPPORTED; the limits apply to the 2H x 2W problem.
 */
size_t conv3x3_up2_workspace_size(int pass, int N, int C, int K, int H, int W, int dtype);

int conv3x3_fwd_up2(const void* x, const void* w, const float* bias, float* y, int N, int C,
                    int K, int H, int W, int dtype, conv3x3_stream_t stream);

int conv3x3_bwd_data_up2(const void* g, const void* w, float* dx, void* workspace,
                         size_t workspace_bytes, int N, int C, int K, int H, int W, int dtype,
                         conv3x3_stream_t stream);

int conv3x3_bwd_weight_up2(const void* x, const void* g, float* dw, float* db, void* workspace,
                           size_t workspace_bytes, int N, int C, int K, int H, int W, int dtype,
                           conv3x3_stream_t stream);

/*
 * Stride-2 3x3 convolution, zero padding 1 (a UNet's downsample block; the
 * StyleGAN2 page's downsampling keeps every second sample after filtering):
 * y[n,k,h,w] = bias[k] + sum x[n,c,2h+r-1,2w+s-1] w[k,c,r,s].  H, W are x's
 * sizes and must be even; y, g are [N][K][H/2][W/2]; dx is [N][C][H][W];
 * backward-weight takes the workspace of conv3x3_bwd_weight_workspace_size
 * (N, C, K, H, W, dtype) (its plan over the H/2 x W/2 grid never needs
 * more).  The forward and backward-weight tile the H/2 x W/2 output and
 * stage x at stride 2; backward-data tiles g's grid and computes the four
 * output-pixel parity classes (dx[2i + ph, 2j + pw] takes the taps r = 1 for
 * ph = 0, r = 0 and 2 for ph = 1, likewise s and pw) from one staged tile.
 * No float32 pass multiplies inserted zeros.  CONV3X3_BF16 (bfloat16 x, w,
 * g; float32 outputs) runs the stride-1 bfloat16 kernels over the full
 * H x W grid: the forward keeps the even output pixels, backward-data and
 * backward-weight read g zero-inserted (g[i/2, j/2] at even (i, j), zero
 * elsewhere), so they spend four times the float32 paths' multiplies.
 * CONV3X3_BF16_IO is CONV3X3_ERR_UNSUPPORTED.
 */
int conv3x3_fwd_s2(const void* x, const void* w, const float* bias, float* y, int N, int C,
                   int K, int H, int W, int dtype, conv3x3_stream_t stream);

int conv3x3_bwd_data_s2(const void* g, const void* w, float* dx, int N, int C, int K, int H,
                        int W, int dtype, conv3x3_stream_t stream);

int conv3x3_bwd_weight_s2(const void* x, const void* g, float* dw, float* db, void* workspace,
                          size_t workspace_bytes, int N, int C, int K, int H, int W, int dtype,
                          conv3x3_stream_t stream);

/* Human-readable text for a status code (static storage). */
const char* conv3x3_status_string(int status);

/*
 * Launch plan the library would use for a pass (host only; no GPU needed).
 * Lets callers and tests see tile shapes, grid, LDS use and split factor.
 */
typedef struct {
  int pass;            /* conv3x3_pass_t */
  int dtype;           /* conv3x3_dtype_t */
  int kernel;          /* fwd/bwd_data: waves along the channel tile (1 or 2); else 0 */
  int tile_m;          /* rows of the WG tile: output channels (fwd, bwd_data) or k (bwd_weight) */
  int tile_n;          /* columns of the WG tile: pixels (fwd, bwd_data) or input channels (bwd_weight) */
  int tile_imgs;       /* pixel tile = tile_imgs x tile_h x tile_w */
  int tile_h;
  int tile_w;
  int chunk;           /* reduction chunk staged per LDS fill: channels, or pixels (bwd_weight) */
  int threads;         /* threads per workgroup */
  int grid_x, grid_y, grid_z;
  int lds_bytes;       /* static LDS per workgroup */
  int split;           /* reduction slices (1 = none): bwd_weight's split-K, and the
                          forward / backward-data split of conv3x3_workspace_size */
  size_t workspace_bytes;
} conv3x3_plan_t;

int conv3x3_plan(int pass, int N, int C, int K, int H, int W, int dtype,
                 conv3x3_plan_t* out);

/* The plan of a *_cat call (C0 + C1 channels in two tensors). */
int conv3x3_plan_cat(int pass, int N, int C0, int C1, int K, int H, int W, int dtype,
                     conv3x3_plan_t* out);

#ifdef __cplusplus
}
#endif

#endif /* CONV3X3_H */
