// Launch planning for the 3x3 convolution kernels (host only, no HIP calls).
//
// The forward and backward-data passes are one implicit GEMM: rows are
// output channels (K for the forward pass, C for backward-data), columns are
// output pixels (M = N*H*W), and the reduction runs over 9 taps x input
// channels.  A workgroup owns a tile of `tile_co` output channels by a pixel
// block of tile_imgs x tile_h x tile_w pixels; the reduction is staged in
// LDS `chunk` input channels at a time.
//
// The backward-weight pass is the GEMM dw[k, (c, tap)] = sum_pixels
// g[k, p] * x[c, p + tap offset]: a workgroup owns 64 k x 64 c x 9 taps and
// walks a slice of the pixel reduction, `chunk` pixels per LDS fill; the
// reduction is split into `split` slices whose partial sums are added by a
// second kernel in a fixed order.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace conv3x3 {

enum Pass { kFwd = 0, kBwdData = 1, kBwdWeight = 2 };
enum DType { kF32 = 0, kBF16 = 1 };

struct Plan {
  int pass = 0;
  int dtype = 0;
  int tile_co = 0;    // fwd/bwd_data: output channels per WG; bwd_weight: k per WG
  int wave_co = 0;    // fwd/bwd_data: waves along the channel dimension
  int tile_ci = 0;    // bwd_weight: input channels per WG
  int tw = 0, th = 0, imgs = 0;  // pixel block (fwd/bwd_data) or chunk (bwd_weight)
  int chunk = 0;      // channels (fwd/bwd_data) or pixels (bwd_weight) per LDS fill
  int threads = 256;
  int tiles_w = 0, tiles_h = 0, tiles_n = 0;
  int grid_x = 0, grid_y = 0, grid_z = 0;
  int lds_bytes = 0;
  int split = 1;          // reduction slices (bwd_weight; bf16 fwd / bwd_data with a workspace)
  int chunks_per_split = 0;
  int nchunks = 0;
  int vec = 0;            // 1: 128-bit global paths allowed (decided at launch; 0 here)
  int stem = 0;           // fwd / bwd_weight: the packed-pair kernel (at most four input
                          // channels); bwd_data: the (channel, tap)-row kernel (at most three)
  size_t workspace_bytes = 0;
};

// Problem dims as the implicit GEMM sees them.  For backward-data the
// "input" channels are K (g is the input) and the output channels are C.
// C0: when x (and dx) is the concatenation of two tensors, the channels of
// the first; -1 (or C) for one tensor.  Channel tiles never straddle the two
// tensors, so the number of C tiles is that of each tensor added.
struct Problem {
  int pass, dtype;
  int N, C, K, H, W;
  int C0 = -1;
  // bf16 forward / backward-data: the caller provides a workspace, so the
  // reduction may be split over several workgroups per output tile (partial
  // sums in the workspace, then a fixed-order reduce)
  bool allow_split = false;
  // float32 passes that stage their source at stride 2, H, W being the
  // output's: the stride-2 forward / backward-weight (x tiles of 2 th + 1
  // input rows of 2 tw + 1 columns) and the upsampling backward-data (g
  // tiles of 2 th + 2 rows of 2 tw + 2 columns)
  bool stride2 = false;
  // float32 passes that keep one accumulator set per output-pixel parity
  // class (stride-2 backward-data, upsampling forward; H, W the grid they
  // tile): 64 x 64 tiles, one 32 x 32 MFMA tile per wave and set
  bool quad = false;
  // bfloat16 backward-data with a fused activation gradient: four-wave
  // tiles only (their staging threads hold the float32 z rows beside gy)
  bool four_waves = false;
  // at most four input channels in one tensor: the packed-pair kernels --
  // backward-weight without fusion (512 threads, 128 k x all (c, tap) pairs
  // per workgroup, 64-pixel chunks), bfloat16 forward without fusion and
  // with float32 outputs (256 threads, 64 output channels x 128-pixel
  // tiles, persistent); at most three output channels: the (channel,
  // tap)-row backward-data (512 threads, one band of image rows per
  // workgroup; see stem_bwd_data_fits)
  bool stem = false;
};

bool plan(const Problem& p, Plan* out);

// Whether the (channel, tap)-row backward-data takes a problem: at most three
// dx channels, at most 128 g channels, and image rows narrow enough for a
// band of at least one output row in LDS (at most 213 pixels).
bool stem_bwd_data_fits(int C, int K, int W);

// Minimum workspace bytes for a bwd_weight plan.
size_t wgrad_workspace_bytes(const Plan& pl, int C, int K);

// Elements of one partial-output slot of a split fwd / bwd_data plan.
long fwd_slot_elems(const Problem& p);

}  // namespace conv3x3
