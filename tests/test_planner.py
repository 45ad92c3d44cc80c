"""CPU checks of the launch planner (through the C ABI's plan query): every
problem is tiled completely, LDS fits a gfx950 compute unit, the
backward-weight split never leaves a slice empty and its workspace formula
holds."""
import math

import pytest

import diffusion_unet_x3_amd as lib3
import workloads as wl

LDS_PER_CU = 160 * 1024
SHAPES = sorted({l.shape for c in wl.CONFIGS.values() for l in c} | set(wl.RAGGED_SHAPES))


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dtype", [0, 1])
def test_forward_type_plans_cover_problem(shape, dtype):
    N, C, K, H, W = shape
    for pass_, cout in ((lib3.PASS_FWD, K), (lib3.PASS_BWD_DATA, C)):
        p = lib3.conv3x3_plan(pass_, N, C, K, H, W, dtype)
        assert p["tile_n"] == p["tile_imgs"] * p["tile_h"] * p["tile_w"]
        tiles = (math.ceil(N / p["tile_imgs"]) * math.ceil(H / p["tile_h"]) *
                 math.ceil(W / p["tile_w"]))
        assert p["grid_x"] == tiles
        assert p["grid_y"] * p["tile_m"] >= cout > (p["grid_y"] - 1) * p["tile_m"]
        assert 0 < p["lds_bytes"] <= LDS_PER_CU
        assert p["threads"] in (256, 512) and p["split"] == 1 and p["workspace_bytes"] == 0


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dtype", [0, 1])
def test_forward_type_tiles_fit_the_image(shape, dtype):
    """On images of at least 8 x 8 pixels (the smallest block), a pixel block
    is never taller than the image rounded up to a power of two (a taller
    block only multiplies zero padding), and on layers whose images are a
    power of two on a side, at least half of the pixels the grid covers are
    pixels of the problem."""
    N, C, K, H, W = shape
    if H < 8 or W < 8:
        pytest.skip("image smaller than the smallest pixel block")
    hp = 1 << max(0, (H - 1).bit_length())
    for pass_, cout in ((lib3.PASS_FWD, K), (lib3.PASS_BWD_DATA, C)):
        p = lib3.conv3x3_plan(pass_, N, C, K, H, W, dtype)
        assert p["tile_h"] <= hp
        if H == hp and W == 1 << max(0, (W - 1).bit_length()):
            assert N * H * W >= 0.5 * p["grid_x"] * p["tile_n"]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dtype", [0, 1])
def test_weight_gradient_plans(shape, dtype):
    N, C, K, H, W = shape
    p = lib3.conv3x3_plan(lib3.PASS_BWD_WEIGHT, N, C, K, H, W, dtype)
    chunks = (math.ceil(N / p["tile_imgs"]) * math.ceil(H / p["tile_h"]) *
              math.ceil(W / p["tile_w"]))
    S = p["split"]
    assert 1 <= S <= chunks
    per = math.ceil(chunks / S)
    assert (S - 1) * per < chunks <= S * per  # no empty slice
    ws = lib3.conv3x3_bwd_weight_workspace_size(N, C, K, H, W, dtype)
    if C <= 4:
        # the packed-pair kernel: 128 k rows x all 9C pairs per 512-thread
        # workgroup, 64-pixel chunks, a workgroup per compute unit; slots of
        # K rows x 32 (C <= 3) or 64 columns; the reported workspace also
        # covers the general kernel's
        assert p["threads"] == 512 and p["tile_m"] == 128 and p["tile_n"] == C
        assert p["tile_imgs"] == 1 and p["tile_h"] * p["tile_w"] == 64
        assert p["tile_w"] >= min(W, 64) and p["tile_w"] in (8, 16, 32, 64)
        assert 0 < p["lds_bytes"] <= LDS_PER_CU
        tiles = math.ceil(K / 128)
        assert p["grid_x"] == S * tiles and S * tiles <= 256 or S == 1
        assert ws == p["workspace_bytes"]
        cols = 32 if C <= 3 else 64
        assert ws >= (0 if S == 1 else S * K * cols * 4)
        return
    tiles = math.ceil(C / p["tile_n"]) * math.ceil(K / p["tile_m"])
    # 1-D grid: S x tiles workgroups padded to whole rounds of the 8 XCDs
    assert p["grid_x"] % 8 == 0 and S * tiles <= p["grid_x"] < S * tiles + 8
    assert p["grid_y"] == 1 and p["grid_z"] == 1
    assert S * tiles <= 256 or S == 1
    assert 0 < p["lds_bytes"] <= LDS_PER_CU
    assert ws == p["workspace_bytes"]
    assert ws == (0 if S == 1 else S * (K * C * 9 + K) * 4)


@pytest.mark.parametrize("shape,dtype", [((2, 24, 40, 9, 80), 0), ((1, 16, 16, 4, 136), 0),
                                         ((2, 32, 48, 9, 80), 1), ((1, 16, 32, 4, 136), 1)])
def test_wide_parity_shapes_span_several_tiles(shape, dtype):
    """The parity shapes that exercise halo-column loads really put more than
    one tile across the width in every pass (with a single tile the halo
    columns are padding and the kernels load nothing for them)."""
    N, C, K, H, W = shape
    for pass_ in (lib3.PASS_FWD, lib3.PASS_BWD_DATA, lib3.PASS_BWD_WEIGHT):
        p = lib3.conv3x3_plan(pass_, N, C, K, H, W, dtype)
        assert math.ceil(W / p["tile_w"]) > 1


@pytest.mark.parametrize("dtype", [lib3.CONV3X3_F32, lib3.CONV3X3_BF16])
def test_few_channel_backward_data_plans(dtype):
    """At most three dx channels and 128 g channels: one 512-thread
    workgroup per band of output rows (8, fewer for rows wider than 64
    pixels) whose band plus one halo row above and below fits 640 pixels;
    rows of 214+ pixels, 129 g channels and four dx channels take the
    general kernel."""
    bd = lib3.PASS_BWD_DATA
    p = lib3.conv3x3_plan(bd, 32, 3, 128, 64, 64, dtype)
    assert (p["tile_m"], p["threads"], p["tile_h"], p["tile_w"]) == (3, 512, 8, 64)
    assert p["grid_x"] == 32 * 8 and p["split"] == 1 and p["workspace_bytes"] == 0
    for W, th in ((1, 8), (64, 8), (65, 7), (100, 4), (200, 1), (213, 1)):
        p = lib3.conv3x3_plan(bd, 2, 2, 16, 13, W, dtype)
        assert p["tile_m"] == 2 and p["tile_h"] == th, (W, p)
        assert (th + 2) * W <= 640
        assert p["grid_x"] == 2 * math.ceil(13 / th)
    for shape in ((2, 3, 16, 13, 214), (2, 3, 129, 8, 8), (2, 4, 16, 8, 8)):
        assert lib3.conv3x3_plan(bd, *shape, dtype)["tile_m"] >= 64, shape
