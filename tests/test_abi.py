"""CPU checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments with the documented status codes
before touching the GPU (no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import diffusion_unet_x3_amd as lib3

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "conv3x3.h")
L = lib3.lib
S = lib3.STATUS

# Distinct non-null fake device addresses: never dereferenced, because every
# call below fails validation first.
X, Wt, B, Y, G, WS, Z = (ctypes.c_void_p(0x10000 * (i + 1)) for i in range(7))


def _declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(conv3x3_[a-z_0-9]+)\s*\(", text)))


def test_header_functions_are_exported():
    names = _declared_functions()
    assert set(names) == set(lib3.EXPORTED), names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for code in range(11):
        assert lib3.conv3x3_status_string(code)
        assert "unknown status" not in lib3.conv3x3_status_string(code)
    assert lib3.conv3x3_status_string(0) == "success"
    assert "unknown" in lib3.conv3x3_status_string(99)


@pytest.mark.parametrize("dims", [(0, 1, 1, 1, 1), (1, 0, 1, 1, 1), (1, 1, 0, 1, 1),
                                  (1, 1, 1, 0, 1), (1, 1, 1, 1, 0), (-1, 4, 4, 4, 4),
                                  (2, 1 << 16, 4, 128, 128),      # x has 2^31 elements
                                  (1, 4, 1 << 16, 1 << 8, 1 << 7),  # y has 2^31 elements
                                  (1, 1 << 14, 1 << 14, 1, 1)])   # w has > 2^31 elements
def test_bad_shapes_rejected(dims):
    N, C, K, H, W = dims
    assert L.conv3x3_fwd(X, Wt, B, Y, N, C, K, H, W, 0, None) == S["ERR_BAD_SHAPE"]
    assert L.conv3x3_bwd_data(G, Wt, Y, N, C, K, H, W, 0, None) == S["ERR_BAD_SHAPE"]
    assert L.conv3x3_bwd_weight(X, G, Y, B, WS, 1 << 40, N, C, K, H, W, 0, None) == S["ERR_BAD_SHAPE"]
    assert L.conv3x3_bwd_weight_workspace_size(N, C, K, H, W, 0) == ctypes.c_size_t(-1).value


def test_null_pointers_rejected():
    d = (2, 3, 4, 5, 6)
    assert L.conv3x3_fwd(None, Wt, B, Y, *d, 0, None) == S["ERR_NULL_POINTER"]
    assert L.conv3x3_fwd(X, None, B, Y, *d, 0, None) == S["ERR_NULL_POINTER"]
    assert L.conv3x3_fwd(X, Wt, B, None, *d, 0, None) == S["ERR_NULL_POINTER"]
    assert L.conv3x3_bwd_data(None, Wt, Y, *d, 0, None) == S["ERR_NULL_POINTER"]
    assert L.conv3x3_bwd_data(G, Wt, None, *d, 0, None) == S["ERR_NULL_POINTER"]
    assert L.conv3x3_bwd_weight(None, G, Y, B, WS, 1 << 40, *d, 0, None) == S["ERR_NULL_POINTER"]
    assert L.conv3x3_bwd_weight(X, G, None, B, WS, 1 << 40, *d, 0, None) == S["ERR_NULL_POINTER"]


@pytest.mark.parametrize("dtype", [-1, 3, 7])
def test_bad_dtype_rejected(dtype):
    d = (2, 3, 4, 5, 6)
    assert L.conv3x3_fwd(X, Wt, B, Y, *d, dtype, None) == S["ERR_BAD_DTYPE"]
    assert L.conv3x3_bwd_data(G, Wt, Y, *d, dtype, None) == S["ERR_BAD_DTYPE"]
    assert L.conv3x3_bwd_weight(X, G, Y, B, WS, 1 << 40, *d, dtype, None) == S["ERR_BAD_DTYPE"]


def test_aliasing_rejected():
    d = (2, 3, 4, 5, 6)
    assert L.conv3x3_fwd(X, Wt, B, X, *d, 0, None) == S["ERR_ALIAS"]
    assert L.conv3x3_fwd(X, Wt, B, B, *d, 0, None) == S["ERR_ALIAS"]
    assert L.conv3x3_bwd_data(G, Wt, G, *d, 0, None) == S["ERR_ALIAS"]
    assert L.conv3x3_bwd_weight(X, G, X, B, WS, 1 << 40, *d, 0, None) == S["ERR_ALIAS"]
    assert L.conv3x3_bwd_weight(X, G, Y, Y, WS, 1 << 40, *d, 0, None) == S["ERR_ALIAS"]


def test_workspace_checked():
    N, C, K, H, W = 32, 64, 64, 64, 64
    need = lib3.conv3x3_bwd_weight_workspace_size(N, C, K, H, W)
    assert need > 0
    assert L.conv3x3_bwd_weight(X, G, Y, B, None, need, N, C, K, H, W, 0, None) == S["ERR_WORKSPACE"]
    assert L.conv3x3_bwd_weight(X, G, Y, B, WS, need - 1, N, C, K, H, W, 0, None) == S["ERR_WORKSPACE"]
    assert L.conv3x3_bwd_weight(X, G, Y, B, X, need, N, C, K, H, W, 0, None) == S["ERR_ALIAS"]


def test_plan_query_errors():
    p = lib3.Plan()
    assert L.conv3x3_plan(3, 1, 1, 1, 1, 1, 0, ctypes.byref(p)) == S["ERR_BAD_PASS"]
    assert L.conv3x3_plan(0, 1, 1, 1, 1, 1, 0, None) == S["ERR_NULL_POINTER"]
    assert L.conv3x3_plan(0, 1, 1, 1, 1, 1, 5, ctypes.byref(p)) == S["ERR_BAD_DTYPE"]


# ---- fused-activation entry points ------------------------------------------

@pytest.mark.parametrize("act", [-1, 3, 17])
def test_bad_activation_rejected(act):
    d = (2, 3, 4, 5, 6)
    assert L.conv3x3_fwd_act(X, Wt, B, Y, Z, *d, 0, act, None) == S["ERR_BAD_ACT"]
    assert L.conv3x3_bwd_data_act(G, Z, Wt, Y, *d, 0, act, None) == S["ERR_BAD_ACT"]
    assert L.conv3x3_bwd_weight_act(X, G, Z, Y, B, WS, 1 << 40, *d, 0, act, None) == \
        S["ERR_BAD_ACT"]


def test_activation_argument_checks():
    d = (2, 3, 4, 5, 6)
    silu = lib3.ACT_SILU
    # shapes, dtypes and required pointers as the plain entry points
    assert L.conv3x3_fwd_act(X, Wt, B, Y, Z, 0, 3, 4, 5, 6, 0, silu, None) == S["ERR_BAD_SHAPE"]
    assert L.conv3x3_fwd_act(None, Wt, B, Y, Z, *d, 0, silu, None) == S["ERR_NULL_POINTER"]
    assert L.conv3x3_fwd_act(X, Wt, B, Y, Z, *d, 3, silu, None) == S["ERR_BAD_DTYPE"]
    # z may not alias another argument
    assert L.conv3x3_fwd_act(X, Wt, B, Y, Y, *d, 0, silu, None) == S["ERR_ALIAS"]
    assert L.conv3x3_fwd_act(X, Wt, B, Y, X, *d, 0, silu, None) == S["ERR_ALIAS"]
    # the backward passes need z for any activation other than none ...
    assert L.conv3x3_bwd_data_act(G, None, Wt, Y, *d, 0, silu, None) == S["ERR_NULL_POINTER"]
    assert L.conv3x3_bwd_weight_act(X, G, None, Y, B, WS, 1 << 40, *d, 0, silu, None) == \
        S["ERR_NULL_POINTER"]
    assert L.conv3x3_bwd_data_act(G, Z, Wt, Z, *d, 0, silu, None) == S["ERR_ALIAS"]
    assert L.conv3x3_bwd_weight_act(X, G, Z, Z, B, WS, 1 << 40, *d, 0, silu, None) == \
        S["ERR_ALIAS"]
    # ... in both dtypes (bfloat16 validates like float32)
    assert L.conv3x3_bwd_data_act(G, None, Wt, Y, *d, 1, silu, None) == S["ERR_NULL_POINTER"]
    assert L.conv3x3_bwd_data_act(G, Z, Wt, Z, *d, 1, silu, None) == S["ERR_ALIAS"]
    assert L.conv3x3_bwd_weight_act(X, G, Z, Z, B, WS, 1 << 40, *d, 1, lib3.ACT_LRELU, None) == \
        S["ERR_ALIAS"]
    # workspace rules carry over
    N, C, K, H, W = 32, 64, 64, 64, 64
    need = lib3.conv3x3_bwd_weight_workspace_size(N, C, K, H, W)
    assert L.conv3x3_bwd_weight_act(X, G, Z, Y, B, WS, need - 1, N, C, K, H, W, 0, silu, None) == \
        S["ERR_WORKSPACE"]
    assert L.conv3x3_bwd_weight_act(X, G, Z, Y, B, Z, need, N, C, K, H, W, 0, silu, None) == \
        S["ERR_ALIAS"]


X1, DX0, DX1 = (ctypes.c_void_p(0x10000 * (i + 11)) for i in range(3))


@pytest.mark.parametrize("halves", [(-1, 4), (4, -1), (0, 0), (2**30, 2**30)])
def test_concat_bad_halves_rejected(halves):
    C0, C1 = halves
    bad = S["ERR_BAD_SHAPE"]
    assert L.conv3x3_fwd_cat(X, X1, C0, C1, Wt, B, Y, 2, 4, 5, 5, 0, None) == bad
    assert L.conv3x3_bwd_data_cat(G, Wt, DX0, DX1, C0, C1, 2, 4, 5, 5, 0, None) == bad
    assert L.conv3x3_bwd_weight_cat(X, X1, C0, C1, G, Y, B, WS, 1 << 30, 2, 4, 5, 5, 0,
                                    None) == bad
    assert L.conv3x3_bwd_weight_cat_workspace_size(2, C0, C1, 4, 5, 5, 0) == \
        ctypes.c_size_t(-1).value
    p = lib3.Plan()
    assert L.conv3x3_plan_cat(0, 2, C0, C1, 4, 5, 5, 0, ctypes.byref(p)) == bad


def test_concat_missing_half_rejected():
    null = S["ERR_NULL_POINTER"]
    # a half with channels needs its pointer
    assert L.conv3x3_fwd_cat(None, X1, 3, 4, Wt, B, Y, 2, 4, 5, 5, 0, None) == null
    assert L.conv3x3_fwd_cat(X, None, 3, 4, Wt, B, Y, 2, 4, 5, 5, 0, None) == null
    assert L.conv3x3_bwd_data_cat(G, Wt, None, DX1, 3, 4, 2, 4, 5, 5, 0, None) == null
    assert L.conv3x3_bwd_data_cat(G, Wt, DX0, None, 3, 4, 2, 4, 5, 5, 0, None) == null
    assert L.conv3x3_bwd_weight_cat(X, None, 3, 4, G, Y, B, WS, 1 << 30, 2, 4, 5, 5, 0,
                                    None) == null
    # an empty half may be NULL: the call then fails on the next check only
    # (a bad dtype here), not on the pointer
    bad_dtype = S["ERR_BAD_DTYPE"]
    assert L.conv3x3_fwd_cat(None, X1, 0, 4, Wt, B, Y, 2, 4, 5, 5, 7, None) == bad_dtype
    assert L.conv3x3_bwd_data_cat(G, Wt, DX0, None, 3, 0, 2, 4, 5, 5, 7, None) == bad_dtype


def test_concat_aliasing_rejected():
    alias = S["ERR_ALIAS"]
    assert L.conv3x3_fwd_cat(X, X1, 3, 4, Wt, B, X1, 2, 4, 5, 5, 0, None) == alias
    assert L.conv3x3_bwd_data_cat(G, Wt, DX0, DX0, 3, 4, 2, 4, 5, 5, 0, None) == alias
    assert L.conv3x3_bwd_data_cat(G, Wt, DX0, G, 3, 4, 2, 4, 5, 5, 0, None) == alias
    assert L.conv3x3_bwd_weight_cat(X, X1, 3, 4, G, X1, B, WS, 1 << 30, 2, 4, 5, 5, 0,
                                    None) == alias


def test_concat_plans_tile_each_half():
    """Channel tiles never straddle the two tensors: the bwd_data grid and the
    bwd_weight tile count are the sums over the halves."""
    p = lib3.conv3x3_plan_cat(lib3.PASS_BWD_DATA, 32, 100, 28, 256, 32, 32)
    q = lib3.conv3x3_plan(lib3.PASS_BWD_DATA, 32, 128, 256, 32, 32)
    m = p["tile_m"]
    assert p["grid_y"] == -(-100 // m) + -(-28 // m)
    assert q["grid_y"] == -(-128 // q["tile_m"])
    # halves that are whole tiles give the plain plan
    assert lib3.conv3x3_plan_cat(lib3.PASS_BWD_DATA, 32, 512, 128, 256, 32, 32) == \
        lib3.conv3x3_plan(lib3.PASS_BWD_DATA, 32, 640, 256, 32, 32)
    assert lib3.conv3x3_plan_cat(lib3.PASS_BWD_WEIGHT, 32, 512, 128, 256, 32, 32) == \
        lib3.conv3x3_plan(lib3.PASS_BWD_WEIGHT, 32, 640, 256, 32, 32)
    # an empty half is the plain plan too
    for pas in (0, 1, 2):
        assert lib3.conv3x3_plan_cat(pas, 4, 0, 24, 16, 9, 9) == \
            lib3.conv3x3_plan(pas, 4, 24, 16, 9, 9)
    # ragged halves: bwd_weight has one more 64-channel tile
    r = lib3.conv3x3_plan_cat(lib3.PASS_BWD_WEIGHT, 2, 40, 40, 64, 8, 8)
    assert r["workspace_bytes"] == \
        lib3.conv3x3_bwd_weight_cat_workspace_size(2, 40, 40, 64, 8, 8, 0)


SC, SH = (ctypes.c_void_p(0x10000 * (i + 21)) for i in range(2))


def test_prologue_argument_checks():
    d = (2, 4, 4, 5, 5)  # N, C, K, H, W
    null, unsup, alias = S["ERR_NULL_POINTER"], S["ERR_UNSUPPORTED"], S["ERR_ALIAS"]
    # scale and shift are required
    assert L.conv3x3_fwd_gnsilu(X, None, SH, Wt, B, Y, *d, 0, None) == null
    assert L.conv3x3_fwd_gnsilu(X, SC, None, Wt, B, Y, *d, 0, None) == null
    assert L.conv3x3_bwd_data_gnsilu(G, Wt, X, SC, None, Y, *d, 0, None) == null
    assert L.conv3x3_bwd_data_gnsilu(G, Wt, None, SC, SH, Y, *d, 0, None) == null
    assert L.conv3x3_bwd_weight_gnsilu(X, None, SH, G, Y, B, WS, 1 << 30, *d, 0, None) == null
    # both dtypes (bfloat16 validates like float32)
    assert L.conv3x3_fwd_gnsilu(X, SC, None, Wt, B, Y, *d, 1, None) == null
    assert L.conv3x3_fwd_gnsilu(X, SC, SH, Wt, B, SC, *d, 1, None) == alias
    assert L.conv3x3_bwd_data_gnsilu(G, Wt, X, SC, SH, X, *d, 1, None) == alias
    assert L.conv3x3_bwd_weight_gnsilu(X, SC, SH, G, SC, B, WS, 1 << 30, *d, 1, None) == alias
    # outputs may not alias scale / shift / x
    assert L.conv3x3_fwd_gnsilu(X, SC, SH, Wt, B, SC, *d, 0, None) == alias
    assert L.conv3x3_bwd_data_gnsilu(G, Wt, X, SC, SH, X, *d, 0, None) == alias
    assert L.conv3x3_bwd_data_gnsilu(G, Wt, X, SC, SH, SH, *d, 0, None) == alias
    assert L.conv3x3_bwd_weight_gnsilu(X, SC, SH, G, SC, B, WS, 1 << 30, *d, 0, None) == alias
    # backward-data's x must stay below 2 GiB (a 32-bit buffer view)
    big = (64, 1024, 4, 128, 128)
    assert L.conv3x3_bwd_data_gnsilu(G, Wt, X, SC, SH, Y, *big, 0, None) == unsup


def test_small_tile_split_rule():
    """With a workspace: bf16 32-image 8x8 layers with 512 channels split the
    eight-wave 256 x 128 tile's 32 fills in eight (32 tiles -> 256
    workgroups, 4 fills per slice); float32 64 x 64 tiles that make half a
    round to one round of workgroups split a reduction of at least 32
    fills (of 8 channels) in four."""
    bf16 = lib3.CONV3X3_BF16
    slot = 32 * 512 * 64 * 4  # one float32 output of a 32-image 8x8 layer with 512 channels
    for p in (lib3.PASS_FWD, lib3.PASS_BWD_DATA):
        assert lib3.conv3x3_workspace_size(p, 32, 512, 512, 8, 8, bf16) == 8 * slot
    # 384 input channels: a 24-fill forward reduction stays whole (a split
    # in two of its 32 big tiles would leave 64 workgroups), its 32-fill
    # backward-data (over 512 channels, 24 big tiles) splits in eight
    assert lib3.conv3x3_workspace_size(lib3.PASS_FWD, 32, 384, 512, 8, 8, bf16) == 0
    assert lib3.conv3x3_workspace_size(lib3.PASS_BWD_DATA, 32, 384, 512, 8, 8, bf16) == \
        8 * 32 * 384 * 64 * 4
    # 16x16, 384 -> 384: 24 fills, 96 big tiles split in two
    assert lib3.conv3x3_workspace_size(lib3.PASS_FWD, 32, 384, 384, 16, 16, bf16) == \
        2 * 32 * 384 * 256 * 4
    # a grid below half a round (4 images: 32 workgroups) is not split
    assert lib3.conv3x3_workspace_size(lib3.PASS_FWD, 4, 512, 512, 8, 8, bf16) == 0
    f32 = lib3.CONV3X3_F32
    for p in (lib3.PASS_FWD, lib3.PASS_BWD_DATA):
        assert lib3.conv3x3_workspace_size(p, 32, 512, 512, 8, 8, f32) == 4 * slot
    # float32, 128 channels: 16 fills, too short
    assert lib3.conv3x3_workspace_size(lib3.PASS_FWD, 32, 128, 512, 8, 8, f32) == 0
    # float32 16x16 images take 768 workgroups of the 64 x 64 tile: no split
    assert lib3.conv3x3_workspace_size(lib3.PASS_FWD, 32, 384, 384, 16, 16, f32) == 0
    # the resampling and prologue entry points take no workspace, so never split
    assert lib3.conv3x3_up2_workspace_size(lib3.PASS_FWD, 32, 512, 512, 16, 16, f32) == 0


def test_tiny_grid_split_rule():
    """float32 problems whose 64 x 64 tiles make at most 64 workgroups split
    the reduction in up to four slices of at least two 8-channel fills, no
    more than 256 / workgroups; bf16 and larger grids do not."""
    f32, bf16 = lib3.CONV3X3_F32, lib3.CONV3X3_BF16
    slot = 2 * 64 * 32 * 32 * 4  # one float32 output of N = 2, 64 channels, 32x32
    for p in (lib3.PASS_FWD, lib3.PASS_BWD_DATA):
        # 32 workgroups, 8 fills: four slices of two fills
        assert lib3.conv3x3_workspace_size(p, 2, 64, 64, 32, 32, f32) == 4 * slot
        # (the plan query describes the call without a workspace: unsplit)
        plan = lib3.conv3x3_plan(p, 2, 64, 64, 32, 32, f32)
        assert plan["split"] == 1 and plan["grid_x"] * plan["grid_y"] == 32
    # 24 channels (3 fills): one slice of at least two fills only
    assert lib3.conv3x3_workspace_size(lib3.PASS_FWD, 2, 24, 64, 32, 32, f32) == 0
    # 40 channels (5 fills): two slices (3 + 2 fills)
    assert lib3.conv3x3_workspace_size(lib3.PASS_FWD, 2, 40, 64, 32, 32, f32) == 2 * slot
    # 160 workgroups (N = 10) is more than a quarter round: no split
    assert lib3.conv3x3_workspace_size(lib3.PASS_FWD, 10, 64, 64, 32, 32, f32) == 0
    # 96 workgroups (N = 6) is too: 256 / 96 = 2 slices only at <= 64 workgroups
    assert lib3.conv3x3_workspace_size(lib3.PASS_FWD, 6, 64, 64, 32, 32, f32) == 0
    # 64 workgroups (N = 4): four slices
    assert lib3.conv3x3_workspace_size(lib3.PASS_FWD, 4, 64, 64, 32, 32, f32) == \
        4 * 2 * slot
    # bf16 stays whole
    assert lib3.conv3x3_workspace_size(lib3.PASS_FWD, 2, 64, 64, 32, 32, bf16) == 0


def test_split_workspace_checks():
    """A bf16 small-image problem needs a workspace on the *_ws entry
    points; without one, or with too little, nothing is launched."""
    d = (32, 1024, 512, 8, 8)
    bf16 = lib3.CONV3X3_BF16
    need = lib3.conv3x3_workspace_size(lib3.PASS_FWD, *d, bf16)
    assert need == 8 * (32 * 512 * 64 * 4)  # eight float32 output-sized slots
    # a 16-fill reduction (K = 256) is too short to split
    assert lib3.conv3x3_workspace_size(lib3.PASS_BWD_DATA, 32, 1024, 256, 8, 8, bf16) == 0
    # a split that would leave the grid at half a round is not taken
    assert lib3.conv3x3_workspace_size(lib3.PASS_FWD, 4, 1024, 512, 8, 8, bf16) == 0
    assert lib3.conv3x3_workspace_size(lib3.PASS_BWD_DATA, 32, 512, 1024, 8, 8, bf16) == need
    # float32: 128 fills of 8 channels on 256 workgroups of 64 x 64 tiles, four slices
    assert lib3.conv3x3_workspace_size(lib3.PASS_FWD, *d, lib3.CONV3X3_F32) == 4 * (32 * 512 * 64 * 4)
    assert lib3.conv3x3_workspace_size(lib3.PASS_FWD, 64, 512, 512, 16, 16, bf16) == 0
    assert lib3.conv3x3_workspace_size(lib3.PASS_BWD_WEIGHT, *d, bf16) == \
        lib3.conv3x3_bwd_weight_workspace_size(*d, bf16)
    ws_err, alias = S["ERR_WORKSPACE"], S["ERR_ALIAS"]
    assert L.conv3x3_fwd_ws(X, Wt, B, Y, None, 0, *d, bf16, None) == ws_err
    assert L.conv3x3_fwd_ws(X, Wt, B, Y, WS, need - 1, *d, bf16, None) == ws_err
    db = (32, 512, 1024, 8, 8)
    assert L.conv3x3_bwd_data_ws(G, Wt, Y, None, 0, *db, bf16, None) == ws_err
    assert L.conv3x3_fwd_ws(X, Wt, B, Y, X, need, *d, bf16, None) == alias
    assert L.conv3x3_bwd_data_ws(G, Wt, Y, Y, need, *db, bf16, None) == alias
    # the plain entry points never need one
    assert L.conv3x3_fwd_ws(X, Wt, B, Y, None, 0, *d, 7, None) == S["ERR_BAD_DTYPE"]
    assert lib3.conv3x3_plan(lib3.PASS_FWD, *d, bf16)["split"] == 1


def test_up2_argument_checks():
    d = (2, 4, 4, 5, 6)  # N, C, K, H, W of the small input
    unsup, alias = S["ERR_UNSUPPORTED"], S["ERR_ALIAS"]
    assert lib3.conv3x3_up2_workspace_size(lib3.PASS_FWD, *d) == 0
    assert lib3.conv3x3_up2_workspace_size(lib3.PASS_BWD_DATA, *d) == 0
    assert lib3.conv3x3_up2_workspace_size(lib3.PASS_BWD_WEIGHT, *d) == \
        lib3.conv3x3_bwd_weight_workspace_size(2, 4, 4, 10, 12)
    # bfloat16 inputs: float32 outputs only (no bf16-output mode)
    assert L.conv3x3_fwd_up2(X, Wt, B, Y, *d, 2, None) == unsup
    assert L.conv3x3_bwd_data_up2(G, Wt, Y, WS, 1 << 30, *d, 2, None) == unsup
    assert L.conv3x3_bwd_weight_up2(X, G, Y, B, WS, 1 << 30, *d, 2, None) == unsup
    assert L.conv3x3_fwd_up2(X, Wt, B, Y, 2, 4, 4, 0, 6, 0, None) == S["ERR_BAD_SHAPE"]
    # float32 backward-data needs no workspace; dx may not be g
    assert L.conv3x3_bwd_data_up2(G, Wt, G, None, 0, *d, 0, None) == alias
    assert L.conv3x3_fwd_up2(X, Wt, B, X, *d, 0, None) == alias
    # bfloat16 backward-data: the upsampled-grid float32 gradient in the
    # workspace, summed over 2 x 2 blocks afterwards
    need = 2 * 4 * 4 * 5 * 6 * 4
    assert lib3.conv3x3_up2_workspace_size(lib3.PASS_BWD_DATA, *d, 1) == need
    assert lib3.conv3x3_up2_workspace_size(lib3.PASS_FWD, *d, 1) == 0
    assert L.conv3x3_bwd_data_up2(G, Wt, Y, None, 0, *d, 1, None) == S["ERR_WORKSPACE"]
    assert L.conv3x3_bwd_data_up2(G, Wt, Y, WS, need - 1, *d, 1, None) == S["ERR_WORKSPACE"]
    assert L.conv3x3_bwd_data_up2(G, Wt, Y, G, need, *d, 1, None) == alias
    assert L.conv3x3_bwd_data_up2(G, Wt, Y, Y, need, *d, 1, None) == alias


def test_s2_argument_checks():
    d = (2, 4, 4, 6, 8)
    assert L.conv3x3_fwd_s2(X, Wt, B, Y, 2, 4, 4, 5, 8, 0, None) == S["ERR_BAD_SHAPE"]  # odd H
    assert L.conv3x3_bwd_data_s2(G, Wt, Y, 2, 4, 4, 6, 7, 0, None) == S["ERR_BAD_SHAPE"]
    # bfloat16 inputs with float32 outputs run; the bf16-output mode does not
    assert L.conv3x3_fwd_s2(X, Wt, B, Y, *d, 2, None) == S["ERR_UNSUPPORTED"]
    assert L.conv3x3_bwd_weight_s2(X, G, Y, B, WS, 1 << 30, *d, 2, None) == S["ERR_UNSUPPORTED"]
    assert L.conv3x3_bwd_weight_s2(X, G, Y, B, None, 0, 2, 64, 64, 64, 64, 1, None) == \
        S["ERR_WORKSPACE"]
    assert L.conv3x3_fwd_s2(None, Wt, B, Y, *d, 0, None) == S["ERR_NULL_POINTER"]
    assert L.conv3x3_fwd_s2(X, Wt, B, X, *d, 0, None) == S["ERR_ALIAS"]
    assert L.conv3x3_bwd_weight_s2(X, G, Y, B, None, 0, 2, 64, 64, 64, 64, 0, None) == \
        S["ERR_WORKSPACE"]


@pytest.mark.parametrize("dims", [(1, 1 << 13, 4, 256, 256),    # x: 2^29 floats = 2 GiB
                                  (2, 4, 1 << 12, 256, 256),    # y, g: 2 GiB
                                  (1, 1 << 13, 1 << 13, 1, 1)])  # w, dw: 2.25 GiB
def test_tensors_of_2gib_or_more_unsupported(dims):
    """Every tensor a call touches must be below 2 GiB (counted as float32):
    larger ones are refused before anything is enqueued."""
    N, C, K, H, W = dims
    un = S["ERR_UNSUPPORTED"]
    for dt in (0, 1):
        assert L.conv3x3_fwd(X, Wt, B, Y, N, C, K, H, W, dt, None) == un
        assert L.conv3x3_bwd_data(G, Wt, Y, N, C, K, H, W, dt, None) == un
        assert L.conv3x3_bwd_weight(X, G, Y, B, WS, 1 << 40, N, C, K, H, W, dt, None) == un
        assert L.conv3x3_fwd_ws(X, Wt, B, Y, WS, 1 << 40, N, C, K, H, W, dt, None) == un
        assert L.conv3x3_bwd_weight_noalloc(X, G, Y, B, N, C, K, H, W, dt, None) == un


def test_noalloc_argument_checks():
    """The no-allocation backward-weight validates like conv3x3_bwd_weight
    (no call here reaches the scratch lookup or a launch)."""
    d = (2, 3, 4, 5, 6)
    assert L.conv3x3_bwd_weight_noalloc(None, G, Y, B, *d, 0, None) == S["ERR_NULL_POINTER"]
    assert L.conv3x3_bwd_weight_noalloc(X, G, None, B, *d, 0, None) == S["ERR_NULL_POINTER"]
    assert L.conv3x3_bwd_weight_noalloc(X, G, Y, B, 0, 3, 4, 5, 6, 0, None) == S["ERR_BAD_SHAPE"]
    assert L.conv3x3_bwd_weight_noalloc(X, G, Y, B, *d, 7, None) == S["ERR_BAD_DTYPE"]
    assert L.conv3x3_bwd_weight_noalloc(X, G, X, B, *d, 0, None) == S["ERR_ALIAS"]
    assert "scratch" in lib3.conv3x3_status_string(S["ERR_NOALLOC"])


def test_noalloc_scratch_covers_every_plan():
    """The planner keeps split x channel tiles <= 256 (64 x 64 x 9 floats
    each), so no problem needs more split-K workspace than the
    no-allocation entry point's 40 MiB array."""
    limit = 40 << 20
    worst = 0
    for dt in (0, 1):
        for C in (1, 3, 17, 64, 65, 128, 200, 256, 384, 512, 640, 1024, 2048, 4096):
            for K in (1, 8, 64, 100, 128, 256, 512, 1024, 4096, 8192):
                for H in (1, 8, 16, 33, 64, 128):
                    for N in (1, 4, 32, 64):
                        n = L.conv3x3_bwd_weight_workspace_size(N, C, K, H, H, dt)
                        if n != ctypes.c_size_t(-1).value:
                            worst = max(worst, n)
    assert 30 << 20 < worst <= limit
