"""GPU parity of the split-reduction bf16 forward / backward-data (the *_ws
entry points on small images) against the oracle, through the C ABI.

Each slice of the channel reduction writes float32 partial sums to the
workspace and a second kernel adds them in slice order.  Same bar as the
plain bf16 passes (the 1e-4 trip-wire; exact on integer inputs, where the
split and unsplit entry points must also agree bit for bit)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import TRIPWIRE, rel_err

pytestmark = pytest.mark.gpu

# (N, C, K, H, W): few output tiles and a long reduction.  1032 channels
# leave a partly filled last fill and a short last slice.
# Shapes that take a split plan in forward and / or backward-data: 8x8 and
# 16x16 images, 24 to 65 fills (1032 channels: a ragged last fill), split
# grids of 192 and 256 workgroups; 512 -> 512 at 8x8 splits in eight slices
# of 4 fills, 520 channels in seven (five fills each, a last one of three),
# 384 -> 384 at 16x16 its 24 fills in two, and 392 -> 384 only its
# backward-data (a ragged last channel tile).
SHAPES = [(32, 1024, 512, 8, 8), (24, 1032, 512, 8, 8), (24, 1024, 128, 16, 16),
          (48, 256, 1024, 8, 8), (32, 512, 384, 16, 16),
          (32, 512, 512, 8, 8), (32, 384, 512, 8, 8), (32, 520, 512, 8, 8),
          (32, 384, 384, 16, 16), (24, 392, 384, 16, 16)]


def _run(inp, split, out_dtype=None):
    import diffusion_unet_x3_amd as lib3
    dev = torch.device("cuda", 0)
    x, w, g, b = (inp[k].to(dev) for k in ("x", "w", "g", "b"))
    y = lib3.conv3x3_fwd(x, w, b, out_dtype=out_dtype, split=split)
    dx = lib3.conv3x3_bwd_data(g, w, out_dtype=out_dtype, split=split)
    torch.cuda.synchronize()
    return y.float().cpu().double().numpy(), dx.float().cpu().double().numpy()


@pytest.mark.parametrize("integer", [False, True], ids=["random", "integer"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_split_reduction_full_compare(shape, integer):
    import diffusion_unet_x3_amd as lib3
    N, C, K, H, W = shape
    assert any(lib3.conv3x3_workspace_size(p, *shape, lib3.CONV3X3_BF16) > 0
               for p in (lib3.PASS_FWD, lib3.PASS_BWD_DATA)), "shape no longer takes a split plan"
    layer = wl.small_layer(*shape, dtype="bf16", seed=71)
    print(f"[parity] split {shape} integer={integer}", flush=True)
    inp = wl.make_inputs(layer, integer_exact=integer)
    y, dx = _run(inp, split=True)
    y_ref = oracle.conv3x3_fwd(inp["x"], inp["w"], inp["b"])
    dx_ref = oracle.conv3x3_bwd_data(inp["g"], inp["w"])
    if integer:
        assert np.array_equal(y, y_ref) and np.array_equal(dx, dx_ref)
        y0, dx0 = _run(inp, split=False)
        assert np.array_equal(y, y0) and np.array_equal(dx, dx0)
    else:
        errs = {"y": rel_err(y, y_ref), "dx": rel_err(dx, dx_ref)}
        print(errs)
        for k, e in errs.items():
            assert e <= TRIPWIRE["bf16"], (shape, k, e)


def test_split_reduction_bf16_outputs():
    """The reduce kernel writes bfloat16 outputs too (integer inputs:
    exactly the oracle rounded to bfloat16)."""
    import diffusion_unet_x3_amd as lib3
    assert lib3.conv3x3_workspace_size(lib3.PASS_FWD, 48, 1024, 256, 8, 8, lib3.CONV3X3_BF16) > 0
    layer = wl.small_layer(48, 1024, 256, 8, 8, dtype="bf16", seed=73)
    inp = wl.make_inputs(layer, integer_exact=True)
    y, dx = _run(inp, split=True, out_dtype=torch.bfloat16)
    assert np.array_equal(y, oracle.round_to_bf16(oracle.conv3x3_fwd(inp["x"], inp["w"],
                                                                     inp["b"])))
    assert np.array_equal(dx, oracle.round_to_bf16(oracle.conv3x3_bwd_data(inp["g"], inp["w"])))


def test_split_reduction_is_reproducible():
    layer = wl.small_layer(4, 1024, 128, 8, 8, dtype="bf16", seed=79)
    inp = wl.make_inputs(layer)
    a = _run(inp, split=True)
    b = _run(inp, split=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# float32: fills of 8 channels, four slices; 8x8 images whose 64 x 64 tiles
# make half a round to one round of workgroups, 32+ fills.  520 channels:
# 65 fills, slices of 17, 17, 17 and 14; 384 -> 512: a 48-fill forward and a 64-fill
# backward-data; 1024 -> 512: only the forward splits (backward-data has
# 512 workgroups).
# Beyond 8x8 tiles: 32x32 (32 x 2 tile) and 16x16 (16 x 4 tile) images with
# 64 fills; 514 channels take the scalar staging path.
# Grids of at most 64 workgroups (a small batch of small images), up to four
# slices of at least two fills: 2 x 64 -> 64 at 32x32 (32 workgroups, four
# slices of two fills), 40 -> 48 channels (two slices of 3 + 2 fills, a
# partial channel tile), a 31 x 33 image on the scalar path (62 workgroups),
# and 33 channels on a 5x7 image (one workgroup, the last fill one channel).
F32_SHAPES = [(32, 512, 512, 8, 8), (24, 520, 512, 8, 8), (32, 384, 512, 8, 8),
              (32, 1024, 512, 8, 8), (2, 512, 512, 32, 32), (8, 512, 512, 16, 16),
              (24, 514, 512, 8, 8),
              (2, 64, 64, 32, 32), (2, 40, 48, 32, 32), (2, 64, 64, 31, 33), (1, 33, 8, 5, 7)]


@pytest.mark.parametrize("integer", [False, True], ids=["random", "integer"])
@pytest.mark.parametrize("shape", F32_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_split_reduction_f32_full_compare(shape, integer):
    import diffusion_unet_x3_amd as lib3
    assert lib3.conv3x3_workspace_size(lib3.PASS_FWD, *shape, lib3.CONV3X3_F32) > 0, \
        "shape no longer takes a split plan"
    layer = wl.small_layer(*shape, dtype="f32", seed=83)
    print(f"[parity] f32 split {shape} integer={integer}", flush=True)
    inp = wl.make_inputs(layer, integer_exact=integer)
    y, dx = _run(inp, split=True)
    y_ref = oracle.conv3x3_fwd(inp["x"], inp["w"], inp["b"])
    dx_ref = oracle.conv3x3_bwd_data(inp["g"], inp["w"])
    if integer:
        assert np.array_equal(y, y_ref) and np.array_equal(dx, dx_ref)
        y0, dx0 = _run(inp, split=False)
        assert np.array_equal(y, y0) and np.array_equal(dx, dx0)
    else:
        errs = {"y": rel_err(y, y_ref), "dx": rel_err(dx, dx_ref)}
        print(errs)
        for k, e in errs.items():
            assert e <= TRIPWIRE["f32"], (shape, k, e)


def test_split_reduction_f32_is_reproducible():
    layer = wl.small_layer(32, 512, 512, 8, 8, dtype="f32", seed=89)
    inp = wl.make_inputs(layer)
    a = _run(inp, split=True)
    b = _run(inp, split=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
