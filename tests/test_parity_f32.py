"""GPU parity of the float32 path against the fp64 oracle, through the C ABI.

Bar: max|err| / max|ref| <= 2e-5 per output tensor (y, dx, dw, db) on seeded
random inputs, and exact equality on integer-valued inputs (every product
and partial sum is then exact in float32, in any summation order, so any
dropped tap, halo or split-K slice shows).  Small and ragged shapes are
compared element by element on whole tensors; the full-size UNet layers in
the launch configuration the benchmark times are compared on sampled output
elements, each computed on its own by the oracle."""
import numpy as np
import pytest

import workloads as wl
from parity_util import check, oracle_full, oracle_sampled, pairs, run_gpu

pytestmark = pytest.mark.gpu

SMALL = [(2, 64, 64, 32, 32)] + wl.RAGGED_SHAPES + [
    (2, 40, 130, 10, 70),   # C not a multiple of the chunk, K over two tiles, W over 64
    (1, 130, 20, 6, 12),    # many channel chunks, small K
    (3, 8, 8, 17, 8),       # W = 8 tiles, H over 16
    (5, 16, 16, 8, 8),      # 8x8 images in pairs, odd image count
    (2, 32, 72, 16, 16),
    (2, 24, 40, 9, 80),     # vector path, two tiles across the width (halo columns loaded)
    (1, 16, 16, 4, 136),    # vector path, three tiles across the width
]


def _flush(label):
    print(f"[parity] {label}", flush=True)


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("exact", [False, True], ids=["random", "integer"])
def test_small_shapes_full_compare(shape, exact):
    layer = wl.small_layer(*shape, dtype="f32", seed=11)
    _flush(f"f32 small {shape} exact={exact}")
    inp = wl.make_inputs(layer, integer_exact=exact)
    gpu = run_gpu(inp)
    ref = oracle_full(inp)
    check(pairs(gpu, ref), "f32", exact=exact, label=str(shape))


# Shapes whose forward or backward-data plan is one of the large tiles
# (256 pixels x 64 channels, 128 x 128, and a ragged channel tile), small
# enough for a full oracle compare.
LARGE_TILES = [((16, 8, 64, 64, 64), "fwd"), ((16, 8, 64, 64, 64), "bwd_data"),
               ((32, 8, 128, 32, 32), "fwd"), ((32, 128, 8, 32, 32), "bwd_data"),
               ((16, 8, 200, 32, 32), "fwd"), ((16, 200, 8, 32, 32), "bwd_data")]


@pytest.mark.parametrize("case", LARGE_TILES, ids=lambda c: "x".join(map(str, c[0])) + "-" + c[1])
@pytest.mark.parametrize("exact", [False, True], ids=["random", "integer"])
def test_large_tiles_full_compare(case, exact):
    import diffusion_unet_x3_amd as lib3
    shape, pass_name = case
    pass_id = lib3.PASS_FWD if pass_name == "fwd" else lib3.PASS_BWD_DATA
    p = lib3.conv3x3_plan(pass_id, *shape, lib3.CONV3X3_F32)
    assert p["tile_m"] * p["tile_n"] == 16384, "shape no longer selects a large tile"
    layer = wl.small_layer(*shape, dtype="f32", seed=31)
    _flush(f"f32 large tile {shape} {pass_name} exact={exact}")
    inp = wl.make_inputs(layer, integer_exact=exact)
    gpu = run_gpu(inp)
    ref = oracle_full(inp)
    check(pairs(gpu, ref), "f32", exact=exact, label=str(shape))


def test_no_bias_and_no_db():
    layer = wl.small_layer(2, 24, 40, 9, 20, dtype="f32", seed=3)
    inp = wl.make_inputs(layer)
    gpu = run_gpu(inp, want_db=False, with_bias=False)
    ref = oracle_full(inp, with_bias=False)
    ref["db"] = None
    check(pairs(gpu, ref), "f32", label="nobias")


def test_config_small_2x64_32x32_seeded():
    layer = wl.CONFIGS[1][0]
    _flush(layer.name)
    inp = wl.make_inputs(layer)
    gpu = run_gpu(inp)
    errs = check(pairs(gpu, oracle_full(inp)), "f32", label=layer.name)
    print(errs)


F32_FULL = wl.CONFIGS[2] + wl.CONFIGS[3] + [l for l in wl.CONFIGS[5] if l.dtype == "f32"]


@pytest.mark.parametrize("layer", F32_FULL, ids=lambda l: l.name)
@pytest.mark.parametrize("exact", [False, True], ids=["random", "integer"])
def test_full_size_layers_sampled(layer, exact):
    _flush(f"{layer.name} exact={exact}")
    inp = wl.make_inputs(layer, integer_exact=exact)
    gpu = run_gpu(inp)
    res = oracle_sampled(inp, gpu, seed=layer.index, count=1500)
    errs = check(res, "f32", exact=exact, label=layer.name)
    print(layer.name, errs)


def test_deterministic_bitwise():
    import torch
    import diffusion_unet_x3_amd as lib3
    layer = wl.CONFIGS[2][0]
    inp = wl.make_inputs(layer)
    a = run_gpu(inp)
    b = run_gpu(inp)
    for k in ("y", "dx", "dw", "db"):
        assert np.array_equal(a[k], b[k]), k
