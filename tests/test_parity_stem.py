"""GPU parity of the few-channel inputs (an RGB image stem, a 4-channel
latent) against the oracle, through the C ABI.  With 3 or 4 input channels
the float32 forward packs the (channel, tap) pairs of the reduction two per
MFMA step; with one to four, the bfloat16 forward runs the persistent
packed-pair kernel (the pairs as the MFMA's reduction, 64-channel tiles,
workgroups looping over 128-pixel tiles -- four tiles each on the full-size
stem) and backward-weight (both dtypes) the packed-pair kernel whose MFMA
columns are the 9C (channel, tap) pairs; with one to three channels and at
most 128 g channels, backward-data makes the 9C pairs the rows of
P = w^T g over bands of image rows and sums each output pixel's nine
shifted taps.  These cases cover them (whole and ragged output tiles,
pixel chunks and bands, widths that are and are not a multiple of 4 or 8,
one to four channels, channel tiles with ragged ends, integer-exact
inputs)."""
import pytest

import workloads as wl
from parity_util import check, oracle_full, oracle_sampled, pairs, run_gpu

pytestmark = pytest.mark.gpu

SHAPES = [(2, 3, 64, 32, 32), (2, 4, 128, 16, 16), (3, 3, 5, 7, 12), (2, 3, 17, 9, 8),
          (2, 4, 130, 10, 72), (1, 3, 64, 13, 10), (4, 3, 128, 8, 8), (2, 3, 256, 16, 16),
          (2, 1, 40, 10, 12), (2, 2, 33, 16, 16), (3, 4, 64, 31, 33), (1, 3, 128, 64, 64),
          # backward-data's (channel, tap)-row kernel: rows of 100 pixels
          # (bands of 4 rows, an odd K on the 64-step sweep), 200 (bands of
          # one row), one pixel wide with K = 1, and the widest row it takes
          (2, 3, 65, 11, 100), (1, 2, 128, 5, 200), (3, 1, 1, 9, 1), (2, 3, 7, 20, 213)]


@pytest.mark.parametrize("exact", [False, True], ids=["random", "integer"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_few_channel_full_compare(shape, dtype, exact):
    layer = wl.small_layer(*shape, dtype=dtype, seed=67)
    print(f"[parity] stem {dtype} {shape} exact={exact}", flush=True)
    inp = wl.make_inputs(layer, integer_exact=exact)
    errs = check(pairs(run_gpu(inp), oracle_full(inp)), dtype, exact=exact, label=str(shape))
    print(errs)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_image_stem_full_size_sampled(dtype):
    layer = wl.IMAGE_STEM[dtype]
    print(f"[parity] {layer.name}", flush=True)
    inp = wl.make_inputs(layer)
    gpu = run_gpu(inp)
    errs = check(oracle_sampled(inp, gpu, seed=5), dtype, label=layer.name)
    print(layer.name, errs)


def test_stem_bwd_data_bf16_outputs_integer_exact():
    """CONV3X3_BF16_IO through the (channel, tap)-row backward-data: with
    integer inputs every sum is exact in float32, so dx rounded to bfloat16
    equals the oracle's exact result rounded to bfloat16."""
    import numpy as np
    import torch

    import diffusion_unet_x3_amd as lib3
    import oracle
    shape = (2, 3, 64, 11, 40)
    plan = lib3.conv3x3_plan(lib3.PASS_BWD_DATA, *shape, lib3.CONV3X3_BF16)
    assert plan["tile_m"] == 3 and plan["threads"] == 512, plan  # the few-channel plan
    inp = wl.make_inputs(wl.small_layer(*shape, dtype="bf16", seed=61), integer_exact=True)
    dev = torch.device("cuda", 0)
    g, w = inp["g"].to(dev), inp["w"].to(dev)
    dx = lib3.conv3x3_bwd_data(g, w, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.round_to_bf16(oracle.conv3x3_bwd_data(inp["g"], inp["w"]))
    assert np.array_equal(dx.float().cpu().double().numpy(), ref)
