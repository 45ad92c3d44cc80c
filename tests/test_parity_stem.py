"""GPU parity of the few-channel inputs (an RGB image stem, a 4-channel
latent) against the oracle, through the C ABI.  With 3 or 4 input channels
the float32 forward packs the (channel, tap) pairs of the reduction two per
MFMA step; with one to four, the bfloat16 forward runs the persistent
packed-pair kernel (the pairs as the MFMA's reduction, 64-channel tiles,
workgroups looping over 128-pixel tiles -- four tiles each on the full-size
stem) and backward-weight (both dtypes) the packed-pair kernel whose MFMA
columns are the 9C (channel, tap) pairs; these cases cover them (whole and
ragged output tiles and pixel chunks, widths that are and are not a
multiple of 4 or 8, one to four channels, channel tiles with ragged ends,
integer-exact inputs) together with the backward-data pass."""
import pytest

import workloads as wl
from parity_util import check, oracle_full, oracle_sampled, pairs, run_gpu

pytestmark = pytest.mark.gpu

SHAPES = [(2, 3, 64, 32, 32), (2, 4, 128, 16, 16), (3, 3, 5, 7, 12), (2, 3, 17, 9, 8),
          (2, 4, 130, 10, 72), (1, 3, 64, 13, 10), (4, 3, 128, 8, 8), (2, 3, 256, 16, 16),
          (2, 1, 40, 10, 12), (2, 2, 33, 16, 16), (3, 4, 64, 31, 33), (1, 3, 128, 64, 64)]


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
