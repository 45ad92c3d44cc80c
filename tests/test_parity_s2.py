"""GPU parity of the stride-2 entry points (conv3x3_*_s2, a UNet's
downsample block) against the oracle, through the C ABI.  Same float32 bar
as the plain passes (2e-5; exact on integer inputs), on small and ragged
shapes in full and on the three UNet downsample layers by sampled elements.
The shapes reach the vector staging (W % 8 == 0, 16-byte aligned) and the
scalar one, output grids wider than one tile (the left halo column of the
stride-2 x tile is loaded), ragged channel fills and tiles, several images
per block, and g grids with odd sizes (every output-pixel parity class of
backward-data gets a ragged edge).  bfloat16 inputs run the stride-1
passes over the full-resolution grid (the forward keeping the even pixels;
backward-data and backward-weight reading g zero-inserted), through the
vector staging paths where the full grid's width is a multiple of 8 and the
channels fill whole 16-channel steps, the scalar ones elsewhere, to the
bf16 trip-wire (1e-4; exact on integer inputs)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import TRIPWIRE, rel_err

pytestmark = pytest.mark.gpu


def _inputs(N, C, K, H, W, seed, integer=False, dtype="f32"):
    """x at H x W, g at H/2 x W/2 (a corner of the full-size draw)."""
    layer = wl.small_layer(N, C, K, H, W, dtype=dtype, seed=seed)
    inp = wl.make_inputs(layer, integer_exact=integer)
    inp["g"] = inp["g"][:, :, :H // 2, :W // 2].contiguous()
    return inp


def _run(inp):
    import diffusion_unet_x3_amd as lib3
    dev = torch.device("cuda", 0)
    x, w, g, b = (inp[k].to(dev) for k in ("x", "w", "g", "b"))
    N, C, H, W = x.shape
    K = w.shape[0]
    nan = float("nan")
    y = torch.full((N, K, H // 2, W // 2), nan, device=dev)
    dx = torch.full((N, C, H, W), nan, device=dev)
    dw = torch.full((K, C, 3, 3), nan, device=dev)
    db = torch.full((K,), nan, device=dev)
    lib3.conv3x3_fwd_s2(x, w, b, out=y)
    lib3.conv3x3_bwd_data_s2(g, w, out=dx)
    lib3.conv3x3_bwd_weight_s2(x, g, dw=dw, db=db)
    torch.cuda.synchronize()
    return {k: v.cpu().double().numpy() for k, v in dict(y=y, dx=dx, dw=dw, db=db).items()}


# (N, C, K, H, W) of the input; H, W even
SHAPES = [(2, 64, 64, 32, 32), (2, 8, 16, 8, 12), (1, 3, 5, 6, 10), (2, 17, 33, 10, 14),
          (2, 32, 48, 16, 80), (1, 16, 24, 4, 136), (4, 128, 64, 16, 16),
          (3, 24, 40, 18, 40), (2, 72, 136, 8, 8), (1, 8, 8, 2, 2)]


@pytest.mark.parametrize("integer", [False, True], ids=["random", "integer"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_s2_full_compare(shape, dtype, integer):
    print(f"[parity] s2 {dtype} {shape} integer={integer}", flush=True)
    inp = _inputs(*shape, seed=97, integer=integer, dtype=dtype)
    gpu = _run(inp)
    ref = {"y": oracle.conv3x3_fwd_s2(inp["x"], inp["w"], inp["b"]),
           "dx": oracle.conv3x3_bwd_data_s2(inp["g"], inp["w"])}
    ref["dw"], ref["db"] = oracle.conv3x3_bwd_weight_s2(inp["x"], inp["g"])
    for k, r in ref.items():
        assert gpu[k].shape == r.shape, k
        if integer:
            assert np.array_equal(gpu[k], r), (shape, k)
        else:
            e = rel_err(gpu[k], r)
            assert e <= TRIPWIRE[dtype], (shape, k, e)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("layer", wl.DOWNSAMPLE, ids=lambda l: l.name)
def test_downsample_layers_sampled(layer, dtype):
    N, C, K, H, W = layer.shape
    print(f"[parity] s2 {layer.name} {dtype}", flush=True)
    inp = _inputs(N, C, K, H, W, seed=101, dtype=dtype)
    gpu = _run(inp)
    x, w, b, g = inp["x"], inp["w"], inp["b"], inp["g"]
    gz = oracle.zero_insert2(g)
    rng = np.random.default_rng(layer.index)
    errs = {}
    i = np.unique(rng.integers(0, N * K * (H // 2) * (W // 2), 1500))
    n, k, r = i // (K * (H // 2) * (W // 2)), (i // ((H // 2) * (W // 2))) % K, \
        i % ((H // 2) * (W // 2))
    full = ((n * K + k) * H + 2 * (r // (W // 2))) * W + 2 * (r % (W // 2))
    errs["y"] = rel_err(gpu["y"].ravel()[i], oracle.conv3x3_fwd_at(x, w, b, full))
    j = np.unique(rng.integers(0, N * C * H * W, 1500))
    errs["dx"] = rel_err(gpu["dx"].ravel()[j], oracle.conv3x3_bwd_data_at(gz, w, j))
    j = np.unique(rng.integers(0, K * C * 9, 400))
    errs["dw"] = rel_err(gpu["dw"].ravel()[j], oracle.conv3x3_bwd_weight_at(x, gz, j))
    print(layer.name, errs)
    for name, e in errs.items():
        assert e <= TRIPWIRE[dtype], (layer.name, name, e)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_s2_deterministic_bitwise(dtype):
    """No atomics in any stride-2 pass: two runs agree bit for bit (the
    128-channel downsample layer, split-K backward-weight included)."""
    layer = wl.DOWNSAMPLE[0]
    inp = _inputs(*layer.shape, seed=103, dtype=dtype)
    a, b = _run(inp), _run(inp)
    for k in ("y", "dx", "dw", "db"):
        assert np.array_equal(a[k], b[k]), k
