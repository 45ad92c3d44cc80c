"""GPU parity of the upsample-then-convolve entry points (conv3x3_*_up2:
nearest 2x upsampling fused into the convolution) against the oracle,
through the C ABI.  Same float32 bar as the plain passes (2e-5; exact on
integer inputs, where the summed taps of the parity-class forward and the
4x4-gather backward-data are exact too), on small and ragged shapes in full
(widths that give the vector and the scalar staging paths, one and several
tiles across -- the backward-data tile's right halo column --, odd heights,
ragged channel fills and tiles, several images per block) and on a
full-size up-path layer by sampled elements.  bfloat16 inputs run the
stride-1 passes over the upsampled grid, the upsampled x read at half
coordinates as it is staged (four source elements spread over eight pixels
by the vector paths, single elements by the scalar ones) and
backward-data's upsampled-grid gradient summed over 2 x 2 blocks afterwards
(through the workspace the binding sizes with conv3x3_up2_workspace_size);
the bar is then the bf16 trip-wire (1e-4), and integer inputs are exact."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import TRIPWIRE, rel_err

pytestmark = pytest.mark.gpu


def _run(inp):
    """All three passes through the C ABI (the binding supplies the
    workspaces)."""
    import diffusion_unet_x3_amd as lib3
    dev = torch.device("cuda", 0)
    x, w, g, b = (inp[k].to(dev) for k in ("x", "w", "g", "b"))
    N, C, H, W = x.shape
    K = w.shape[0]
    nan = float("nan")
    y = torch.full((N, K, 2 * H, 2 * W), nan, device=dev)
    dx = torch.full((N, C, H, W), nan, device=dev)
    dw = torch.full((K, C, 3, 3), nan, device=dev)
    db = torch.full((K,), nan, device=dev)
    lib3.conv3x3_fwd_up2(x, w, b, out=y)
    lib3.conv3x3_bwd_data_up2(g, w, out=dx)
    lib3.conv3x3_bwd_weight_up2(x, g, dw=dw, db=db)
    torch.cuda.synchronize()
    return {k: v.cpu().double().numpy() for k, v in dict(y=y, dx=dx, dw=dw, db=db).items()}


def _inputs(N, C, K, H, W, seed, integer=False, dtype="f32"):
    """x at H x W, g at 2H x 2W (the layer record is drawn at the upsampled
    size; x is its top-left quarter, so every draw stays seeded)."""
    layer = wl.small_layer(N, C, K, 2 * H, 2 * W, dtype=dtype, seed=seed)
    inp = wl.make_inputs(layer, integer_exact=integer)
    inp["x"] = inp["x"][:, :, :H, :W].contiguous()
    return inp


# (N, C, K, H, W) of the small input
SHAPES = [(2, 64, 64, 16, 16), (2, 8, 16, 4, 6), (1, 3, 5, 7, 9), (2, 17, 33, 5, 13),
          (2, 32, 48, 8, 40), (1, 16, 24, 3, 68), (4, 128, 64, 8, 8),
          (3, 40, 136, 9, 20), (2, 136, 72, 4, 4), (1, 8, 8, 1, 1)]


@pytest.mark.parametrize("integer", [False, True], ids=["random", "integer"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_up2_full_compare(shape, dtype, integer):
    print(f"[parity] up2 {dtype} {shape} integer={integer}", flush=True)
    inp = _inputs(*shape, seed=83, integer=integer, dtype=dtype)
    gpu = _run(inp)
    ref = {"y": oracle.conv3x3_fwd_up2(inp["x"], inp["w"], inp["b"]),
           "dx": oracle.conv3x3_bwd_data_up2(inp["g"], inp["w"])}
    ref["dw"], ref["db"] = oracle.conv3x3_bwd_weight_up2(inp["x"], inp["g"])
    for k, r in ref.items():
        assert gpu[k].shape == r.shape, k
        if integer:
            assert np.array_equal(gpu[k], r), (shape, k)
        else:
            e = rel_err(gpu[k], r)
            assert e <= TRIPWIRE[dtype], (shape, k, e)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_full_size_up_layer_sampled(dtype):
    """The 32x32 -> 64x64 up step of the UNet (N = 32, 128 channels)."""
    N, C, K, H, W = 32, 128, 128, 32, 32
    print(f"[parity] up2 full-size {dtype}", flush=True)
    inp = _inputs(N, C, K, H, W, seed=89, dtype=dtype)
    gpu = _run(inp)
    x, w, b, g = inp["x"], inp["w"], inp["b"], inp["g"]
    u = oracle.upsample2(x)
    rng = np.random.default_rng(5)
    i = np.unique(rng.integers(0, N * K * 4 * H * W, 2000))
    errs = {"y": rel_err(gpu["y"].ravel()[i], oracle.conv3x3_fwd_at(u, w, b, i))}
    # dx: each sampled element is the sum of four backward-data elements
    j = np.unique(rng.integers(0, N * C * H * W, 1000))
    n, c, r = j // (C * H * W), (j // (H * W)) % C, j % (H * W)
    hh, ww = r // W, r % W
    big = []
    for a in (0, 1):
        for bb in (0, 1):
            big.append(((n * C + c) * 2 * H + 2 * hh + a) * 2 * W + 2 * ww + bb)
    parts = oracle.conv3x3_bwd_data_at(g, w, np.concatenate(big)).reshape(4, -1)
    errs["dx"] = rel_err(gpu["dx"].ravel()[j], parts.sum(axis=0))
    k = np.unique(rng.integers(0, K * C * 9, 400))
    errs["dw"] = rel_err(gpu["dw"].ravel()[k], oracle.conv3x3_bwd_weight_at(u, g, k))
    print(errs)
    for name, e in errs.items():
        assert e <= TRIPWIRE[dtype], (name, e)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_up2_deterministic_bitwise(dtype):
    """No atomics in any upsampling pass: two runs agree bit for bit."""
    inp = _inputs(4, 128, 64, 8, 8, seed=107, dtype=dtype)
    a, b = _run(inp), _run(inp)
    for k in ("y", "dx", "dw", "db"):
        assert np.array_equal(a[k], b[k]), k
