"""GPU parity of the concatenated-input entry points (conv3x3_*_cat) against
the oracle, through the C ABI.

The input is the channel concatenation [x0 ; x1] (a UNet's up-path skip
input) held as two tensors; the oracle computes the convolution of the
concatenated tensor.  Same bars as the plain passes: max|err| / max|ref| <=
2e-5 (float32) and the 1e-4 trip-wire (bfloat16), exact equality on
integer-valued inputs.  Cases cover halves that are whole LDS fills and
channel tiles (vector paths), ragged halves (a partly filled fill or tile at
the end of the first half), empty halves, the eight-wave bfloat16 tiles, and
full-size UNet up-path layers on sampled outputs.  Where every fill and tile
boundary of the concatenation coincides with one of the plain problem, the
summation order is the plain kernel's, so the results must also equal the
plain entry points' on the concatenated tensor bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import TRIPWIRE, rel_err

pytestmark = pytest.mark.gpu


def _split_inputs(layer, C0, exact=False):
    inp = wl.make_inputs(layer, integer_exact=exact)
    x = inp["x"]
    inp["x0"] = x[:, :C0].contiguous()
    inp["x1"] = x[:, C0:].contiguous()
    return inp


def _run_cat(inp, C0):
    import diffusion_unet_x3_amd as lib3
    dev = torch.device("cuda", 0)
    x0, x1, w, g = (inp[k].to(dev) for k in ("x0", "x1", "w", "g"))
    b = inp["b"].to(dev)
    N, _, H, W = g.shape
    K = w.shape[0]
    C = w.shape[1]
    nan = float("nan")
    y = torch.full((N, K, H, W), nan, device=dev)
    dx0 = torch.full((N, C0, H, W), nan, device=dev)
    dx1 = torch.full((N, C - C0, H, W), nan, device=dev)
    dw = torch.full((K, C, 3, 3), nan, device=dev)
    db = torch.full((K,), nan, device=dev)
    lib3.conv3x3_fwd_cat(x0, x1, w, b, out=y)
    lib3.conv3x3_bwd_data_cat(g, w, C0, out0=dx0, out1=dx1)
    lib3.conv3x3_bwd_weight_cat(x0, x1, g, dw=dw, db=db)
    torch.cuda.synchronize()
    return {k: v.cpu().double().numpy() for k, v in
            dict(y=y, dx0=dx0, dx1=dx1, dw=dw, db=db).items()}


def _run_plain(inp):
    import diffusion_unet_x3_amd as lib3
    dev = torch.device("cuda", 0)
    x, w, g, b = (inp[k].to(dev) for k in ("x", "w", "g", "b"))
    # (the *_cat entry points take no workspace, so they run the unsplit
    # plan: compare with that)
    y = lib3.conv3x3_fwd(x, w, b, split=False)
    dx = lib3.conv3x3_bwd_data(g, w, split=False)
    dw, db = lib3.conv3x3_bwd_weight(x, g)
    torch.cuda.synchronize()
    return y.cpu(), dx.cpu(), dw.cpu(), db.cpu()


def _oracle(inp, C0):
    y = oracle.conv3x3_fwd_cat(inp["x0"], inp["x1"], inp["w"], inp["b"])
    dx0, dx1 = oracle.conv3x3_bwd_data_cat(inp["g"], inp["w"], C0)
    dw, db = oracle.conv3x3_bwd_weight_cat(inp["x0"], inp["x1"], inp["g"])
    return dict(y=y, dx0=dx0, dx1=dx1, dw=dw, db=db)


def _compare(gpu, ref, dtype, exact, label):
    errs = {}
    for k, r in ref.items():
        got = gpu[k]
        assert got.shape == r.shape, (label, k)
        assert np.all(np.isfinite(got)), (label, k, "unwritten element")
        if exact:
            bad = np.flatnonzero(got != r)
            assert bad.size == 0, (label, k, "integer-exact mismatch", bad[:10])
            errs[k] = 0.0
        else:
            errs[k] = rel_err(got, r)
            assert errs[k] <= TRIPWIRE[dtype], (label, k, errs[k])
    return errs


# (N, C0, C1, K, H, W)
F32 = [(2, 8, 8, 16, 8, 8), (2, 64, 64, 64, 16, 16), (2, 5, 13, 7, 9, 11),
       (2, 12, 20, 24, 8, 16), (2, 100, 28, 130, 8, 8), (2, 96, 160, 136, 16, 16),
       (1, 0, 16, 8, 8, 8), (1, 16, 0, 8, 8, 8), (1, 3, 1, 5, 6, 7), (2, 24, 40, 9, 8, 80)]
BF16 = [(2, 16, 16, 32, 8, 8), (2, 32, 48, 64, 16, 16), (2, 8, 24, 16, 8, 8),
        (2, 5, 11, 9, 8, 8), (1, 0, 32, 16, 8, 8), (1, 32, 0, 16, 8, 8),
        (2, 72, 56, 136, 8, 16),
        # eight-wave tiles: forward with 16 + 16 input channels, backward-data
        # with 128 + 128 and 72 + 128 output channels
        (32, 16, 16, 256, 32, 32), (32, 128, 128, 16, 32, 32), (32, 72, 128, 16, 32, 32)]


def _id(s):
    return "x".join(map(str, s))


@pytest.mark.parametrize("exact", [False, True], ids=["random", "integer"])
@pytest.mark.parametrize("shape", F32, ids=_id)
def test_f32_concat_full_compare(shape, exact):
    N, C0, C1, K, H, W = shape
    layer = wl.small_layer(N, C0 + C1, K, H, W, dtype="f32", seed=31)
    print(f"[parity] cat f32 {shape} exact={exact}", flush=True)
    inp = _split_inputs(layer, C0, exact)
    errs = _compare(_run_cat(inp, C0), _oracle(inp, C0), "f32", exact, shape)
    print(errs)


@pytest.mark.parametrize("exact", [False, True], ids=["random", "integer"])
@pytest.mark.parametrize("shape", BF16, ids=_id)
def test_bf16_concat_full_compare(shape, exact):
    N, C0, C1, K, H, W = shape
    layer = wl.small_layer(N, C0 + C1, K, H, W, dtype="bf16", seed=37)
    print(f"[parity] cat bf16 {shape} exact={exact}", flush=True)
    inp = _split_inputs(layer, C0, exact)
    errs = _compare(_run_cat(inp, C0), _oracle(inp, C0), "bf16", exact, shape)
    print(errs)


# Halves whose boundary falls on a fill and tile boundary of the plain plan
# (float32 fills 8 channels, tiles 64 / 128; bfloat16 fills 16).
ALIGNED = [("f32", (2, 64, 64, 64, 16, 16)), ("f32", (2, 128, 128, 128, 8, 8)),
           ("bf16", (2, 32, 48, 64, 16, 16)), ("bf16", (32, 128, 128, 16, 32, 32))]


@pytest.mark.parametrize("case", ALIGNED, ids=lambda c: c[0] + "-" + _id(c[1]))
def test_aligned_halves_match_plain_bitwise(case):
    dtype, (N, C0, C1, K, H, W) = case
    import diffusion_unet_x3_amd as lib3
    code = lib3.CONV3X3_F32 if dtype == "f32" else lib3.CONV3X3_BF16
    for p in (0, 1, 2):
        assert lib3.conv3x3_plan_cat(p, N, C0, C1, K, H, W, code) == \
            lib3.conv3x3_plan(p, N, C0 + C1, K, H, W, code)
    layer = wl.small_layer(N, C0 + C1, K, H, W, dtype=dtype, seed=41)
    inp = _split_inputs(layer, C0)
    cat = _run_cat(inp, C0)
    y, dx, dw, db = _run_plain(inp)
    assert np.array_equal(cat["y"], y.double().numpy())
    assert np.array_equal(cat["dx0"], dx[:, :C0].double().numpy())
    assert np.array_equal(cat["dx1"], dx[:, C0:].double().numpy())
    assert np.array_equal(cat["dw"], dw.double().numpy())
    assert np.array_equal(cat["db"], db.double().numpy())


def _up_layer(name):
    for layers in wl.CONFIGS.values():
        for l in layers:
            if l.name == name:
                return l
    raise KeyError(name)


# Up-path layers whose input is [upsampled features ; skip]: (layer, C0).
FULL = [("up0_28_384to128_64x64_f32", 256), ("up1_24_640to256_32x32_f32", 384),
        ("up2_20_896to384_16x16_bf16", 512), ("up3_18_1024to512_8x8_bf16", 512)]


@pytest.mark.parametrize("case", FULL, ids=lambda c: c[0])
def test_full_size_up_layers_sampled(case):
    name, C0 = case
    layer = _up_layer(name)
    print(f"[parity] cat {name} C0={C0}", flush=True)
    inp = _split_inputs(layer, C0)
    gpu = _run_cat(inp, C0)
    rng = np.random.default_rng(layer.index)
    x0, x1, w, b, g = (inp[k] for k in ("x0", "x1", "w", "b", "g"))
    N, C, H, W = inp["x"].shape
    K = w.shape[0]
    errs = {}
    i = np.unique(rng.integers(0, N * K * H * W, 2000))
    errs["y"] = rel_err(gpu["y"].ravel()[i], oracle.conv3x3_fwd_cat_at(x0, x1, w, b, i))
    # dx halves: sampled elements of the plain backward-data, split at C0
    dx = np.concatenate([gpu["dx0"], gpu["dx1"]], axis=1)
    j = np.unique(rng.integers(0, N * C * H * W, 2000))
    errs["dx"] = rel_err(dx.ravel()[j], oracle.conv3x3_bwd_data_at(g, w, j))
    j = np.unique(rng.integers(0, K * C * 9, 600))
    errs["dw"] = rel_err(gpu["dw"].ravel()[j], oracle.conv3x3_bwd_weight_cat_at(x0, x1, g, j))
    j = np.arange(K)
    errs["db"] = rel_err(gpu["db"][j], oracle.conv3x3_bias_grad_at(g, j))
    print(name, errs)
    for k, e in errs.items():
        assert e <= TRIPWIRE[layer.dtype], (name, k, e)
