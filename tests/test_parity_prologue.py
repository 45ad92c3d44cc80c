"""GPU parity of the input-prologue entry points (conv3x3_*_gnsilu) against
the oracle, through the C ABI.

The convolution's input is SiLU(x * scale[n, c] + shift[n, c]), formed in
the loader; backward-data returns du = bwd_data(g, w) * SiLU'(u).  Same bar
as the plain passes (max|err| / max|ref| <= 2e-5 for float32, the 1e-4
trip-wire for bfloat16, whose staged a is rounded to bfloat16 -- the oracle
rounds the exact a once), on small and ragged shapes in full (vector and
scalar staging, halo columns loaded or not, ragged channel tiles) and on
full-size layers by sampled elements."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import TRIPWIRE, rel_err

pytestmark = pytest.mark.gpu


def _run(inp, scale, shift):
    import diffusion_unet_x3_amd as lib3
    dev = torch.device("cuda", 0)
    x, w, g, b = (inp[k].to(dev) for k in ("x", "w", "g", "b"))
    s, t = scale.to(dev), shift.to(dev)
    N, C, H, W = x.shape
    K = w.shape[0]
    nan = float("nan")
    y = torch.full((N, K, H, W), nan, device=dev)
    du = torch.full((N, C, H, W), nan, device=dev)
    dw = torch.full((K, C, 3, 3), nan, device=dev)
    db = torch.full((K,), nan, device=dev)
    lib3.conv3x3_fwd_gnsilu(x, s, t, w, b, out=y)
    lib3.conv3x3_bwd_data_gnsilu(g, w, x, s, t, out=du)
    lib3.conv3x3_bwd_weight_gnsilu(x, s, t, g, dw=dw, db=db)
    torch.cuda.synchronize()
    return {k: v.cpu().double().numpy() for k, v in dict(y=y, du=du, dw=dw, db=db).items()}


SMALL = [(2, 64, 64, 32, 32), (1, 3, 5, 7, 9), (2, 17, 33, 5, 13), (3, 64, 64, 31, 33),
         (2, 24, 40, 9, 80), (5, 16, 16, 8, 8), (2, 40, 130, 10, 72), (1, 513, 7, 8, 8),
         (2, 128, 128, 16, 16), (1, 32, 256, 8, 8)]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_prologue_full_compare(shape):
    layer = wl.small_layer(*shape, dtype="f32", seed=43)
    print(f"[parity] gnsilu f32 {shape}", flush=True)
    inp = wl.make_inputs(layer)
    s, t = wl.make_prologue(layer)
    gpu = _run(inp, s, t)
    x, w, b, g = inp["x"], inp["w"], inp["b"], inp["g"]
    ref = {"y": oracle.conv3x3_fwd_gnsilu(x, s, t, w, b),
           "du": oracle.conv3x3_bwd_data_gnsilu(g, w, x, s, t)}
    ref["dw"], ref["db"] = oracle.conv3x3_bwd_weight_gnsilu(x, s, t, g)
    errs = {k: rel_err(gpu[k], ref[k]) for k in ref}
    print(errs)
    for k, e in errs.items():
        assert e <= TRIPWIRE["f32"], (shape, k, e)


FULL = [wl.CONFIGS[2][0], wl.CONFIGS[3][1]]


@pytest.mark.parametrize("layer", FULL, ids=lambda l: l.name)
def test_full_size_prologue_sampled(layer):
    print(f"[parity] gnsilu {layer.name}", flush=True)
    inp = wl.make_inputs(layer)
    s, t = wl.make_prologue(layer)
    gpu = _run(inp, s, t)
    x, w, b, g = inp["x"], inp["w"], inp["b"], inp["g"]
    N, C, H, W = x.shape
    K = w.shape[0]
    a = oracle.prologue_apply(x, s, t)
    u = x.double().numpy() * s.double().numpy()[:, :, None, None] + \
        t.double().numpy()[:, :, None, None]
    rng = np.random.default_rng(layer.index + 7)
    errs = {}
    i = np.unique(rng.integers(0, N * K * H * W, 2000))
    errs["y"] = rel_err(gpu["y"].ravel()[i], oracle.conv3x3_fwd_at(a, w, b, i))
    j = np.unique(rng.integers(0, N * C * H * W, 2000))
    du_ref = oracle.act_grad(oracle.conv3x3_bwd_data_at(g, w, j), u.ravel()[j], oracle.ACT_SILU)
    errs["du"] = rel_err(gpu["du"].ravel()[j], du_ref)
    j = np.unique(rng.integers(0, K * C * 9, 600))
    errs["dw"] = rel_err(gpu["dw"].ravel()[j], oracle.conv3x3_bwd_weight_at(a, g, j))
    j = np.arange(K)
    errs["db"] = rel_err(gpu["db"][j], oracle.conv3x3_bias_grad_at(g, j))
    print(layer.name, errs)
    for k, e in errs.items():
        assert e <= TRIPWIRE["f32"], (layer.name, k, e)


def test_plain_entry_points_unchanged_by_the_prologue_build():
    """The plain passes are separate instantiations: the same inputs give
    bitwise the same results whether or not a prologue call ran before."""
    import diffusion_unet_x3_amd as lib3
    layer = wl.small_layer(2, 64, 64, 16, 16, dtype="f32", seed=47)
    inp = wl.make_inputs(layer)
    dev = torch.device("cuda", 0)
    x, w, g, b = (inp[k].to(dev) for k in ("x", "w", "g", "b"))
    y0 = lib3.conv3x3_fwd(x, w, b)
    s, t = (v.to(dev) for v in wl.make_prologue(layer))
    lib3.conv3x3_fwd_gnsilu(x, s, t, w, b)
    y1 = lib3.conv3x3_fwd(x, w, b)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


SMALL_BF16 = [(2, 64, 64, 32, 32), (2, 17, 33, 5, 13), (2, 32, 48, 9, 80), (5, 16, 16, 8, 8),
              (2, 128, 128, 16, 16), (1, 32, 256, 8, 8), (3, 64, 64, 31, 33)]


def _bf16_inputs(shape, seed):
    layer = wl.small_layer(*shape, dtype="bf16", seed=seed)
    inp = wl.make_inputs(layer)
    s, t = wl.make_prologue(layer)
    return inp, s, t


@pytest.mark.parametrize("shape", SMALL_BF16, ids=lambda s: "x".join(map(str, s)))
def test_bf16_prologue_full_compare(shape):
    """bfloat16: the loaders stage a = SiLU(x * scale + shift) rounded to
    bfloat16 as the exact value rounds; y, dw and db against the oracle on
    that rounded a, du (float32) against the exact du, all under the 1e-4
    trip-wire (vector staging with and without halo columns, and the
    scalar path for ragged shapes)."""
    print(f"[parity] gnsilu bf16 {shape}", flush=True)
    inp, s, t = _bf16_inputs(shape, 53)
    gpu = _run(inp, s, t)
    x, w, b, g = inp["x"], inp["w"], inp["b"], inp["g"]
    ref = {"y": oracle.conv3x3_fwd_gnsilu(x, s, t, w, b, bf16=True),
           "du": oracle.conv3x3_bwd_data_gnsilu(g, w, x, s, t)}
    ref["dw"], ref["db"] = oracle.conv3x3_bwd_weight_gnsilu(x, s, t, g, bf16=True)
    errs = {k: rel_err(gpu[k], ref[k]) for k in ref}
    print(errs)
    for k, e in errs.items():
        assert e <= TRIPWIRE["bf16"], (shape, k, e)


FULL_BF16 = [wl.CONFIGS[4][0], wl.CONFIGS[4][1], wl.CONFIGS[5][32]]


@pytest.mark.parametrize("layer", FULL_BF16, ids=lambda l: l.name)
def test_bf16_full_size_prologue_sampled(layer):
    print(f"[parity] gnsilu {layer.name}", flush=True)
    inp = wl.make_inputs(layer)
    s, t = wl.make_prologue(layer)
    gpu = _run(inp, s, t)
    x, w, b, g = inp["x"], inp["w"], inp["b"], inp["g"]
    N, C, H, W = x.shape
    K = w.shape[0]
    a = oracle.prologue_apply(x, s, t, bf16=True)
    u = x.double().numpy() * s.double().numpy()[:, :, None, None] + \
        t.double().numpy()[:, :, None, None]
    rng = np.random.default_rng(layer.index + 11)
    errs = {}
    i = np.unique(rng.integers(0, N * K * H * W, 2000))
    errs["y"] = rel_err(gpu["y"].ravel()[i], oracle.conv3x3_fwd_at(a, w, b, i))
    j = np.unique(rng.integers(0, N * C * H * W, 2000))
    du_ref = oracle.act_grad(oracle.conv3x3_bwd_data_at(g, w, j), u.ravel()[j], oracle.ACT_SILU)
    errs["du"] = rel_err(gpu["du"].ravel()[j], du_ref)
    j = np.unique(rng.integers(0, K * C * 9, 400))
    errs["dw"] = rel_err(gpu["dw"].ravel()[j], oracle.conv3x3_bwd_weight_at(a, g, j))
    j = np.arange(K)
    errs["db"] = rel_err(gpu["db"][j], oracle.conv3x3_bias_grad_at(g, j))
    print(layer.name, errs)
    for k, e in errs.items():
        assert e <= TRIPWIRE["bf16"], (layer.name, k, e)
