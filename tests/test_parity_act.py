"""GPU parity of the fused-activation entry points against the oracle,
through the C ABI.

Forward: y = act(z) and z = conv(x; w) + b against the oracle's; backward
(both dtypes): dx, dw, db from gy and z against the oracle's backward on
g = gy * act'(z) (for bfloat16 that exact product rounded once to
bfloat16), fed the z the GPU produced (the backward is a function of
the z it is given; on the leaky ReLU's kink an independently rounded z could
pick the other slope).  Same bar as the plain passes (max|err| / max|ref|
<= 2e-5 for float32, the 1e-4 trip-wire for bfloat16), on small and ragged
shapes in full and on full-size layers by sampled elements."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import TRIPWIRE, rel_err

pytestmark = pytest.mark.gpu

ACTS = {"silu": oracle.ACT_SILU, "lrelu": oracle.ACT_LRELU, "none": oracle.ACT_NONE}


def _run(inp, act, backward=True):
    import diffusion_unet_x3_amd as lib3
    dev = torch.device("cuda", 0)
    x, w, gy = (inp[k].to(dev) for k in ("x", "w", "g"))
    b = inp["b"].to(dev)
    N, C, H, W = x.shape
    K = w.shape[0]
    nan = float("nan")
    y = torch.full((N, K, H, W), nan, device=dev)
    z = torch.full((N, K, H, W), nan, device=dev)
    lib3.conv3x3_fwd_act(x, w, b, act=act, out=y, z=z)
    out = {"y": y, "z": z}
    if backward:
        dx = torch.full((N, C, H, W), nan, device=dev)
        dw = torch.full((K, C, 3, 3), nan, device=dev)
        db = torch.full((K,), nan, device=dev)
        lib3.conv3x3_bwd_data_act(gy, z, w, act=act, out=dx)
        lib3.conv3x3_bwd_weight_act(x, gy, z, act=act, dw=dw, db=db)
        out.update(dx=dx, dw=dw, db=db)
    torch.cuda.synchronize()
    return {k: v.cpu().double().numpy() for k, v in out.items()}


def _check(errs, dtype, label):
    for name, e in errs.items():
        assert e <= TRIPWIRE[dtype], (label, name, e)


SMALL_F32 = [(2, 64, 64, 32, 32), (1, 3, 5, 7, 9), (2, 17, 33, 5, 13), (3, 64, 64, 31, 33),
             (1, 513, 7, 8, 8), (2, 40, 130, 10, 70), (2, 24, 40, 9, 80), (5, 16, 16, 8, 8)]


@pytest.mark.parametrize("act", sorted(ACTS), ids=str)
@pytest.mark.parametrize("shape", SMALL_F32, ids=lambda s: "x".join(map(str, s)))
def test_f32_fused_full_compare(shape, act):
    a = ACTS[act]
    layer = wl.small_layer(*shape, dtype="f32", seed=17)
    print(f"[parity] act={act} f32 {shape}", flush=True)
    inp = wl.make_inputs(layer)
    gpu = _run(inp, a)
    y_ref, z_ref = oracle.conv3x3_fwd_act(inp["x"], inp["w"], inp["b"], a)
    dx_ref, dw_ref, db_ref = oracle.conv3x3_bwd_act(inp["x"], inp["w"], inp["g"], gpu["z"], a)
    errs = {"y": rel_err(gpu["y"], y_ref), "z": rel_err(gpu["z"], z_ref),
            "dx": rel_err(gpu["dx"], dx_ref), "dw": rel_err(gpu["dw"], dw_ref),
            "db": rel_err(gpu["db"], db_ref)}
    print(errs)
    _check(errs, "f32", (shape, act))


def test_act_none_matches_plain_entry_points_bitwise():
    import diffusion_unet_x3_amd as lib3
    layer = wl.small_layer(3, 64, 64, 31, 33, dtype="f32", seed=19)
    inp = wl.make_inputs(layer)
    dev = torch.device("cuda", 0)
    x, w, g, b = (inp[k].to(dev) for k in ("x", "w", "g", "b"))
    y0 = lib3.conv3x3_fwd(x, w, b)
    y1, z1 = lib3.conv3x3_fwd_act(x, w, b, act=lib3.ACT_NONE)
    dx0 = lib3.conv3x3_bwd_data(g, w)
    dx1 = lib3.conv3x3_bwd_data_act(g, None, w, act=lib3.ACT_NONE)
    dw0, db0 = lib3.conv3x3_bwd_weight(x, g)
    dw1, db1 = lib3.conv3x3_bwd_weight_act(x, g, None, act=lib3.ACT_NONE)
    torch.cuda.synchronize()
    for p, q in ((y0, y1), (y0, z1), (dx0, dx1), (dw0, dw1), (db0, db1)):
        assert torch.equal(p, q)


SMALL_BF16 = [(2, 64, 64, 32, 32), (2, 17, 33, 5, 13), (2, 32, 48, 9, 80), (5, 16, 16, 8, 8),
              (32, 16, 256, 32, 32)]


@pytest.mark.parametrize("act", ["silu", "lrelu"])
@pytest.mark.parametrize("shape", SMALL_BF16, ids=lambda s: "x".join(map(str, s)))
def test_bf16_fused_forward_full_compare(shape, act):
    a = ACTS[act]
    layer = wl.small_layer(*shape, dtype="bf16", seed=23)
    print(f"[parity] act={act} bf16 fwd {shape}", flush=True)
    inp = wl.make_inputs(layer)
    gpu = _run(inp, a, backward=False)
    y_ref, z_ref = oracle.conv3x3_fwd_act(inp["x"], inp["w"], inp["b"], a)
    errs = {"y": rel_err(gpu["y"], y_ref), "z": rel_err(gpu["z"], z_ref)}
    print(errs)
    _check(errs, "bf16", (shape, act))


@pytest.mark.parametrize("act", ["silu", "lrelu"])
@pytest.mark.parametrize("shape", SMALL_BF16, ids=lambda s: "x".join(map(str, s)))
def test_bf16_fused_backward_full_compare(shape, act):
    """bfloat16 backward through the activation: the kernels form
    g = RNE_bf16(gy * act'(z)) while staging gy; the oracle rounds the exact
    product once.  The two can land on neighbouring bfloat16 values in rare
    elements (the kernel's product is float32), which the 1e-4 trip-wire
    covers."""
    a = ACTS[act]
    layer = wl.small_layer(*shape, dtype="bf16", seed=29)
    print(f"[parity] act={act} bf16 bwd {shape}", flush=True)
    inp = wl.make_inputs(layer)
    gpu = _run(inp, a)
    dx_ref, dw_ref, db_ref = oracle.conv3x3_bwd_act(inp["x"], inp["w"], inp["g"], gpu["z"], a,
                                                    bf16=True)
    errs = {"dx": rel_err(gpu["dx"], dx_ref), "dw": rel_err(gpu["dw"], dw_ref),
            "db": rel_err(gpu["db"], db_ref)}
    print(errs)
    _check(errs, "bf16", (shape, act))


@pytest.mark.parametrize("shape", [(2, 64, 64, 32, 32), (2, 17, 33, 5, 13), (5, 16, 16, 8, 8),
                                   (4, 32, 128, 16, 16)], ids=lambda s: "x".join(map(str, s)))
def test_bf16_fused_backward_integer_exact(shape):
    """Integer gy and weights with the leaky ReLU: every g = RNE_bf16(gy * 0.2)
    or gy is a multiple of 2^-10 that both sides round identically, and every
    sum is exact in float32, so dx, dw and db equal the oracle's bit for bit
    (an element staged without its slope, or a dropped tap, shows)."""
    import diffusion_unet_x3_amd as lib3
    a = oracle.ACT_LRELU
    layer = wl.small_layer(*shape, dtype="bf16", seed=31)
    inp = wl.make_inputs(layer, integer_exact=True)
    for k in ("x", "w", "g"):
        inp[k] = inp[k].bfloat16()
    dev = torch.device("cuda", 0)
    N, C, H, W = inp["x"].shape
    K = inp["w"].shape[0]
    # z: integers and half-integers around 0, both signs, and exact zeros
    gen = torch.Generator().manual_seed(5)
    z = (torch.randint(-6, 7, (N, K, H, W), generator=gen).float() * 0.5)
    x, w, gy, zd = (t.to(dev) for t in (inp["x"], inp["w"], inp["g"], z))
    dx = lib3.conv3x3_bwd_data_act(gy, zd, w, act=a)
    dw, db = lib3.conv3x3_bwd_weight_act(x, gy, zd, act=a)
    torch.cuda.synchronize()
    dx_ref, dw_ref, db_ref = oracle.conv3x3_bwd_act(inp["x"], inp["w"], inp["g"], z, a,
                                                    bf16=True)
    assert np.array_equal(dx.cpu().double().numpy(), dx_ref)
    assert np.array_equal(dw.cpu().double().numpy(), dw_ref)
    assert np.array_equal(db.cpu().double().numpy(), db_ref)


def test_bf16_fused_backward_act_none_is_plain():
    """act = none with a z given: the slope is 1, so the bf16 fused passes
    equal the plain entry points bit for bit."""
    import diffusion_unet_x3_amd as lib3
    layer = wl.small_layer(2, 64, 64, 16, 16, dtype="bf16", seed=33)
    inp = wl.make_inputs(layer)
    dev = torch.device("cuda", 0)
    x, w, g = (inp[k].to(dev) for k in ("x", "w", "g"))
    z = torch.randn((2, 64, 16, 16), device=dev)
    dx0 = lib3.conv3x3_bwd_data(g, w, split=False)
    dx1 = lib3.conv3x3_bwd_data_act(g, z, w, act=lib3.ACT_NONE)
    dw0, db0 = lib3.conv3x3_bwd_weight(x, g)
    dw1, db1 = lib3.conv3x3_bwd_weight_act(x, g, z, act=lib3.ACT_NONE)
    torch.cuda.synchronize()
    for p, q in ((dx0, dx1), (dw0, dw1), (db0, db1)):
        assert torch.equal(p, q)


FULL = [wl.CONFIGS[2][0], wl.CONFIGS[3][1], wl.CONFIGS[4][0], wl.CONFIGS[4][1]]


@pytest.mark.parametrize("layer", FULL, ids=lambda l: l.name)
def test_full_size_fused_silu_sampled(layer):
    """The stem layer and a mid-resolution layer (float32) and the bf16
    bottlenecks, all passes, SiLU, on sampled outputs."""
    a = oracle.ACT_SILU
    print(f"[parity] act=silu {layer.name}", flush=True)
    inp = wl.make_inputs(layer)
    f32 = layer.dtype == "f32"
    gpu = _run(inp, a)
    rng = np.random.default_rng(layer.index)
    x, w, b, gy = inp["x"], inp["w"], inp["b"], inp["g"]
    N, C, H, W = x.shape
    K = w.shape[0]
    i = np.unique(rng.integers(0, N * K * H * W, 3000))
    z_ref = oracle.conv3x3_fwd_at(x, w, b, i)
    errs = {"z": rel_err(gpu["z"].ravel()[i], z_ref),
            "y": rel_err(gpu["y"].ravel()[i], oracle.act_forward(z_ref, a))}
    g = oracle.act_grad(gy, gpu["z"], a, bf16=not f32)
    j = np.unique(rng.integers(0, N * C * H * W, 3000))
    errs["dx"] = rel_err(gpu["dx"].ravel()[j], oracle.conv3x3_bwd_data_at(g, w, j))
    j = np.unique(rng.integers(0, K * C * 9, 600))
    errs["dw"] = rel_err(gpu["dw"].ravel()[j], oracle.conv3x3_bwd_weight_at(x, g, j))
    j = np.arange(K)
    errs["db"] = rel_err(gpu["db"][j], oracle.conv3x3_bias_grad_at(g, j))
    print(layer.name, errs)
    _check(errs, layer.dtype, layer.name)
