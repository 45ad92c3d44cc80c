"""GPU parity of the bfloat16-output mode (CONV3X3_BF16_IO: bf16 inputs,
y and dx written as bf16) against the oracle, through the C ABI.

The kernel rounds its float32 accumulator; the oracle rounds its exact
result (round to nearest, ties to even).  On integer-valued inputs the
float32 sums are exact, so both round the same value: bit-exact.  On random
inputs the float32 sum differs from the exact one by a few float32 ulps, so
an element may land on the other bfloat16 neighbour only when the exact
value lies within that error of a rounding midpoint: each element must be
within half a bfloat16 spacing of the exact value (plus the float32
accumulation error), and the tensor within the bf16 bar.  The float32
outputs of the same call (the fused activation's z) keep the 1e-4
trip-wire."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import TOL, TRIPWIRE, rel_err

pytestmark = pytest.mark.gpu


def _check_bf16(got, exact, integer, label):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == exact.shape, label
    assert np.all(np.isfinite(got)), (label, "unwritten element")
    if integer:
        bad = np.flatnonzero(got != oracle.round_to_bf16(exact))
        assert bad.size == 0, (label, "integer-exact mismatch", bad[:10])
        return 0.0
    scale = np.max(np.abs(exact))
    # half the bfloat16 spacing at |exact| (8-bit significand), plus a
    # float32 accumulation allowance relative to the tensor's scale
    spacing = np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(exact), 1e-30))).astype(int) - 7)
    slack = 0.5 * spacing * (1 + 2.0 ** -10) + 1e-5 * scale
    bad = np.flatnonzero(np.abs(got - exact) > slack)
    assert bad.size == 0, (label, "beyond half a bfloat16 spacing", bad[:10])
    e = rel_err(got, exact)
    assert e <= TOL["bf16"], (label, e)
    return e


def _gpu(inp, C0=None, act=None):
    import diffusion_unet_x3_amd as lib3
    dev = torch.device("cuda", 0)
    x, w, g, b = (inp[k].to(dev) for k in ("x", "w", "g", "b"))
    bf = torch.bfloat16
    out = {}
    if act is not None:
        y, z = lib3.conv3x3_fwd_act(x, w, b, act=act, out_dtype=bf)
        out.update(y=y, z=z)
    elif C0 is not None:
        x0, x1 = x[:, :C0].contiguous(), x[:, C0:].contiguous()
        out["y"] = lib3.conv3x3_fwd_cat(x0, x1, w, b, out_dtype=bf)
        out["dx0"], out["dx1"] = lib3.conv3x3_bwd_data_cat(g, w, C0, out_dtype=bf)
    else:
        out["y"] = lib3.conv3x3_fwd(x, w, b, out_dtype=bf)
        out["dx"] = lib3.conv3x3_bwd_data(g, w, out_dtype=bf)
    torch.cuda.synchronize()
    for k, v in out.items():
        assert v.dtype == (torch.float32 if k == "z" else bf), k
    return {k: v.float().cpu().double().numpy() for k, v in out.items()}


SHAPES = [(2, 64, 64, 32, 32), (2, 17, 33, 5, 13), (2, 32, 48, 9, 80), (5, 16, 16, 8, 8),
          (32, 16, 256, 32, 32), (32, 256, 16, 32, 32), (2, 40, 130, 10, 72),
          (64, 16, 512, 8, 8)]


@pytest.mark.parametrize("integer", [False, True], ids=["random", "integer"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bf16_outputs_full_compare(shape, integer):
    layer = wl.small_layer(*shape, dtype="bf16", seed=53)
    print(f"[parity] bf16 out {shape} integer={integer}", flush=True)
    inp = wl.make_inputs(layer, integer_exact=integer)
    gpu = _gpu(inp)
    errs = {"y": _check_bf16(gpu["y"], oracle.conv3x3_fwd(inp["x"], inp["w"], inp["b"]),
                             integer, (shape, "y")),
            "dx": _check_bf16(gpu["dx"], oracle.conv3x3_bwd_data(inp["g"], inp["w"]), integer,
                              (shape, "dx"))}
    print(errs)


@pytest.mark.parametrize("integer", [False, True], ids=["random", "integer"])
def test_bf16_outputs_concat(integer):
    N, C0, C1, K, H, W = 2, 32, 48, 64, 16, 16
    layer = wl.small_layer(N, C0 + C1, K, H, W, dtype="bf16", seed=59)
    inp = wl.make_inputs(layer, integer_exact=integer)
    gpu = _gpu(inp, C0=C0)
    _check_bf16(gpu["y"], oracle.conv3x3_fwd(inp["x"], inp["w"], inp["b"]), integer, "cat y")
    dx = oracle.conv3x3_bwd_data(inp["g"], inp["w"])
    _check_bf16(gpu["dx0"], dx[:, :C0], integer, "cat dx0")
    _check_bf16(gpu["dx1"], dx[:, C0:], integer, "cat dx1")


@pytest.mark.parametrize("act", [oracle.ACT_SILU, oracle.ACT_LRELU], ids=["silu", "lrelu"])
def test_bf16_outputs_with_fused_activation(act):
    layer = wl.small_layer(2, 64, 64, 32, 32, dtype="bf16", seed=61)
    inp = wl.make_inputs(layer)
    gpu = _gpu(inp, act=act)
    y_ref, z_ref = oracle.conv3x3_fwd_act(inp["x"], inp["w"], inp["b"], act)
    assert rel_err(gpu["z"], z_ref) <= TRIPWIRE["bf16"]
    _check_bf16(gpu["y"], y_ref, False, "act y")


def test_full_size_bottleneck_sampled():
    layer = wl.CONFIGS[4][0]
    print(f"[parity] bf16 out {layer.name}", flush=True)
    inp = wl.make_inputs(layer)
    gpu = _gpu(inp)
    x, w, b, g = inp["x"], inp["w"], inp["b"], inp["g"]
    N, C, H, W = x.shape
    K = w.shape[0]
    rng = np.random.default_rng(3)
    i = np.unique(rng.integers(0, N * K * H * W, 3000))
    _check_bf16(gpu["y"].ravel()[i], oracle.conv3x3_fwd_at(x, w, b, i), False, "y")
    j = np.unique(rng.integers(0, N * C * H * W, 3000))
    _check_bf16(gpu["dx"].ravel()[j], oracle.conv3x3_bwd_data_at(g, w, j), False, "dx")
