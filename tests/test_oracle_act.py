"""Pins for the oracle's fused-activation functions (CPU only).

The activation reading (identity, SiLU, leaky ReLU with slope 0.2 on the
biased convolution output; the backward multiplies by act'(z)) is checked
against things other than itself: special values worked out by hand, the
exact identities silu(z) - silu(-z) = z and silu'(z) + silu'(-z) = 1, torch's
float64 activations and autograd, central finite differences (elementwise
and through the whole fused convolution), and, for the bfloat16 operand, a
brute-force nearest-value search over every bfloat16 value."""
import numpy as np
import pytest
import torch

import oracle
from bf16_ref import nearest_bf16

ACTS = [oracle.ACT_NONE, oracle.ACT_SILU, oracle.ACT_LRELU]


def test_special_values():
    z = np.array([0.0, 3.0, -3.0, 40.0, -40.0])
    # identity
    assert np.array_equal(oracle.act_forward(z, oracle.ACT_NONE), z)
    assert np.array_equal(oracle.act_grad(np.ones(5), z, oracle.ACT_NONE), np.ones(5))
    # SiLU: sigmoid(0) = 1/2, so silu(0) = 0 and silu'(0) = 1/2; far from 0
    # silu(z) -> max(z, 0) and silu'(z) -> [z > 0]
    y = oracle.act_forward(z, oracle.ACT_SILU)
    d = oracle.act_grad(np.ones(5), z, oracle.ACT_SILU)
    assert y[0] == 0.0 and d[0] == 0.5
    assert abs(y[3] - 40.0) < 1e-12 and abs(y[4]) < 1e-12
    assert abs(d[3] - 1.0) < 1e-12 and abs(d[4]) < 1e-12
    # leaky ReLU, slope 0.2 below zero; the slope at 0 is the negative side's
    y = oracle.act_forward(z, oracle.ACT_LRELU)
    d = oracle.act_grad(np.ones(5), z, oracle.ACT_LRELU)
    assert np.allclose(y, [0.0, 3.0, -0.6, 40.0, -8.0], rtol=0, atol=1e-15)
    assert np.allclose(d, [0.2, 1.0, 0.2, 1.0, 0.2], rtol=0, atol=1e-15)


def test_silu_odd_part_identities():
    z = np.random.default_rng(0).normal(0.0, 3.0, 1000)
    y = oracle.act_forward(z, oracle.ACT_SILU)
    ym = oracle.act_forward(-z, oracle.ACT_SILU)
    assert np.max(np.abs((y - ym) - z)) < 1e-13
    d = oracle.act_grad(np.ones_like(z), z, oracle.ACT_SILU)
    dm = oracle.act_grad(np.ones_like(z), -z, oracle.ACT_SILU)
    assert np.max(np.abs(d + dm - 1.0)) < 1e-14


@pytest.mark.parametrize("act", [oracle.ACT_SILU, oracle.ACT_LRELU])
def test_against_torch_float64(act):
    z = torch.randn(5000, dtype=torch.float64, generator=torch.Generator().manual_seed(1)) * 4
    zr = z.clone().requires_grad_(True)
    f = torch.nn.functional.silu if act == oracle.ACT_SILU else \
        (lambda t: torch.nn.functional.leaky_relu(t, negative_slope=0.2))
    yt = f(zr)
    gy = torch.randn(5000, dtype=torch.float64, generator=torch.Generator().manual_seed(2))
    (gt,) = torch.autograd.grad(yt, zr, gy)
    y = oracle.act_forward(z.numpy(), act)
    g = oracle.act_grad(gy.numpy(), z.numpy(), act)
    assert np.max(np.abs(y - yt.detach().numpy())) < 1e-13
    assert np.max(np.abs(g - gt.numpy())) < 1e-13


@pytest.mark.parametrize("act", [oracle.ACT_SILU, oracle.ACT_LRELU])
def test_slope_is_central_difference(act):
    z = np.random.default_rng(3).normal(0.0, 3.0, 2000)
    if act == oracle.ACT_LRELU:
        z = z[np.abs(z) > 1e-3]  # the kink
    h = 1e-5
    fd = (oracle.act_forward(z + h, act) - oracle.act_forward(z - h, act)) / (2 * h)
    g = oracle.act_grad(np.ones_like(z), z, act)
    assert np.max(np.abs(fd - g)) < 1e-8


@pytest.mark.parametrize("act", ACTS)
def test_fused_backward_is_gradient_of_fused_forward(act):
    """Central differences of L = <act(conv(x, w) + b), gy> in every input,
    weight and bias entry of a tiny problem."""
    rng = np.random.default_rng(4 + act)
    N, C, K, H, W = 1, 2, 2, 4, 5
    x = rng.normal(size=(N, C, H, W))
    w = rng.normal(size=(K, C, 3, 3)) * 0.5
    b = rng.normal(size=K) * 0.5
    gy = rng.normal(size=(N, K, H, W))

    def loss(x_, w_, b_):
        y, _ = oracle.conv3x3_fwd_act(x_, w_, b_, act)
        return float(np.sum(y * gy))

    y, z = oracle.conv3x3_fwd_act(x, w, b, act)
    assert np.min(np.abs(z)) > 1e-4  # no pre-activation on the leaky ReLU's kink
    dx, dw, db = oracle.conv3x3_bwd_act(x, w, gy, z, act)
    h = 1e-6
    for arr, grad in ((x, dx), (w, dw), (b, db)):
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            keep = arr[i]
            arr[i] = keep + h
            lp = loss(x, w, b)
            arr[i] = keep - h
            lm = loss(x, w, b)
            arr[i] = keep
            assert abs((lp - lm) / (2 * h) - grad[i]) < 1e-6, (i, grad[i])


def _torch_slope(z, act):
    zt = torch.from_numpy(np.asarray(z, np.float64)).requires_grad_(True)
    f = torch.nn.functional.silu if act == oracle.ACT_SILU else \
        (lambda t: torch.nn.functional.leaky_relu(t, negative_slope=0.2))
    (s,) = torch.autograd.grad(f(zt), zt, torch.ones_like(zt))
    return s.numpy()


@pytest.mark.parametrize("act", ACTS)
def test_bf16_operand_is_exact_product_rounded_once(act):
    """The bfloat16 path's operand: g = gy * act'(z) exactly, rounded once to
    the nearest bfloat16 value (ties to even).  gy is a bfloat16 gradient and
    z the float32 pre-activation."""
    rng = np.random.default_rng(5 + act)
    gy = torch.from_numpy(rng.normal(size=20000)).bfloat16().double().numpy()
    z = rng.normal(0.0, 3.0, size=20000).astype(np.float32).astype(np.float64)
    slope = np.ones_like(z) if act == oracle.ACT_NONE else _torch_slope(z, act)
    g = oracle.act_grad(gy, z, act, bf16=True)
    assert np.array_equal(g, nearest_bf16(gy * slope))
    # every value is a bfloat16 value
    assert np.array_equal(g, torch.from_numpy(g).float().bfloat16().double().numpy())


def test_bf16_operand_does_not_round_through_float32():
    """Where the float32 product gy32 * silu'32(z) lands on the other side of a
    bfloat16 rounding boundary than the exact product, the operand follows
    the exact product.  The search keeps only such elements, so a
    float32-product oracle would fail every one of them."""
    rng = np.random.default_rng(11)
    gy = torch.from_numpy(rng.normal(size=2_000_000)).bfloat16().double().numpy()
    z = rng.normal(0.0, 3.0, size=gy.size).astype(np.float32)
    zt = torch.from_numpy(z).requires_grad_(True)
    (s32,) = torch.autograd.grad(torch.nn.functional.silu(zt), zt, torch.ones_like(zt))
    f32_path = (torch.from_numpy(gy.astype(np.float32)) * s32).bfloat16().double().numpy()
    exact = nearest_bf16(gy * _torch_slope(z, oracle.ACT_SILU))
    differ = f32_path != exact
    assert differ.sum() >= 10
    g = oracle.act_grad(gy[differ], z[differ].astype(np.float64), oracle.ACT_SILU, bf16=True)
    assert np.array_equal(g, exact[differ])
