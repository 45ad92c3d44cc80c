"""Pins for the oracle's input-prologue functions (CPU only).

The prologue reading: the convolution's input is a = SiLU(x * scale[n, c] +
shift[n, c]) (GroupNorm-apply + SiLU), zero-padded after the activation;
backward-data returns the gradient with respect to u = x * scale + shift,
backward-weight the plain one on a.  Checked against things other than the
oracle itself: torch's float64 GroupNorm-free formulation with autograd
(torch.nn.functional.silu and conv2d), an actual torch GroupNorm + SiLU whose
statistics and affine fold into scale and shift, closed forms (scale = 1,
shift = 0 is SiLU(x); scale = 0 makes the input constant per channel inside
the image, and the border outputs then see zeros, not SiLU(shift)), central
differences, and planted slips (padding the activated input with SiLU(shift),
dropping SiLU' from du, swapping the affine order, a per-channel instead of
per-sample scale) that the pins reject."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

SHAPES = [(2, 3, 4, 5, 6), (1, 8, 8, 8, 8), (3, 5, 2, 7, 4), (1, 1, 1, 3, 3)]


def _draw(N, C, K, H, W, seed):
    rng = np.random.default_rng(seed)
    return (rng.normal(size=(N, C, H, W)), rng.uniform(0.3, 1.7, (N, C)),
            rng.normal(size=(N, C)), rng.normal(size=(K, C, 3, 3)) / 3, rng.normal(size=K),
            rng.normal(size=(N, K, H, W)))


def torch_reference(x, s, t, w, b, g):
    T = lambda a, grad=False: torch.tensor(a, dtype=torch.float64, requires_grad=grad)
    tx, tw, tb = T(x, True), T(w, True), T(b, True)
    u = tx * T(s)[:, :, None, None] + T(t)[:, :, None, None]
    u.retain_grad()
    y = F.conv2d(F.silu(u), tw, tb, padding=1)
    (y * T(g)).sum().backward()
    return y.detach().numpy(), u.grad.numpy(), tw.grad.numpy(), tb.grad.numpy()


def check_against_torch(x, s, t, w, b, g, tol=1e-10):
    y_t, du_t, dw_t, db_t = torch_reference(x, s, t, w, b, g)
    got = (oracle.conv3x3_fwd_gnsilu(x, s, t, w, b), oracle.conv3x3_bwd_data_gnsilu(g, w, x, s, t),
           *oracle.conv3x3_bwd_weight_gnsilu(x, s, t, g))
    for a, r in zip(got, (y_t, du_t, dw_t, db_t)):
        assert a.shape == r.shape
        assert np.max(np.abs(a - r)) <= tol * max(1.0, np.max(np.abs(r)))


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_against_torch_autograd(shape):
    check_against_torch(*_draw(*shape, seed=1))


def test_folded_groupnorm_matches_torch_groupnorm():
    """scale / shift folded from a GroupNorm's statistics and affine reproduce
    torch's GroupNorm followed by SiLU."""
    N, C, H, W, G = 2, 8, 5, 6, 4
    rng = np.random.default_rng(2)
    x = rng.normal(1.0, 2.0, (N, C, H, W))
    gamma, beta = rng.normal(size=C), rng.normal(size=C)
    eps = 1e-5
    xg = x.reshape(N, G, -1)
    mean, var = xg.mean(-1), xg.var(-1)
    rstd = 1.0 / np.sqrt(var + eps)
    grp = np.arange(C) // (C // G)
    scale = gamma[None, :] * rstd[:, grp]
    shift = beta[None, :] - mean[:, grp] * scale
    ref = F.silu(F.group_norm(torch.tensor(x), G, torch.tensor(gamma), torch.tensor(beta),
                              eps)).numpy()
    assert np.max(np.abs(oracle.prologue_apply(x, scale, shift) - ref)) < 1e-12


def test_identity_affine_is_silu():
    x, _, _, w, b, _ = _draw(2, 3, 4, 5, 6, seed=3)
    one, zero = np.ones((2, 3)), np.zeros((2, 3))
    assert np.array_equal(oracle.prologue_apply(x, one, zero),
                          oracle.act_forward(x, oracle.ACT_SILU))


def test_padding_is_applied_after_the_activation():
    """scale = 0: the activated input is SiLU(shift) inside the image; outside
    it is zero, so a corner output sees 4 of the 9 taps and an interior one 9."""
    N, C, K, H, W = 1, 2, 1, 4, 5
    x = np.random.default_rng(4).normal(size=(N, C, H, W))
    s = np.zeros((N, C))
    t = np.array([[0.7, -1.3]])
    w = np.ones((K, C, 3, 3))
    y = oracle.conv3x3_fwd_gnsilu(x, s, t, w)
    a = t / (1.0 + np.exp(-t))
    per_tap = a.sum()
    assert abs(y[0, 0, 0, 0] - 4 * per_tap) < 1e-12
    assert abs(y[0, 0, 0, 2] - 6 * per_tap) < 1e-12
    assert abs(y[0, 0, 1, 1] - 9 * per_tap) < 1e-12


def test_du_central_differences():
    N, C, K, H, W = 1, 2, 2, 4, 4
    x, s, t, w, b, g = _draw(N, C, K, H, W, seed=5)
    du = oracle.conv3x3_bwd_data_gnsilu(g, w, x, s, t)
    # u -> x = (u - t) / s: perturbing u by e perturbs x by e / s
    h = 1e-6
    L = lambda xx: float(np.sum(oracle.conv3x3_fwd_gnsilu(xx, s, t, w, b) * g))
    for idx in [(0, 0, 0, 0), (0, 1, 2, 3), (0, 0, 3, 1), (0, 1, 1, 1)]:
        step = h / s[idx[0], idx[1]]
        xp, xm = x.copy(), x.copy()
        xp[idx] += step
        xm[idx] -= step
        fd = (L(xp) - L(xm)) / (2 * h)
        assert abs(fd - du[idx]) < 1e-6 * max(1.0, abs(fd))


MISTAKES = ["pad with silu(shift)", "no silu slope", "affine order", "per-channel scale"]


@pytest.mark.parametrize("mistake", MISTAKES)
def test_planted_mistakes_are_caught(monkeypatch, mistake):
    real_u = oracle._prologue_u
    if mistake == "pad with silu(shift)":
        # the slip: x is zero-padded before the affine and the activation, so
        # the halo holds SiLU(shift) instead of zero
        def fwd(x, s, t, w, b=None):
            xp = np.pad(oracle._f64(x), ((0, 0), (0, 0), (1, 1), (1, 1)))
            a = oracle.act_forward(real_u(xp, s, t), oracle.ACT_SILU)
            return _valid_conv(a, w, b)
        monkeypatch.setattr(oracle, "conv3x3_fwd_gnsilu", fwd)
    elif mistake == "no silu slope":
        monkeypatch.setattr(oracle, "conv3x3_bwd_data_gnsilu",
                            lambda g, w, x, s, t: oracle.conv3x3_bwd_data(g, w))
    elif mistake == "affine order":
        monkeypatch.setattr(oracle, "_prologue_u", lambda x, s, t: (
            oracle._f64(x) + oracle._f64(t)[:, :, None, None]) * oracle._f64(s)[:, :, None, None])
    else:
        monkeypatch.setattr(oracle, "_prologue_u", lambda x, s, t: real_u(
            x, np.broadcast_to(oracle._f64(s)[:1], oracle._f64(s).shape), t))
    args = _draw(2, 3, 4, 5, 6, seed=6)
    with pytest.raises(AssertionError):
        check_against_torch(*args)


def _valid_conv(a_padded, w, b):
    """3x3 'valid' cross-correlation of an already padded input (numpy)."""
    N, C, Hp, Wp = a_padded.shape
    H, W = Hp - 2, Wp - 2
    K = w.shape[0]
    y = np.zeros((N, K, H, W)) + (0 if b is None else np.asarray(b)[None, :, None, None])
    for r in range(3):
        for s in range(3):
            y += np.einsum("nchw,kc->nkhw", a_padded[:, :, r:r + H, s:s + W], w[:, :, r, s])
    return y


def test_bf16_operand_is_exact_activation_rounded_once():
    """bfloat16 mode: the operand is a = SiLU(x * scale + shift) for the
    bfloat16 x, rounded once to the nearest bfloat16 value -- against torch's
    float64 SiLU and a brute-force nearest search over all bfloat16 values;
    the zero padding and the convolutions on it follow."""
    from bf16_ref import nearest_bf16
    x, s, t, w, b, g = _draw(2, 6, 3, 5, 7, 51)
    x = torch.from_numpy(x).bfloat16().double().numpy()
    s = s.astype(np.float32).astype(np.float64)
    t = t.astype(np.float32).astype(np.float64)
    u = torch.from_numpy(x * s[:, :, None, None] + t[:, :, None, None])
    ref = nearest_bf16(F.silu(u).numpy())
    a = oracle.prologue_apply(x, s, t, bf16=True)
    assert np.array_equal(a, ref)
    assert not np.array_equal(a, oracle.prologue_apply(x, s, t))  # it does round
    y = oracle.conv3x3_fwd_gnsilu(x, s, t, w, b, bf16=True)
    assert np.allclose(y, F.conv2d(torch.from_numpy(ref), torch.from_numpy(w),
                                   torch.from_numpy(b), padding=1).numpy(), rtol=0, atol=1e-12)
    dw, db = oracle.conv3x3_bwd_weight_gnsilu(x, s, t, g, bf16=True)
    dw_ref = torch.nn.grad.conv2d_weight(torch.from_numpy(ref), w.shape, torch.from_numpy(g),
                                         padding=1).numpy()
    assert np.allclose(dw, dw_ref, rtol=0, atol=1e-12)
    assert np.allclose(db, g.sum(axis=(0, 2, 3)), rtol=0, atol=1e-12)
