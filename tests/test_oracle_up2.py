"""Pins for the oracle's upsample-then-convolve functions (CPU only).

Reading: nearest-neighbour 2x upsampling (the zero-insertion-plus-FIR
upsampling of the StyleGAN2 page with a 2x2 box filter), then the 3x3
convolution at the upsampled resolution.  Checked against torch
(F.interpolate(mode="nearest") + conv2d, float64 autograd for dx, dw, db),
against an explicit zero insertion followed by the 2x2 box filter, the
adjoint identity <upsample2(x), v> = <x, downsum2(v)>, and planted slips
(a half-pixel shift, a missing block term in the adjoint) that fail them."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

SHAPES = [(2, 3, 4, 3, 5), (1, 8, 8, 4, 4), (2, 5, 2, 1, 1), (1, 2, 3, 6, 2)]


def _draw(N, C, K, H, W, seed):
    rng = np.random.default_rng(seed)
    return (rng.normal(size=(N, C, H, W)), rng.normal(size=(K, C, 3, 3)) / 3,
            rng.normal(size=K), rng.normal(size=(N, K, 2 * H, 2 * W)))


def torch_reference(x, w, b, g):
    T = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    tx, tw, tb = T(x), T(w), T(b)
    y = F.conv2d(F.interpolate(tx, scale_factor=2, mode="nearest"), tw, tb, padding=1)
    (y * torch.tensor(g)).sum().backward()
    return y.detach().numpy(), tx.grad.numpy(), tw.grad.numpy(), tb.grad.numpy()


def check_against_torch(x, w, b, g, tol=1e-10):
    ref = torch_reference(x, w, b, g)
    got = (oracle.conv3x3_fwd_up2(x, w, b), oracle.conv3x3_bwd_data_up2(g, w),
           *oracle.conv3x3_bwd_weight_up2(x, g))
    for a, r in zip(got, ref):
        assert a.shape == r.shape
        assert np.max(np.abs(a - r)) <= tol * max(1.0, np.max(np.abs(r)))


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_against_torch(shape):
    check_against_torch(*_draw(*shape, seed=1))


def test_nearest_is_zero_insertion_then_box_filter():
    x = np.random.default_rng(2).normal(size=(2, 3, 4, 5))
    N, C, H, W = x.shape
    z = np.zeros((N, C, 2 * H, 2 * W))
    z[:, :, ::2, ::2] = x  # a sample after each pixel, as zeros
    # 2x2 box FIR anchored at the inserted sample: out[i, j] = sum of z over
    # rows i-1..i and columns j-1..j (zeros before the start)
    zp = np.pad(z, ((0, 0), (0, 0), (1, 0), (1, 0)))
    box = zp[:, :, 1:, 1:] + zp[:, :, :-1, 1:] + zp[:, :, 1:, :-1] + zp[:, :, :-1, :-1]
    assert np.array_equal(oracle.upsample2(x), box)


def test_downsum_is_the_adjoint():
    rng = np.random.default_rng(3)
    x = rng.normal(size=(2, 3, 4, 5))
    v = rng.normal(size=(2, 3, 8, 10))
    lhs = np.sum(oracle.upsample2(x) * v)
    rhs = np.sum(x * oracle.downsum2(v))
    assert abs(lhs - rhs) < 1e-10 * max(1.0, abs(lhs))


@pytest.mark.parametrize("mistake", ["shifted copies", "three of four terms"])
def test_planted_mistakes_are_caught(monkeypatch, mistake):
    if mistake == "shifted copies":
        def up(x):
            x = oracle._f64(x)
            u = np.repeat(np.repeat(x, 2, axis=2), 2, axis=3)
            return np.concatenate([u[:, :, :1], u[:, :, :-1]], axis=2)  # rows off by one
        monkeypatch.setattr(oracle, "upsample2", up)
    else:
        def ds(du):
            du = oracle._f64(du)
            N, C, H2, W2 = du.shape
            r = du.reshape(N, C, H2 // 2, 2, W2 // 2, 2)
            return r[:, :, :, 0, :, 0] + r[:, :, :, 1, :, 0] + r[:, :, :, 0, :, 1]
        monkeypatch.setattr(oracle, "downsum2", ds)
    with pytest.raises(AssertionError):
        check_against_torch(*_draw(2, 3, 4, 3, 5, seed=4))
