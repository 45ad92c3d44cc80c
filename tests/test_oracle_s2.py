"""Pins for the oracle's stride-2 convolution (CPU only): torch's float64
conv2d(stride=2, padding=1) and autograd, a direct evaluation of one output
from its nine taps, the adjoint identity <conv_s2(x), g> = <x, bwd_data_s2(g)>,
and planted slips (odd pixels kept, zeros inserted at the odd pixels) that
the pins reject."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

SHAPES = [(2, 3, 4, 6, 8), (1, 8, 8, 8, 8), (2, 5, 2, 2, 2), (1, 2, 3, 10, 4)]


def _draw(N, C, K, H, W, seed):
    rng = np.random.default_rng(seed)
    return (rng.normal(size=(N, C, H, W)), rng.normal(size=(K, C, 3, 3)) / 3,
            rng.normal(size=K), rng.normal(size=(N, K, H // 2, W // 2)))


def torch_reference(x, w, b, g):
    T = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    tx, tw, tb = T(x), T(w), T(b)
    y = F.conv2d(tx, tw, tb, stride=2, padding=1)
    (y * torch.tensor(g)).sum().backward()
    return y.detach().numpy(), tx.grad.numpy(), tw.grad.numpy(), tb.grad.numpy()


def check_against_torch(x, w, b, g, tol=1e-10):
    ref = torch_reference(x, w, b, g)
    got = (oracle.conv3x3_fwd_s2(x, w, b), oracle.conv3x3_bwd_data_s2(g, w),
           *oracle.conv3x3_bwd_weight_s2(x, g))
    for a, r in zip(got, ref):
        assert a.shape == r.shape
        assert np.max(np.abs(a - r)) <= tol * max(1.0, np.max(np.abs(r)))


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_against_torch(shape):
    check_against_torch(*_draw(*shape, seed=1))


def test_one_output_by_hand():
    x, w, b, _ = _draw(1, 2, 1, 6, 6, seed=2)
    y = oracle.conv3x3_fwd_s2(x, w, b)
    h, ww = 1, 2  # reads input rows 1..3 and columns 3..5
    ref = b[0] + sum(x[0, c, 2 * h + r - 1, 2 * ww + s - 1] * w[0, c, r, s]
                     for c in range(2) for r in range(3) for s in range(3))
    assert abs(y[0, 0, h, ww] - ref) < 1e-12


def test_adjoint():
    x, w, _, g = _draw(2, 3, 4, 6, 8, seed=3)
    lhs = np.sum(oracle.conv3x3_fwd_s2(x, w) * g)
    rhs = np.sum(x * oracle.conv3x3_bwd_data_s2(g, w))
    assert abs(lhs - rhs) < 1e-10 * max(1.0, abs(lhs))


@pytest.mark.parametrize("mistake", ["odd pixels kept", "zeros at the even pixels"])
def test_planted_mistakes_are_caught(monkeypatch, mistake):
    if mistake == "odd pixels kept":
        monkeypatch.setattr(oracle, "conv3x3_fwd_s2",
                            lambda x, w, b=None: oracle.conv3x3_fwd(x, w, b)[:, :, 1::2, 1::2])
    else:
        def zi(g):
            g = oracle._f64(g)
            N, K, H, W = g.shape
            z = np.zeros((N, K, 2 * H, 2 * W))
            z[:, :, 1::2, 1::2] = g
            return z
        monkeypatch.setattr(oracle, "zero_insert2", zi)
    with pytest.raises(AssertionError):
        check_against_torch(*_draw(2, 3, 4, 6, 8, seed=4))
