"""Pins for the oracle's concatenated-input functions (CPU only).

The oracle defines the convolution of the channel concatenation [x0 ; x1]
by concatenating and calling its plain convolution.  These tests check it
against things other than itself: torch's float64 convolution and autograd
on torch.cat, the block identities that follow from linearity (the forward
is the sum of the two half convolutions with the matching halves of w; each
input gradient is the plain backward-data through its half of w; each half
of dw is the plain backward-weight of its half of the input), the
degenerate splits with an empty half, and exact integer results.  A planted
mistake (halves swapped, split at the wrong channel) fails them."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

SHAPES = [(2, 3, 5, 4, 7, 6), (1, 8, 8, 16, 8, 8), (2, 1, 6, 3, 5, 9), (1, 13, 3, 7, 4, 11)]


def _draw(N, C0, C1, K, H, W, seed, integer=False):
    rng = np.random.default_rng(seed)
    if integer:
        d = lambda *s: rng.integers(-2, 3, s).astype(np.float64)
    else:
        d = lambda *s: rng.normal(size=s)
    return d(N, C0, H, W), d(N, C1, H, W), d(K, C0 + C1, 3, 3), d(K), d(N, K, H, W)


def torch_reference(x0, x1, w, b, g):
    """float64 torch: forward and gradients of <conv(cat(x0, x1)), g>."""
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    tx0, tx1, tw, tb = t(x0), t(x1), t(w), t(b)
    y = F.conv2d(torch.cat([tx0, tx1], 1), tw, tb, padding=1)
    (y * torch.tensor(g)).sum().backward()
    return (y.detach().numpy(), tx0.grad.numpy(), tx1.grad.numpy(), tw.grad.numpy(),
            tb.grad.numpy())


def check_against_torch(x0, x1, w, b, g, tol=1e-10):
    C0 = x0.shape[1]
    y_t, dx0_t, dx1_t, dw_t, db_t = torch_reference(x0, x1, w, b, g)
    y = oracle.conv3x3_fwd_cat(x0, x1, w, b)
    dx0, dx1 = oracle.conv3x3_bwd_data_cat(g, w, C0)
    dw, db = oracle.conv3x3_bwd_weight_cat(x0, x1, g)
    for got, ref in ((y, y_t), (dx0, dx0_t), (dx1, dx1_t), (dw, dw_t), (db, db_t)):
        assert got.shape == ref.shape
        assert np.max(np.abs(got - ref)) <= tol * max(1.0, np.max(np.abs(ref)))


def check_block_identities(x0, x1, w, b, g, tol=1e-12):
    C0 = x0.shape[1]
    w0, w1 = w[:, :C0], w[:, C0:]
    scale = lambda r: tol * max(1.0, np.max(np.abs(r)))
    y = oracle.conv3x3_fwd_cat(x0, x1, w, b)
    ref = oracle.conv3x3_fwd(x0, w0, b) + oracle.conv3x3_fwd(x1, w1, None)
    assert np.max(np.abs(y - ref)) <= scale(ref)
    dx0, dx1 = oracle.conv3x3_bwd_data_cat(g, w, C0)
    for got, wh in ((dx0, w0), (dx1, w1)):
        ref = oracle.conv3x3_bwd_data(g, wh)
        assert got.shape == ref.shape
        assert np.max(np.abs(got - ref)) <= scale(ref)
    dw, db = oracle.conv3x3_bwd_weight_cat(x0, x1, g)
    for got, xh in ((dw[:, :C0], x0), (dw[:, C0:], x1)):
        ref, _ = oracle.conv3x3_bwd_weight(xh, g, False)
        assert np.max(np.abs(got - ref)) <= scale(ref)
    assert np.allclose(db, g.sum(axis=(0, 2, 3)), rtol=0, atol=1e-10)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_against_torch(shape):
    check_against_torch(*_draw(*shape, seed=1))


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_block_identities(shape):
    check_block_identities(*_draw(*shape, seed=2))


def test_integer_inputs_exact():
    x0, x1, w, b, g = _draw(2, 5, 3, 4, 6, 7, seed=3, integer=True)
    y_t, dx0_t, dx1_t, dw_t, db_t = torch_reference(x0, x1, w, b, g)
    assert np.array_equal(oracle.conv3x3_fwd_cat(x0, x1, w, b), y_t)
    dx0, dx1 = oracle.conv3x3_bwd_data_cat(g, w, 5)
    assert np.array_equal(dx0, dx0_t) and np.array_equal(dx1, dx1_t)
    dw, db = oracle.conv3x3_bwd_weight_cat(x0, x1, g)
    assert np.array_equal(dw, dw_t) and np.array_equal(db, db_t)


@pytest.mark.parametrize("empty", [0, 1])
def test_empty_half_is_the_plain_convolution(empty):
    x0, x1, w, b, g = _draw(2, 4, 4, 3, 5, 6, seed=4)
    full = x1 if empty == 0 else x0
    none = np.zeros((2, 0, 5, 6))
    halves = (none, full) if empty == 0 else (full, none)
    w4 = w[:, :4]
    assert np.array_equal(oracle.conv3x3_fwd_cat(*halves, w4, b), oracle.conv3x3_fwd(full, w4, b))
    dx0, dx1 = oracle.conv3x3_bwd_data_cat(g, w4, 0 if empty == 0 else 4)
    assert (dx0 if empty == 0 else dx1).shape == (2, 0, 5, 6)
    assert np.array_equal(dx1 if empty == 0 else dx0, oracle.conv3x3_bwd_data(g, w4))
    dw, db = oracle.conv3x3_bwd_weight_cat(*halves, g)
    ref_dw, ref_db = oracle.conv3x3_bwd_weight(full, g)
    assert np.array_equal(dw, ref_dw) and np.array_equal(db, ref_db)


def test_sampled_functions_match_full():
    x0, x1, w, b, g = _draw(2, 3, 5, 4, 7, 6, seed=5)
    y = oracle.conv3x3_fwd_cat(x0, x1, w, b)
    i = np.arange(0, y.size, 7)
    assert np.allclose(oracle.conv3x3_fwd_cat_at(x0, x1, w, b, i), y.ravel()[i], rtol=0,
                       atol=1e-12)
    dw, _ = oracle.conv3x3_bwd_weight_cat(x0, x1, g)
    j = np.arange(0, dw.size, 5)
    assert np.allclose(oracle.conv3x3_bwd_weight_cat_at(x0, x1, g, j), dw.ravel()[j], rtol=0,
                       atol=1e-12)


@pytest.mark.parametrize("mistake", ["swapped halves", "split at C1"])
def test_planted_mistakes_are_caught(monkeypatch, mistake):
    """A plausible slip in the concatenation functions fails the pins."""
    if mistake == "swapped halves":
        monkeypatch.setattr(oracle, "_cat", lambda a, b: np.concatenate(
            [oracle._f64(b), oracle._f64(a)], axis=1))
    else:
        real = oracle.conv3x3_bwd_data_cat

        def split_wrong(g, w, C0):
            dx0, dx1 = real(g, w, w.shape[1] - C0)
            return dx0, dx1
        monkeypatch.setattr(oracle, "conv3x3_bwd_data_cat", split_wrong)
    args = _draw(2, 3, 5, 4, 7, 6, seed=6)
    with pytest.raises(AssertionError):
        check_against_torch(*args)
    with pytest.raises(AssertionError):
        check_block_identities(*args)
