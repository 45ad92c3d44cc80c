"""Pin the oracle with invariants that follow from the definition: delta
kernels give the identity, one-hot kernels give zero-filled shifts (computed
here with array slicing), the map is bilinear, and it commutes with interior
translations."""
import numpy as np
import pytest

import oracle


def _shift(a, dr, dc):
    """out[..., h, w] = a[..., h+dr, w+dc], zero outside (slicing, no loops)."""
    out = np.zeros_like(a)
    H, W = a.shape[-2:]
    hs, he = max(0, -dr), min(H, H - dr)
    ws, we = max(0, -dc), min(W, W - dc)
    if hs < he and ws < we:
        out[..., hs:he, ws:we] = a[..., hs + dr:he + dr, ws + dc:we + dc]
    return out


def test_delta_kernel_is_identity():
    rng = np.random.default_rng(2)
    C = 4
    x = rng.standard_normal((2, C, 5, 7))
    w = np.zeros((C, C, 3, 3))
    for c in range(C):
        w[c, c, 1, 1] = 1.0
    assert np.array_equal(oracle.conv3x3_fwd(x, w), x)
    assert np.array_equal(oracle.conv3x3_bwd_data(x, w), x)


@pytest.mark.parametrize("r", [0, 1, 2])
@pytest.mark.parametrize("s", [0, 1, 2])
def test_one_hot_kernel_is_shift(r, s):
    rng = np.random.default_rng(3 + 3 * r + s)
    C, K = 3, 2
    x = rng.standard_normal((2, C, 6, 5))
    g = rng.standard_normal((2, K, 6, 5))
    w = np.zeros((K, C, 3, 3))
    # output k reads input channel (k+1) % C through tap (r, s) with weight 2
    for k in range(K):
        w[k, (k + 1) % C, r, s] = 2.0
    y = oracle.conv3x3_fwd(x, w)
    for k in range(K):
        assert np.array_equal(y[:, k], 2.0 * _shift(x[:, (k + 1) % C], r - 1, s - 1))
    dx = oracle.conv3x3_bwd_data(g, w)
    exp = np.zeros_like(x)
    for k in range(K):
        exp[:, (k + 1) % C] += 2.0 * _shift(g[:, k], 1 - r, 1 - s)
    assert np.array_equal(dx, exp)


def test_weight_gradient_of_single_tap_is_shifted_inner_product():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 2, 5, 4))
    g = rng.standard_normal((3, 3, 5, 4))
    dw, db = oracle.conv3x3_bwd_weight(x, g)
    for k in range(3):
        for c in range(2):
            for r in range(3):
                for s in range(3):
                    ref = np.sum(g[:, k] * _shift(x[:, c], r - 1, s - 1))
                    assert abs(dw[k, c, r, s] - ref) <= 1e-12 * max(1.0, abs(ref))
    assert np.allclose(db, g.sum(axis=(0, 2, 3)), rtol=1e-13, atol=1e-13)


def test_bilinearity():
    rng = np.random.default_rng(5)
    x1, x2 = rng.standard_normal((2, 2, 3, 6, 5))
    w1, w2 = rng.standard_normal((2, 4, 3, 3, 3))
    g1, g2 = rng.standard_normal((2, 2, 4, 6, 5))
    a, b = 0.75, -1.5

    def close(u, v):
        return np.max(np.abs(u - v)) <= 1e-12 * max(1.0, np.max(np.abs(v)))

    f = oracle.conv3x3_fwd
    assert close(f(a * x1 + b * x2, w1), a * f(x1, w1) + b * f(x2, w1))
    assert close(f(x1, a * w1 + b * w2), a * f(x1, w1) + b * f(x1, w2))
    bd = oracle.conv3x3_bwd_data
    assert close(bd(a * g1 + b * g2, w1), a * bd(g1, w1) + b * bd(g2, w1))
    assert close(bd(g1, a * w1 + b * w2), a * bd(g1, w1) + b * bd(g1, w2))
    bw = lambda x, g: oracle.conv3x3_bwd_weight(x, g)[0]
    assert close(bw(a * x1 + b * x2, g1), a * bw(x1, g1) + b * bw(x2, g1))
    assert close(bw(x1, a * g1 + b * g2), a * bw(x1, g1) + b * bw(x1, g2))


def test_interior_translation_equivariance():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((1, 2, 9, 10))
    w = rng.standard_normal((3, 2, 3, 3))
    y = oracle.conv3x3_fwd(x, w)
    xs = _shift(x, -1, -2)  # xs[h, w] = x[h-1, w-2]
    ys = oracle.conv3x3_fwd(xs, w)
    # away from borders the shifted input gives the shifted output
    assert np.allclose(ys[..., 2:-1, 3:-1], y[..., 1:-2, 1:-3], rtol=0, atol=1e-12)


def test_border_taps_read_zero_padding():
    # a 1x1 image: only the centre tap can contribute
    rng = np.random.default_rng(7)
    x = rng.standard_normal((2, 3, 1, 1))
    w = rng.standard_normal((4, 3, 3, 3))
    b = rng.standard_normal(4)
    y = oracle.conv3x3_fwd(x, w, b)
    exp = np.einsum("nc,kc->nk", x[:, :, 0, 0], w[:, :, 1, 1]) + b
    assert np.allclose(y[:, :, 0, 0], exp, rtol=1e-13, atol=1e-13)
