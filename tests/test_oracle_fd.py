"""Pin the backward passes as derivatives: central finite differences of
L(x, w, b) = <conv(x; w) + b, g>.  L is linear in each argument, so the
central difference with step 2^-10 is exact up to float64 rounding."""
import numpy as np

import oracle

EPS = 2.0 ** -10


def _L(x, w, b, g):
    return float(np.sum(oracle.conv3x3_fwd(x, w, b) * g))


def test_weight_gradient_finite_differences():
    N, C, K, H, W = 2, 2, 3, 4, 5
    rng = np.random.default_rng(11)
    x = rng.standard_normal((N, C, H, W))
    w = rng.standard_normal((K, C, 3, 3))
    b = rng.standard_normal(K)
    g = rng.standard_normal((N, K, H, W))
    dw, db = oracle.conv3x3_bwd_weight(x, g)
    scale = np.max(np.abs(dw))
    for i in range(w.size):  # all 54 weights
        wp, wm = w.copy(), w.copy()
        wp.flat[i] += EPS
        wm.flat[i] -= EPS
        fd = (_L(x, wp, b, g) - _L(x, wm, b, g)) / (2 * EPS)
        assert abs(fd - dw.flat[i]) <= 1e-9 * scale, i
    for k in range(K):
        bp, bm = b.copy(), b.copy()
        bp[k] += EPS
        bm[k] -= EPS
        fd = (_L(x, w, bp, g) - _L(x, w, bm, g)) / (2 * EPS)
        assert abs(fd - db[k]) <= 1e-9 * max(1.0, abs(db[k])), k


def test_input_gradient_finite_differences():
    N, C, K, H, W = 1, 2, 3, 4, 5
    rng = np.random.default_rng(12)
    x = rng.standard_normal((N, C, H, W))
    w = rng.standard_normal((K, C, 3, 3))
    g = rng.standard_normal((N, K, H, W))
    dx = oracle.conv3x3_bwd_data(g, w)
    scale = np.max(np.abs(dx))
    for i in range(x.size):  # all 40 inputs, borders included
        xp, xm = x.copy(), x.copy()
        xp.flat[i] += EPS
        xm.flat[i] -= EPS
        fd = (_L(xp, w, None, g) - _L(xm, w, None, g)) / (2 * EPS)
        assert abs(fd - dx.flat[i]) <= 1e-9 * scale, i
