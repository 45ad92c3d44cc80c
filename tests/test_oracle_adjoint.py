"""Pin the three oracle passes to each other through the adjoint identities
of the bilinear map y = conv(x; w):  <conv(x;w), g> = <x, bwd_data(g;w)>,
<bwd_weight(x,g), v> = <conv(x;v), g>, <db, u> = <u broadcast, g>."""
import numpy as np
import pytest

import oracle

SHAPES = [(1, 1, 1, 1, 1), (1, 1, 1, 3, 3), (2, 3, 4, 5, 6), (1, 8, 8, 9, 11), (2, 5, 3, 1, 7),
          (2, 8, 8, 9, 11), (1, 2, 3, 7, 1)]


@pytest.mark.parametrize("shape", SHAPES)
def test_adjoint_identities(shape):
    N, C, K, H, W = shape
    rng = np.random.default_rng(sum(shape))
    x = rng.standard_normal((N, C, H, W))
    w = rng.standard_normal((K, C, 3, 3))
    v = rng.standard_normal((K, C, 3, 3))
    g = rng.standard_normal((N, K, H, W))
    u = rng.standard_normal(K)

    def rel(a, b):
        return abs(a - b) / max(1.0, abs(a), abs(b))

    lhs = np.sum(oracle.conv3x3_fwd(x, w) * g)
    rhs = np.sum(x * oracle.conv3x3_bwd_data(g, w))
    assert rel(lhs, rhs) < 1e-12
    dw, db = oracle.conv3x3_bwd_weight(x, g)
    assert rel(np.sum(dw * v), np.sum(oracle.conv3x3_fwd(x, v) * g)) < 1e-12
    assert rel(np.sum(db * u), np.sum(u[None, :, None, None] * g)) < 1e-12
