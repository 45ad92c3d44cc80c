"""Pin the oracle to two independent formulations of the same special case:
PyTorch's CPU convolution and its gradients in float64, and an explicit
im2col + numpy matrix product in float64."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

SHAPES = [(1, 1, 1, 1, 1), (2, 3, 4, 5, 6), (1, 7, 5, 8, 3), (3, 4, 6, 2, 9), (1, 16, 8, 12, 12)]


def _im2col_fwd(x, w, b):
    N, C, H, W = x.shape
    K = w.shape[0]
    xp = np.pad(x, ((0, 0), (0, 0), (1, 1), (1, 1)))
    cols = np.empty((N, C, 3, 3, H, W))
    for r in range(3):
        for s in range(3):
            cols[:, :, r, s] = xp[:, :, r:r + H, s:s + W]
    A = cols.reshape(N, C * 9, H * W)
    y = np.matmul(w.reshape(K, C * 9)[None], A).reshape(N, K, H, W)
    return y + b[None, :, None, None]


@pytest.mark.parametrize("shape", SHAPES)
def test_against_torch_float64(shape):
    N, C, K, H, W = shape
    rng = np.random.default_rng(100 + sum(shape))
    x = rng.standard_normal((N, C, H, W))
    w = rng.standard_normal((K, C, 3, 3))
    b = rng.standard_normal(K)
    g = rng.standard_normal((N, K, H, W))
    tx, tw, tb, tg = (torch.from_numpy(a) for a in (x, w, b, g))
    y_ref = F.conv2d(tx, tw, tb, stride=1, padding=1).numpy()
    dx_ref = torch.nn.grad.conv2d_input(tx.shape, tw, tg, stride=1, padding=1).numpy()
    dw_ref = torch.nn.grad.conv2d_weight(tx, tw.shape, tg, stride=1, padding=1).numpy()

    def rel(a, r):
        return np.max(np.abs(a - r)) / max(1e-300, np.max(np.abs(r)))

    assert rel(oracle.conv3x3_fwd(x, w, b), y_ref) < 1e-12
    assert rel(oracle.conv3x3_bwd_data(g, w), dx_ref) < 1e-12
    dw, db = oracle.conv3x3_bwd_weight(x, g)
    assert rel(dw, dw_ref) < 1e-12
    assert rel(db, g.sum(axis=(0, 2, 3))) < 1e-12


@pytest.mark.parametrize("shape", SHAPES)
def test_against_im2col(shape):
    N, C, K, H, W = shape
    rng = np.random.default_rng(200 + sum(shape))
    x = rng.standard_normal((N, C, H, W))
    w = rng.standard_normal((K, C, 3, 3))
    b = rng.standard_normal(K)
    ref = _im2col_fwd(x, w, b)
    got = oracle.conv3x3_fwd(x, w, b)
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))
