"""CPU checks of the GPU parity tests' sampler: on every full-size layer it
compares at least one element of every workgroup tile (and 32-channel
group) of the forward and backward-data plans, and of every (32 k, 32 c,
tap) block of dw -- so a wrong tile, wave or slice cannot hide between
random samples."""
import numpy as np
import pytest

import workloads as wl
from parity_util import stratified_indices

LAYERS = [l for c in (2, 3, 4, 5) for l in wl.CONFIGS[c]]


def _cdiv(a, b):
    return -(-a // b)


@pytest.mark.parametrize("layer", LAYERS, ids=lambda l: l.name)
def test_every_tile_has_a_compared_element(layer):
    import diffusion_unet_x3_amd as lib3
    N, C, K, H, W = layer.shape
    code = lib3.CONV3X3_BF16 if layer.dtype == "bf16" else lib3.CONV3X3_F32
    rng = np.random.default_rng(layer.index)
    iy, idx, iw = stratified_indices(N, C, K, H, W, layer.dtype, 100, rng)
    for ind, Co, pass_ in ((iy, K, lib3.PASS_FWD), (idx, C, lib3.PASS_BWD_DATA)):
        p = lib3.conv3x3_plan(pass_, N, C, K, H, W, code)
        assert ind.min() >= 0 and ind.max() < N * Co * H * W
        w_ = ind % W
        h_ = (ind // W) % H
        c_ = (ind // (W * H)) % Co
        n_ = ind // (W * H * Co)
        ti, th, tw = p["tile_imgs"], p["tile_h"], p["tile_w"]
        hit = set(zip((n_ // ti).tolist(), (h_ // th).tolist(), (w_ // tw).tolist(),
                      (c_ // 32).tolist()))
        want = _cdiv(N, ti) * _cdiv(H, th) * _cdiv(W, tw) * _cdiv(Co, 32)
        assert len(hit) == want, (layer.name, pass_, len(hit), want)
        # and every channel tile of the plan
        chans = set((c_ // p["tile_m"]).tolist())
        assert len(chans) == _cdiv(Co, p["tile_m"])
    t = iw % 9
    c_ = (iw // 9) % C
    k_ = iw // (9 * C)
    assert iw.max() < K * C * 9
    hit = set(zip((k_ // 32).tolist(), (c_ // 32).tolist(), t.tolist()))
    assert len(hit) == _cdiv(K, 32) * _cdiv(C, 32) * 9
