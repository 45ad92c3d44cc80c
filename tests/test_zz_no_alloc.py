"""conv3x3_bwd_weight_noalloc against conv3x3_bwd_weight (GPU).

The no-allocation entry point runs the same kernels with the split-K partial
sums in the library's own device array instead of a caller workspace, so its
dw and db must equal the plain entry point's bit for bit, and both must meet
the oracle's bar.  Two calls in a row share the array: the second, on a
smaller problem, must not see the first one's leftovers.  Everything goes
through the C ABI with preallocated outputs."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import TRIPWIRE, rel_err

pytestmark = pytest.mark.gpu

# (first, second): the second is smaller; both need split-K scratch.  The
# few-channel pair runs the image-stem backward-weight kernel, whose
# slices use their own slot layout ([K][32 NB] per slice).
PAIRS = [
    ((8, 64, 64, 32, 32, "f32"), (2, 24, 40, 10, 12, "f32")),
    ((8, 64, 64, 32, 32, "bf16"), (2, 32, 24, 8, 16, "bf16")),
    ((8, 3, 128, 64, 64, "bf16"), (2, 4, 40, 16, 24, "bf16")),
]


def _lib():
    import diffusion_unet_x3_amd as lib3
    return lib3


def _inputs(shape, seed):
    N, C, K, H, W, dt = shape
    inp = wl.make_inputs(wl.small_layer(N, C, K, H, W, dt, seed=seed))
    dev = torch.device("cuda", 0)
    return inp, inp["x"].to(dev), inp["g"].to(dev)


def _plain(lib3, x, g):
    """conv3x3_bwd_weight with a torch workspace, through the C ABI."""
    N, C, H, W = x.shape
    K = g.shape[1]
    code = lib3.CONV3X3_F32 if x.dtype == torch.float32 else lib3.CONV3X3_BF16
    need = lib3.lib.conv3x3_bwd_weight_workspace_size(N, C, K, H, W, code)
    assert 0 < need <= 40 << 20
    ws = torch.empty(need, dtype=torch.uint8, device=x.device)
    dw = torch.full((K, C, 3, 3), float("nan"), device=x.device)
    db = torch.full((K,), float("nan"), device=x.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib3.lib.conv3x3_bwd_weight(x.data_ptr(), g.data_ptr(), dw.data_ptr(), db.data_ptr(),
                                     ws.data_ptr(), need, N, C, K, H, W, code, stream)
    assert rc == 0, lib3.conv3x3_status_string(rc)
    return dw, db


def _noalloc(lib3, x, g):
    N, C, H, W = x.shape
    K = g.shape[1]
    code = lib3.CONV3X3_F32 if x.dtype == torch.float32 else lib3.CONV3X3_BF16
    dw = torch.full((K, C, 3, 3), float("nan"), device=x.device)
    db = torch.full((K,), float("nan"), device=x.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib3.lib.conv3x3_bwd_weight_noalloc(x.data_ptr(), g.data_ptr(), dw.data_ptr(),
                                             db.data_ptr(), N, C, K, H, W, code, stream)
    assert rc == 0, lib3.conv3x3_status_string(rc)
    return dw, db


@pytest.mark.parametrize("pair", PAIRS, ids=["f32", "bf16", "bf16_few_channel"])
def test_noalloc_matches_plain_entry_point(pair):
    lib3 = _lib()
    for i, shape in enumerate(pair):
        print(f"noalloc call {i}: shape {shape}", flush=True)
        inp, x, g = _inputs(shape, seed=20 + i)
        dw, db = _noalloc(lib3, x, g)
        torch.cuda.synchronize()
        dw_ref, db_ref = _plain(lib3, x, g)
        torch.cuda.synchronize()
        assert torch.equal(dw, dw_ref), f"call {i}: dw differs from conv3x3_bwd_weight"
        assert torch.equal(db, db_ref), f"call {i}: db differs from conv3x3_bwd_weight"
        odw, odb = oracle.conv3x3_bwd_weight(inp["x"], inp["g"])
        tol = TRIPWIRE[shape[-1]]
        assert rel_err(dw.cpu().double().numpy(), odw) <= tol
        assert rel_err(db.cpu().double().numpy(), odb) <= tol


def test_noalloc_without_db_and_back_to_back():
    """db = NULL, and two calls enqueued back to back on one stream (the
    second reuses the array only after the first's reduce has run)."""
    lib3 = _lib()
    inp_a, xa, ga = _inputs((8, 64, 64, 32, 32, "f32"), seed=30)
    inp_b, xb, gb = _inputs((4, 64, 64, 16, 16, "f32"), seed=31)
    dwa = torch.empty((64, 64, 3, 3), device="cuda")
    dwb = torch.empty((64, 64, 3, 3), device="cuda")
    lib3.conv3x3_bwd_weight_noalloc(xa, ga, dwa)
    lib3.conv3x3_bwd_weight_noalloc(xb, gb, dwb)
    torch.cuda.synchronize()
    ra, _ = _plain(lib3, xa, ga)
    rb, _ = _plain(lib3, xb, gb)
    torch.cuda.synchronize()
    assert torch.equal(dwa, ra) and torch.equal(dwb, rb)
    assert np.isfinite(dwb.cpu().numpy()).all()
