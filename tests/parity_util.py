"""Helpers for the GPU parity tests: run the three passes through the C ABI
on seeded inputs, compute the oracle (whole tensors, or a sample of output
elements for full-size layers), and compare with the max|err| / max|ref|
metric.  Not collected by pytest."""
import numpy as np
import torch

import oracle
import workloads as wl

TOL = {"f32": 2e-5, "bf16": 1e-2}
# bf16 inputs: products are exact and the sums are float32, so the error
# against the oracle run on the same bf16 values is float32 rounding only.
# This tighter trip-wire catches a dropped term that 1e-2 could hide.
TRIPWIRE = {"f32": 2e-5, "bf16": 1e-4}


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), "non-finite output (unwritten element?)"
    scale = np.max(np.abs(ref)) if ref.size else 0.0
    err = np.max(np.abs(got - ref)) if ref.size else 0.0
    if scale == 0.0:
        return 0.0 if err == 0.0 else float("inf")
    return float(err / scale)


def run_gpu(inp, want_db=True, with_bias=True):
    """All three passes on cuda:0; outputs prefilled with NaN so that an
    element a kernel forgets to write cannot pass."""
    import diffusion_unet_x3_amd as lib3
    dev = torch.device("cuda", 0)
    x, w, g = (inp[k].to(dev) for k in ("x", "w", "g"))
    b = inp["b"].to(dev) if (with_bias and inp["b"] is not None) else None
    N, C, H, W = x.shape
    K = w.shape[0]
    nan = float("nan")
    y = torch.full((N, K, H, W), nan, device=dev)
    dx = torch.full((N, C, H, W), nan, device=dev)
    dw = torch.full((K, C, 3, 3), nan, device=dev)
    db = torch.full((K,), nan, device=dev) if want_db else None
    lib3.conv3x3_fwd(x, w, b, out=y)
    lib3.conv3x3_bwd_data(g, w, out=dx)
    lib3.conv3x3_bwd_weight(x, g, want_db=want_db, dw=dw, db=db)
    torch.cuda.synchronize()
    out = {"y": y.cpu().double().numpy(), "dx": dx.cpu().double().numpy(),
           "dw": dw.cpu().double().numpy()}
    out["db"] = db.cpu().double().numpy() if want_db else None
    return out


def oracle_full(inp, with_bias=True):
    b = inp["b"] if with_bias else None
    y = oracle.conv3x3_fwd(inp["x"], inp["w"], b)
    dx = oracle.conv3x3_bwd_data(inp["g"], inp["w"])
    dw, db = oracle.conv3x3_bwd_weight(inp["x"], inp["g"])
    return {"y": y, "dx": dx, "dw": dw, "db": db}


def _border_and_random(shape, count, rng):
    """Flat indices into a [A, B, H, W] tensor: every border pixel of the
    first and last (a, b) planes, plus `count` random elements."""
    A, B, H, W = shape
    idx = []
    for a, bb in ((0, 0), (A - 1, B - 1), (0, B - 1)):
        base = (a * B + bb) * H * W
        for h in range(H):
            for w in range(W):
                if h in (0, H - 1) or w in (0, W - 1):
                    idx.append(base + h * W + w)
    idx.extend(rng.integers(0, A * B * H * W, count).tolist())
    return np.unique(np.array(idx, dtype=np.int64))


def _dw_indices(K, C, count, rng):
    idx = []
    for k in (0, K - 1):
        for c in (0, C - 1):
            idx.extend(((k * C + c) * 9 + t) for t in range(9))
    idx.extend(rng.integers(0, K * C * 9, count).tolist())
    return np.unique(np.array(idx, dtype=np.int64))


def oracle_sampled(inp, gpu, seed=0, count=1500, with_bias=True):
    """Compare gpu outputs with the oracle on sampled elements; returns
    {name: (got, ref)} for y, dx, dw, db."""
    rng = np.random.default_rng(seed)
    x, w, g = inp["x"], inp["w"], inp["g"]
    b = inp["b"] if with_bias else None
    N, C, H, W = x.shape
    K = w.shape[0]
    res = {}
    i = _border_and_random((N, K, H, W), count, rng)
    res["y"] = (gpu["y"].ravel()[i], oracle.conv3x3_fwd_at(x, w, b, i))
    i = _border_and_random((N, C, H, W), count, rng)
    res["dx"] = (gpu["dx"].ravel()[i], oracle.conv3x3_bwd_data_at(g, w, i))
    i = _dw_indices(K, C, count // 4, rng)
    res["dw"] = (gpu["dw"].ravel()[i], oracle.conv3x3_bwd_weight_at(x, g, i))
    if gpu.get("db") is not None:
        i = np.arange(K) if K <= 512 else np.unique(rng.integers(0, K, 512))
        res["db"] = (gpu["db"][i], oracle.conv3x3_bias_grad_at(g, i))
    return res


def check(pairs_or_full, dtype, exact=False, label=""):
    """Assert the parity bar on every output; returns the errors."""
    errs = {}
    for name, (got, ref) in pairs_or_full.items():
        if exact:
            assert np.all(np.isfinite(got)), (label, name, "non-finite")
            bad = np.flatnonzero(np.asarray(got) != np.asarray(ref))
            assert bad.size == 0, (label, name, "integer-exact mismatch", bad[:10])
            errs[name] = 0.0
        else:
            e = rel_err(got, ref)
            errs[name] = e
            assert e <= TRIPWIRE[dtype], (label, name, e)
    return errs


def pairs(gpu, ref):
    return {k: (gpu[k], ref[k]) for k in ("y", "dx", "dw", "db") if ref.get(k) is not None}
