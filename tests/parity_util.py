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


def _cdiv(a, b):
    return -(-a // b)


def tile_strata(shape, plan, rng):
    """Flat indices into an output [N, Co, H, W] (y of the forward, dx of
    backward-data): one random element in every (pixel tile of the plan,
    32-channel group) -- so every workgroup's tile and every wave's 32-row
    block within it has a compared element.  (A split reduction adds every
    slice into every element of its tile, so the slices are covered too.)"""
    N, Co, H, W = shape
    ti, th, tw = plan["tile_imgs"], plan["tile_h"], plan["tile_w"]
    nb, hb, wb, cb = np.meshgrid(np.arange(_cdiv(N, ti)), np.arange(_cdiv(H, th)),
                                 np.arange(_cdiv(W, tw)), np.arange(_cdiv(Co, 32)),
                                 indexing="ij")
    nb, hb, wb, cb = (a.ravel() for a in (nb, hb, wb, cb))

    def pick(block, size, extent):
        lo = block * size
        return lo + (rng.random(lo.shape) * np.minimum(size, extent - lo)).astype(np.int64)

    n, h, w, c = pick(nb, ti, N), pick(hb, th, H), pick(wb, tw, W), pick(cb, 32, Co)
    return ((n * Co + c) * H + h) * W + w


def dw_strata(K, C, rng):
    """Flat indices into dw [K, C, 3, 3]: one random element in every
    (32-k block, 32-c block, tap) -- every wave's accumulator block of every
    backward-weight tile."""
    kb, cb, t = np.meshgrid(np.arange(_cdiv(K, 32)), np.arange(_cdiv(C, 32)), np.arange(9),
                            indexing="ij")
    kb, cb, t = kb.ravel(), cb.ravel(), t.ravel()
    k = kb * 32 + (rng.random(kb.shape) * np.minimum(32, K - kb * 32)).astype(np.int64)
    c = cb * 32 + (rng.random(cb.shape) * np.minimum(32, C - cb * 32)).astype(np.int64)
    return (k * C + c) * 9 + t


def stratified_indices(N, C, K, H, W, dtype, count, rng):
    """The compared elements of y, dx and dw: the borders, `count` random
    elements, and the strata of the launch plans the library uses."""
    import diffusion_unet_x3_amd as lib3
    code = lib3.CONV3X3_BF16 if dtype == "bf16" else lib3.CONV3X3_F32
    pf = lib3.conv3x3_plan(lib3.PASS_FWD, N, C, K, H, W, code)
    pd = lib3.conv3x3_plan(lib3.PASS_BWD_DATA, N, C, K, H, W, code)
    iy = np.unique(np.concatenate([_border_and_random((N, K, H, W), count, rng),
                                   tile_strata((N, K, H, W), pf, rng)]))
    idx = np.unique(np.concatenate([_border_and_random((N, C, H, W), count, rng),
                                    tile_strata((N, C, H, W), pd, rng)]))
    iw = np.unique(np.concatenate([_dw_indices(K, C, count // 4, rng), dw_strata(K, C, rng)]))
    return iy, idx, iw


def oracle_sampled(inp, gpu, seed=0, count=1500, with_bias=True):
    """Compare gpu outputs with the oracle on sampled elements (every tile of
    the launch plans, the borders and random elements); returns
    {name: (got, ref)} for y, dx, dw, db."""
    rng = np.random.default_rng(seed)
    x, w, g = inp["x"], inp["w"], inp["g"]
    b = inp["b"] if with_bias else None
    N, C, H, W = x.shape
    K = w.shape[0]
    dtype = "bf16" if x.dtype == torch.bfloat16 else "f32"
    iy, idx, iw = stratified_indices(N, C, K, H, W, dtype, count, rng)
    res = {}
    res["y"] = (gpu["y"].ravel()[iy], oracle.conv3x3_fwd_at(x, w, b, iy))
    res["dx"] = (gpu["dx"].ravel()[idx], oracle.conv3x3_bwd_data_at(g, w, idx))
    res["dw"] = (gpu["dw"].ravel()[iw], oracle.conv3x3_bwd_weight_at(x, g, iw))
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
