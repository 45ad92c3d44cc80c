"""Python binding of the gfx950 conv3x3 library (libconv3x3.so).

Argument marshalling only: every step of the convolution runs in the HIP
kernels behind the C ABI declared in ``include/conv3x3.h``; PyTorch supplies
device memory and the current stream.  The functions carry the C names:

    conv3x3_fwd(x, w, bias=None, out=None, out_dtype=None, split=True,
                workspace=None)                               -> y
    conv3x3_bwd_data(g, w, out=None, out_dtype=None, split=True,
                     workspace=None)                          -> dx
    conv3x3_workspace_size(pass_, N, C, K, H, W, dtype)       -> bytes
    conv3x3_bwd_weight(x, g, want_db=True, dw=None, db=None,
                       workspace=None)                        -> (dw, db)
    conv3x3_bwd_weight_workspace_size(N, C, K, H, W, dtype)   -> bytes
    conv3x3_bwd_weight_noalloc(x, g, dw, db=None)             -> (dw, db)
    conv3x3_fwd_act(x, w, bias=None, act=ACT_SILU, want_z=True,
                    out=None, z=None)                         -> (y, z)
    conv3x3_bwd_data_act(gy, z, w, act=ACT_SILU, out=None)    -> dx
    conv3x3_bwd_weight_act(x, gy, z, act=ACT_SILU, want_db=True,
                           dw=None, db=None, workspace=None)  -> (dw, db)
    conv3x3_fwd_cat(x0, x1, w, bias=None, out=None)           -> y
    conv3x3_bwd_data_cat(g, w, C0, out0=None, out1=None)      -> (dx0, dx1)
    conv3x3_bwd_weight_cat(x0, x1, g, want_db=True, dw=None, db=None,
                           workspace=None)                    -> (dw, db)
    conv3x3_bwd_weight_cat_workspace_size(N, C0, C1, K, H, W, dtype) -> bytes
    conv3x3_fwd_gnsilu(x, scale, shift, w, bias=None, out=None) -> y
    conv3x3_bwd_data_gnsilu(g, w, x, scale, shift, out=None)  -> du
    conv3x3_bwd_weight_gnsilu(x, scale, shift, g, want_db=True, dw=None,
                              db=None, workspace=None)        -> (dw, db)
    conv3x3_fwd_up2(x, w, bias=None, out=None)                -> y [N, K, 2H, 2W]
    conv3x3_bwd_data_up2(g, w, out=None, workspace=None)      -> dx [N, C, H, W]
    conv3x3_bwd_weight_up2(x, g, want_db=True, dw=None, db=None,
                           workspace=None)                    -> (dw, db)
    conv3x3_up2_workspace_size(pass_, N, C, K, H, W, dtype)   -> bytes
    conv3x3_fwd_s2(x, w, bias=None, out=None)                 -> y [N, K, H/2, W/2]
    conv3x3_bwd_data_s2(g, w, out=None)                       -> dx [N, C, 2h, 2w]
    conv3x3_bwd_weight_s2(x, g, want_db=True, dw=None, db=None,
                          workspace=None)                     -> (dw, db)
    conv3x3_status_string(code)                               -> str
    conv3x3_plan(pass_, N, C, K, H, W, dtype)                 -> dict
    conv3x3_plan_cat(pass_, N, C0, C1, K, H, W, dtype)        -> dict

The *_act functions fuse an activation (ACT_NONE, ACT_SILU, ACT_LRELU) into
the forward epilogue and, through z = the forward's pre-activation, into the
gradient loader of the backward passes (bfloat16: g = gy * act'(z) rounded
to bfloat16 as it is staged).  The *_cat
functions take the input as two tensors x0, x1 whose channel concatenation
[x0 ; x1] is the convolution's input (a UNet's up-path skip input) and never
form the concatenation; backward-data returns the two gradient halves.  The
*_gnsilu functions fuse a GroupNorm-apply + SiLU input prologue: the
convolution's input is SiLU(x * scale[n, c] + shift[n, c]) (scale, shift
float32 [N, C]); backward-data returns du, the gradient at
u = x * scale + shift (float32 only).

Tensors are NCHW / OIHW, contiguous, on a GPU; x, w, g are float32 or
bfloat16 (all three alike), bias is float32, outputs are float32 -- except
that with bfloat16 inputs y and dx may be written as bfloat16 (pass a
bfloat16 ``out`` or ``out_dtype=torch.bfloat16``; CONV3X3_BF16_IO).  There is
no fallback: if the library is missing, importing this package raises.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# CONV3X3_LIB selects another build of the same library (e.g. to compare two
# builds in one process); by default the in-tree one is loaded.
LIB_PATH = os.environ.get("CONV3X3_LIB") or os.path.join(_HERE, "libconv3x3.so")

CONV3X3_F32 = 0
CONV3X3_BF16 = 1
CONV3X3_BF16_IO = 2  # bf16 inputs, bf16 y / dx
PASS_FWD, PASS_BWD_DATA, PASS_BWD_WEIGHT = 0, 1, 2
ACT_NONE, ACT_SILU, ACT_LRELU = 0, 1, 2
STATUS = {
    "OK": 0, "ERR_NULL_POINTER": 1, "ERR_BAD_SHAPE": 2, "ERR_BAD_DTYPE": 3,
    "ERR_WORKSPACE": 4, "ERR_ALIAS": 5, "ERR_HIP": 6, "ERR_BAD_PASS": 7,
    "ERR_BAD_ACT": 8, "ERR_UNSUPPORTED": 9, "ERR_NOALLOC": 10,
}
EXPORTED = ["conv3x3_fwd", "conv3x3_bwd_data", "conv3x3_bwd_weight_workspace_size",
            "conv3x3_bwd_weight", "conv3x3_status_string", "conv3x3_plan",
            "conv3x3_fwd_act", "conv3x3_bwd_data_act", "conv3x3_bwd_weight_act",
            "conv3x3_fwd_cat", "conv3x3_bwd_data_cat", "conv3x3_bwd_weight_cat_workspace_size",
            "conv3x3_bwd_weight_cat", "conv3x3_plan_cat", "conv3x3_fwd_gnsilu",
            "conv3x3_bwd_data_gnsilu", "conv3x3_bwd_weight_gnsilu", "conv3x3_workspace_size",
            "conv3x3_fwd_ws", "conv3x3_bwd_data_ws", "conv3x3_up2_workspace_size",
            "conv3x3_fwd_up2", "conv3x3_bwd_data_up2", "conv3x3_bwd_weight_up2",
            "conv3x3_fwd_s2", "conv3x3_bwd_data_s2", "conv3x3_bwd_weight_s2",
            "conv3x3_bwd_weight_noalloc"]


class Plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "pass_", "dtype", "kernel", "tile_m", "tile_n", "tile_imgs", "tile_h", "tile_w",
        "chunk", "threads", "grid_x", "grid_y", "grid_z", "lds_bytes", "split")] + \
        [("workspace_bytes", ctypes.c_size_t)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first (python diffusion_unet_x3_amd/build.py "
            "or __graft_entry__.build()); there is no CPU fallback")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, fp = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p
    lib.conv3x3_fwd.argtypes = [vp, vp, fp, fp, i, i, i, i, i, i, vp]
    lib.conv3x3_fwd.restype = i
    lib.conv3x3_bwd_data.argtypes = [vp, vp, fp, i, i, i, i, i, i, vp]
    lib.conv3x3_bwd_data.restype = i
    lib.conv3x3_bwd_weight_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.conv3x3_bwd_weight_workspace_size.restype = ctypes.c_size_t
    lib.conv3x3_bwd_weight.argtypes = [vp, vp, fp, fp, vp, ctypes.c_size_t,
                                       i, i, i, i, i, i, vp]
    lib.conv3x3_bwd_weight.restype = i
    lib.conv3x3_fwd_act.argtypes = [vp, vp, fp, fp, fp, i, i, i, i, i, i, i, vp]
    lib.conv3x3_fwd_act.restype = i
    lib.conv3x3_bwd_data_act.argtypes = [vp, fp, vp, fp, i, i, i, i, i, i, i, vp]
    lib.conv3x3_bwd_data_act.restype = i
    lib.conv3x3_bwd_weight_act.argtypes = [vp, vp, fp, fp, fp, vp, ctypes.c_size_t,
                                           i, i, i, i, i, i, i, vp]
    lib.conv3x3_bwd_weight_act.restype = i
    lib.conv3x3_status_string.argtypes = [i]
    lib.conv3x3_status_string.restype = ctypes.c_char_p
    lib.conv3x3_plan.argtypes = [i, i, i, i, i, i, i, ctypes.POINTER(Plan)]
    lib.conv3x3_plan.restype = i
    lib.conv3x3_fwd_cat.argtypes = [vp, vp, i, i, vp, fp, fp, i, i, i, i, i, vp]
    lib.conv3x3_fwd_cat.restype = i
    lib.conv3x3_bwd_data_cat.argtypes = [vp, vp, fp, fp, i, i, i, i, i, i, i, vp]
    lib.conv3x3_bwd_data_cat.restype = i
    lib.conv3x3_bwd_weight_cat_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.conv3x3_bwd_weight_cat_workspace_size.restype = ctypes.c_size_t
    lib.conv3x3_bwd_weight_cat.argtypes = [vp, vp, i, i, vp, fp, fp, vp, ctypes.c_size_t,
                                           i, i, i, i, i, vp]
    lib.conv3x3_bwd_weight_cat.restype = i
    lib.conv3x3_plan_cat.argtypes = [i, i, i, i, i, i, i, i, ctypes.POINTER(Plan)]
    lib.conv3x3_plan_cat.restype = i
    lib.conv3x3_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.conv3x3_workspace_size.restype = ctypes.c_size_t
    lib.conv3x3_fwd_ws.argtypes = [vp, vp, fp, fp, vp, ctypes.c_size_t, i, i, i, i, i, i, vp]
    lib.conv3x3_fwd_ws.restype = i
    lib.conv3x3_bwd_data_ws.argtypes = [vp, vp, fp, vp, ctypes.c_size_t, i, i, i, i, i, i, vp]
    lib.conv3x3_bwd_data_ws.restype = i
    lib.conv3x3_up2_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.conv3x3_up2_workspace_size.restype = ctypes.c_size_t
    lib.conv3x3_fwd_up2.argtypes = [vp, vp, fp, fp, i, i, i, i, i, i, vp]
    lib.conv3x3_fwd_up2.restype = i
    lib.conv3x3_bwd_data_up2.argtypes = [vp, vp, fp, vp, ctypes.c_size_t, i, i, i, i, i, i, vp]
    lib.conv3x3_bwd_data_up2.restype = i
    lib.conv3x3_bwd_weight_up2.argtypes = [vp, vp, fp, fp, vp, ctypes.c_size_t,
                                           i, i, i, i, i, i, vp]
    lib.conv3x3_bwd_weight_up2.restype = i
    lib.conv3x3_fwd_s2.argtypes = [vp, vp, fp, fp, i, i, i, i, i, i, vp]
    lib.conv3x3_fwd_s2.restype = i
    lib.conv3x3_bwd_data_s2.argtypes = [vp, vp, fp, i, i, i, i, i, i, vp]
    lib.conv3x3_bwd_data_s2.restype = i
    lib.conv3x3_bwd_weight_s2.argtypes = [vp, vp, fp, fp, vp, ctypes.c_size_t, i, i, i, i, i, i, vp]
    lib.conv3x3_bwd_weight_s2.restype = i
    lib.conv3x3_fwd_gnsilu.argtypes = [vp, fp, fp, vp, fp, fp, i, i, i, i, i, i, vp]
    lib.conv3x3_fwd_gnsilu.restype = i
    lib.conv3x3_bwd_data_gnsilu.argtypes = [vp, vp, vp, fp, fp, fp, i, i, i, i, i, i, vp]
    lib.conv3x3_bwd_data_gnsilu.restype = i
    lib.conv3x3_bwd_weight_gnsilu.argtypes = [vp, fp, fp, vp, fp, fp, vp, ctypes.c_size_t,
                                              i, i, i, i, i, i, vp]
    lib.conv3x3_bwd_weight_gnsilu.restype = i
    lib.conv3x3_bwd_weight_noalloc.argtypes = [vp, vp, fp, fp, i, i, i, i, i, i, vp]
    lib.conv3x3_bwd_weight_noalloc.restype = i
    return lib


lib = _load()


def conv3x3_status_string(code):
    return lib.conv3x3_status_string(int(code)).decode()


def _raise(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what}: {conv3x3_status_string(rc)} (status {rc})")


def _dtype_code(t):
    if t.dtype == torch.float32:
        return CONV3X3_F32
    if t.dtype == torch.bfloat16:
        return CONV3X3_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _check(t, name, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor")


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _act_out(out, shape, like, name, out_dtype):
    """The activation-shaped output (y or dx) and the dtype code of the call:
    bfloat16 inputs may write it as bfloat16 (out given as a bfloat16 tensor,
    or out_dtype=torch.bfloat16), everything else writes float32."""
    want = out.dtype if out is not None else (out_dtype or torch.float32)
    if want == torch.bfloat16:
        if like.dtype != torch.bfloat16:
            raise ValueError("bfloat16 outputs need bfloat16 inputs")
        if out is None:
            out = torch.empty(shape, dtype=torch.bfloat16, device=like.device)
        _check(out, name, len(shape))
        if tuple(out.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}")
        return out, CONV3X3_BF16_IO
    return _f32_out(out, shape, like, name), _dtype_code(like)


def _f32_out(out, shape, like, name):
    if out is None:
        return torch.empty(shape, dtype=torch.float32, device=like.device)
    _check(out, name, len(shape))
    if out.dtype != torch.float32 or tuple(out.shape) != tuple(shape):
        raise ValueError(f"{name} must be float32 of shape {tuple(shape)}")
    return out


def conv3x3_workspace_size(pass_, N, C, K, H, W, dtype=CONV3X3_F32):
    n = lib.conv3x3_workspace_size(pass_, N, C, K, H, W, dtype)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid problem for conv3x3_workspace_size")
    return n


def _workspace(need, workspace, like):
    """(pointer, bytes) of a workspace of at least `need` bytes: the given
    one, or a new torch allocation."""
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=like.device)
    if workspace is None:
        return None, 0
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def conv3x3_fwd(x, w, bias=None, out=None, out_dtype=None, split=True, workspace=None):
    """y = conv3x3(x; w) + bias (stride 1, zero padding 1); float32 output, or
    bfloat16 for bfloat16 inputs with a bfloat16 out / out_dtype.  split:
    run through conv3x3_fwd_ws, which may split a small-image
    reduction (the workspace is allocated unless given)."""
    _check(x, "x", 4)
    _check(w, "w", 4)
    N, C, H, W = x.shape
    K = w.shape[0]
    if tuple(w.shape) != (K, C, 3, 3) or w.dtype != x.dtype:
        raise ValueError("w must be [K, C, 3, 3] with x's dtype")
    if bias is not None:
        _check(bias, "bias", 1)
        if bias.dtype != torch.float32 or bias.shape[0] != K:
            raise ValueError("bias must be float32 [K]")
    y, code = _act_out(out, (N, K, H, W), x, "out", out_dtype)
    b = None if bias is None else bias.data_ptr()
    if split:
        ws, nb = _workspace(conv3x3_workspace_size(PASS_FWD, N, C, K, H, W, code), workspace, x)
        rc = lib.conv3x3_fwd_ws(x.data_ptr(), w.data_ptr(), b, y.data_ptr(), ws, nb,
                                N, C, K, H, W, code, _stream(x))
        _raise(rc, "conv3x3_fwd_ws")
    else:
        rc = lib.conv3x3_fwd(x.data_ptr(), w.data_ptr(), b, y.data_ptr(),
                             N, C, K, H, W, code, _stream(x))
        _raise(rc, "conv3x3_fwd")
    return y


def conv3x3_bwd_data(g, w, out=None, out_dtype=None, split=True, workspace=None):
    """dx = d<conv3x3(x; w), g>/dx; float32 output, or bfloat16 as
    conv3x3_fwd; split / workspace as conv3x3_fwd."""
    _check(g, "g", 4)
    _check(w, "w", 4)
    N, K, H, W = g.shape
    C = w.shape[1]
    if tuple(w.shape) != (K, C, 3, 3) or w.dtype != g.dtype:
        raise ValueError("w must be [K, C, 3, 3] with g's dtype")
    dx, code = _act_out(out, (N, C, H, W), g, "out", out_dtype)
    if split:
        ws, nb = _workspace(conv3x3_workspace_size(PASS_BWD_DATA, N, C, K, H, W, code),
                            workspace, g)
        rc = lib.conv3x3_bwd_data_ws(g.data_ptr(), w.data_ptr(), dx.data_ptr(), ws, nb,
                                     N, C, K, H, W, code, _stream(g))
        _raise(rc, "conv3x3_bwd_data_ws")
    else:
        rc = lib.conv3x3_bwd_data(g.data_ptr(), w.data_ptr(), dx.data_ptr(),
                                  N, C, K, H, W, code, _stream(g))
        _raise(rc, "conv3x3_bwd_data")
    return dx


def conv3x3_bwd_weight_workspace_size(N, C, K, H, W, dtype=CONV3X3_F32):
    n = lib.conv3x3_bwd_weight_workspace_size(N, C, K, H, W, dtype)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid problem for conv3x3_bwd_weight_workspace_size")
    return n


def conv3x3_bwd_weight(x, g, want_db=True, dw=None, db=None, workspace=None):
    """(dw, db) = gradients of <conv3x3(x; w) + b, g> w.r.t. w and b, float32."""
    _check(x, "x", 4)
    _check(g, "g", 4)
    N, C, H, W = x.shape
    K = g.shape[1]
    if tuple(g.shape) != (N, K, H, W) or g.dtype != x.dtype:
        raise ValueError("g must be [N, K, H, W] with x's dtype")
    code = _dtype_code(x)
    dw = _f32_out(dw, (K, C, 3, 3), x, "dw")
    if want_db:
        db = _f32_out(db, (K,), x, "db")
    else:
        db = None
    need = conv3x3_bwd_weight_workspace_size(N, C, K, H, W, code)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.conv3x3_bwd_weight(x.data_ptr(), g.data_ptr(), dw.data_ptr(),
                                None if db is None else db.data_ptr(), ws_ptr, ws_bytes,
                                N, C, K, H, W, code, _stream(x))
    _raise(rc, "conv3x3_bwd_weight")
    return dw, db


def conv3x3_bwd_weight_noalloc(x, g, dw, db=None):
    """conv3x3_bwd_weight with the split-K partial sums in the library's own
    device array instead of a workspace: the call allocates nothing (dw and
    the optional db are given).  Calls that overlap on one GPU race."""
    _check(x, "x", 4)
    _check(g, "g", 4)
    N, C, H, W = x.shape
    K = g.shape[1]
    if tuple(g.shape) != (N, K, H, W) or g.dtype != x.dtype:
        raise ValueError("g must be [N, K, H, W] with x's dtype")
    dw = _f32_out(dw, (K, C, 3, 3), x, "dw")
    if db is not None:
        db = _f32_out(db, (K,), x, "db")
    rc = lib.conv3x3_bwd_weight_noalloc(x.data_ptr(), g.data_ptr(), dw.data_ptr(),
                                        None if db is None else db.data_ptr(),
                                        N, C, K, H, W, _dtype_code(x), _stream(x))
    _raise(rc, "conv3x3_bwd_weight_noalloc")
    return dw, db


def conv3x3_fwd_act(x, w, bias=None, act=ACT_SILU, want_z=True, out=None, z=None,
                    out_dtype=None):
    """(y, z): z = conv3x3(x; w) + bias, y = act(z), both float32 (z None
    unless want_z)."""
    _check(x, "x", 4)
    _check(w, "w", 4)
    N, C, H, W = x.shape
    K = w.shape[0]
    if tuple(w.shape) != (K, C, 3, 3) or w.dtype != x.dtype:
        raise ValueError("w must be [K, C, 3, 3] with x's dtype")
    if bias is not None:
        _check(bias, "bias", 1)
        if bias.dtype != torch.float32 or bias.shape[0] != K:
            raise ValueError("bias must be float32 [K]")
    y, code = _act_out(out, (N, K, H, W), x, "out", out_dtype)
    z = _f32_out(z, (N, K, H, W), x, "z") if want_z else None
    rc = lib.conv3x3_fwd_act(x.data_ptr(), w.data_ptr(),
                             None if bias is None else bias.data_ptr(), y.data_ptr(),
                             None if z is None else z.data_ptr(),
                             N, C, K, H, W, code, int(act), _stream(x))
    _raise(rc, "conv3x3_fwd_act")
    return y, z


def _check_z(z, shape):
    _check(z, "z", 4)
    if z.dtype != torch.float32 or tuple(z.shape) != tuple(shape):
        raise ValueError(f"z must be float32 of shape {tuple(shape)}")


def conv3x3_bwd_data_act(gy, z, w, act=ACT_SILU, out=None):
    """dx of <act(conv3x3(x; w) + b), gy>, given z = conv3x3(x; w) + b."""
    _check(gy, "gy", 4)
    _check(w, "w", 4)
    N, K, H, W = gy.shape
    C = w.shape[1]
    if tuple(w.shape) != (K, C, 3, 3) or w.dtype != gy.dtype:
        raise ValueError("w must be [K, C, 3, 3] with gy's dtype")
    if z is not None:
        _check_z(z, (N, K, H, W))
    dx = _f32_out(out, (N, C, H, W), gy, "out")
    rc = lib.conv3x3_bwd_data_act(gy.data_ptr(), None if z is None else z.data_ptr(),
                                  w.data_ptr(), dx.data_ptr(), N, C, K, H, W, _dtype_code(gy),
                                  int(act), _stream(gy))
    _raise(rc, "conv3x3_bwd_data_act")
    return dx


def conv3x3_bwd_weight_act(x, gy, z, act=ACT_SILU, want_db=True, dw=None, db=None,
                           workspace=None):
    """(dw, db) of <act(conv3x3(x; w) + b), gy>, given z = conv3x3(x; w) + b."""
    _check(x, "x", 4)
    _check(gy, "gy", 4)
    N, C, H, W = x.shape
    K = gy.shape[1]
    if tuple(gy.shape) != (N, K, H, W) or gy.dtype != x.dtype:
        raise ValueError("gy must be [N, K, H, W] with x's dtype")
    if z is not None:
        _check_z(z, (N, K, H, W))
    code = _dtype_code(x)
    dw = _f32_out(dw, (K, C, 3, 3), x, "dw")
    db = _f32_out(db, (K,), x, "db") if want_db else None
    need = conv3x3_bwd_weight_workspace_size(N, C, K, H, W, code)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.conv3x3_bwd_weight_act(x.data_ptr(), gy.data_ptr(),
                                    None if z is None else z.data_ptr(), dw.data_ptr(),
                                    None if db is None else db.data_ptr(), ws_ptr, ws_bytes,
                                    N, C, K, H, W, code, int(act), _stream(x))
    _raise(rc, "conv3x3_bwd_weight_act")
    return dw, db


def conv3x3_plan(pass_, N, C, K, H, W, dtype=CONV3X3_F32):
    """The launch plan the library uses for one pass (host-side query)."""
    p = Plan()
    rc = lib.conv3x3_plan(pass_, N, C, K, H, W, dtype, ctypes.byref(p))
    _raise(rc, "conv3x3_plan")
    return {name: getattr(p, name) for name, _ in Plan._fields_}


def _halves(x0, x1):
    _check(x0, "x0", 4)
    _check(x1, "x1", 4)
    N, C0, H, W = x0.shape
    if (x1.shape[0], x1.shape[2], x1.shape[3]) != (N, H, W) or x1.dtype != x0.dtype:
        raise ValueError("x1 must be [N, C1, H, W] with x0's N, H, W and dtype")
    return N, C0, x1.shape[1], H, W


def _ptr(t):
    """Device address of t, or None for a tensor with no elements."""
    return t.data_ptr() if t.numel() else None


def conv3x3_fwd_cat(x0, x1, w, bias=None, out=None, out_dtype=None):
    """y = conv3x3([x0 ; x1]; w) + bias, the input being the channel
    concatenation of x0 and x1 (never formed)."""
    N, C0, C1, H, W = _halves(x0, x1)
    _check(w, "w", 4)
    K = w.shape[0]
    if tuple(w.shape) != (K, C0 + C1, 3, 3) or w.dtype != x0.dtype:
        raise ValueError("w must be [K, C0 + C1, 3, 3] with x0's dtype")
    if bias is not None:
        _check(bias, "bias", 1)
        if bias.dtype != torch.float32 or bias.shape[0] != K:
            raise ValueError("bias must be float32 [K]")
    y, code = _act_out(out, (N, K, H, W), x0, "out", out_dtype)
    rc = lib.conv3x3_fwd_cat(_ptr(x0), _ptr(x1), C0, C1, w.data_ptr(),
                             None if bias is None else bias.data_ptr(), y.data_ptr(),
                             N, K, H, W, code, _stream(w))
    _raise(rc, "conv3x3_fwd_cat")
    return y


def conv3x3_bwd_data_cat(g, w, C0, out0=None, out1=None, out_dtype=None):
    """(dx0, dx1): the input gradient of conv3x3([x0 ; x1]; w) split at
    channel C0, float32."""
    _check(g, "g", 4)
    _check(w, "w", 4)
    N, K, H, W = g.shape
    C = w.shape[1]
    if tuple(w.shape) != (K, C, 3, 3) or w.dtype != g.dtype:
        raise ValueError("w must be [K, C, 3, 3] with g's dtype")
    if not 0 <= C0 <= C:
        raise ValueError("C0 must lie in [0, C]")
    dx0, code = _act_out(out0, (N, C0, H, W), g, "out0", out_dtype)
    dx1, code1 = _act_out(out1, (N, C - C0, H, W), g, "out1", out_dtype or dx0.dtype)
    if code1 != code:
        raise ValueError("out0 and out1 must have the same dtype")
    rc = lib.conv3x3_bwd_data_cat(g.data_ptr(), w.data_ptr(), _ptr(dx0), _ptr(dx1), C0, C - C0,
                                  N, K, H, W, code, _stream(g))
    _raise(rc, "conv3x3_bwd_data_cat")
    return dx0, dx1


def conv3x3_bwd_weight_cat_workspace_size(N, C0, C1, K, H, W, dtype=CONV3X3_F32):
    n = lib.conv3x3_bwd_weight_cat_workspace_size(N, C0, C1, K, H, W, dtype)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid problem for conv3x3_bwd_weight_cat_workspace_size")
    return n


def conv3x3_bwd_weight_cat(x0, x1, g, want_db=True, dw=None, db=None, workspace=None):
    """(dw, db) of <conv3x3([x0 ; x1]; w) + b, g>, float32."""
    N, C0, C1, H, W = _halves(x0, x1)
    _check(g, "g", 4)
    K = g.shape[1]
    if tuple(g.shape) != (N, K, H, W) or g.dtype != x0.dtype:
        raise ValueError("g must be [N, K, H, W] with x0's dtype")
    code = _dtype_code(x0)
    dw = _f32_out(dw, (K, C0 + C1, 3, 3), g, "dw")
    db = _f32_out(db, (K,), g, "db") if want_db else None
    need = conv3x3_bwd_weight_cat_workspace_size(N, C0, C1, K, H, W, code)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=g.device)
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.conv3x3_bwd_weight_cat(_ptr(x0), _ptr(x1), C0, C1, g.data_ptr(), dw.data_ptr(),
                                    None if db is None else db.data_ptr(), ws_ptr, ws_bytes,
                                    N, K, H, W, code, _stream(g))
    _raise(rc, "conv3x3_bwd_weight_cat")
    return dw, db


def conv3x3_plan_cat(pass_, N, C0, C1, K, H, W, dtype=CONV3X3_F32):
    """The launch plan of a *_cat call (host-side query)."""
    p = Plan()
    rc = lib.conv3x3_plan_cat(pass_, N, C0, C1, K, H, W, dtype, ctypes.byref(p))
    _raise(rc, "conv3x3_plan_cat")
    return {name: getattr(p, name) for name, _ in Plan._fields_}


def _check_affine(scale, shift, N, C):
    for t, name in ((scale, "scale"), (shift, "shift")):
        _check(t, name, 2)
        if t.dtype != torch.float32 or tuple(t.shape) != (N, C):
            raise ValueError(f"{name} must be float32 [N, C] = [{N}, {C}]")


def conv3x3_fwd_gnsilu(x, scale, shift, w, bias=None, out=None):
    """y = conv3x3(SiLU(x * scale + shift); w) + bias, float32."""
    _check(x, "x", 4)
    _check(w, "w", 4)
    N, C, H, W = x.shape
    K = w.shape[0]
    _check_affine(scale, shift, N, C)
    if tuple(w.shape) != (K, C, 3, 3) or w.dtype != x.dtype:
        raise ValueError("w must be [K, C, 3, 3] with x's dtype")
    if bias is not None:
        _check(bias, "bias", 1)
        if bias.dtype != torch.float32 or bias.shape[0] != K:
            raise ValueError("bias must be float32 [K]")
    y = _f32_out(out, (N, K, H, W), x, "out")
    rc = lib.conv3x3_fwd_gnsilu(x.data_ptr(), scale.data_ptr(), shift.data_ptr(), w.data_ptr(),
                                None if bias is None else bias.data_ptr(), y.data_ptr(),
                                N, C, K, H, W, _dtype_code(x), _stream(x))
    _raise(rc, "conv3x3_fwd_gnsilu")
    return y


def conv3x3_bwd_data_gnsilu(g, w, x, scale, shift, out=None):
    """du = conv3x3_bwd_data(g, w) * SiLU'(x * scale + shift), float32."""
    _check(g, "g", 4)
    _check(w, "w", 4)
    _check(x, "x", 4)
    N, K, H, W = g.shape
    C = w.shape[1]
    if tuple(w.shape) != (K, C, 3, 3) or w.dtype != g.dtype:
        raise ValueError("w must be [K, C, 3, 3] with g's dtype")
    if tuple(x.shape) != (N, C, H, W) or x.dtype != g.dtype:
        raise ValueError("x must be [N, C, H, W] with g's dtype")
    _check_affine(scale, shift, N, C)
    du = _f32_out(out, (N, C, H, W), g, "out")
    rc = lib.conv3x3_bwd_data_gnsilu(g.data_ptr(), w.data_ptr(), x.data_ptr(), scale.data_ptr(),
                                     shift.data_ptr(), du.data_ptr(), N, C, K, H, W,
                                     _dtype_code(g), _stream(g))
    _raise(rc, "conv3x3_bwd_data_gnsilu")
    return du


def conv3x3_bwd_weight_gnsilu(x, scale, shift, g, want_db=True, dw=None, db=None,
                              workspace=None):
    """(dw, db) of <conv3x3(SiLU(x * scale + shift); w) + b, g>, float32."""
    _check(x, "x", 4)
    _check(g, "g", 4)
    N, C, H, W = x.shape
    K = g.shape[1]
    if tuple(g.shape) != (N, K, H, W) or g.dtype != x.dtype:
        raise ValueError("g must be [N, K, H, W] with x's dtype")
    _check_affine(scale, shift, N, C)
    code = _dtype_code(x)
    dw = _f32_out(dw, (K, C, 3, 3), x, "dw")
    db = _f32_out(db, (K,), x, "db") if want_db else None
    need = conv3x3_bwd_weight_workspace_size(N, C, K, H, W, code)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.conv3x3_bwd_weight_gnsilu(x.data_ptr(), scale.data_ptr(), shift.data_ptr(),
                                       g.data_ptr(), dw.data_ptr(),
                                       None if db is None else db.data_ptr(), ws_ptr, ws_bytes,
                                       N, C, K, H, W, code, _stream(x))
    _raise(rc, "conv3x3_bwd_weight_gnsilu")
    return dw, db


def conv3x3_up2_workspace_size(pass_, N, C, K, H, W, dtype=CONV3X3_F32):
    n = lib.conv3x3_up2_workspace_size(pass_, N, C, K, H, W, dtype)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid problem for conv3x3_up2_workspace_size")
    return n


def conv3x3_fwd_up2(x, w, bias=None, out=None):
    """y = conv3x3(nearest_upsample_2x(x); w) + bias, y [N, K, 2H, 2W]."""
    _check(x, "x", 4)
    _check(w, "w", 4)
    N, C, H, W = x.shape
    K = w.shape[0]
    if tuple(w.shape) != (K, C, 3, 3) or w.dtype != x.dtype:
        raise ValueError("w must be [K, C, 3, 3] with x's dtype")
    if bias is not None:
        _check(bias, "bias", 1)
        if bias.dtype != torch.float32 or bias.shape[0] != K:
            raise ValueError("bias must be float32 [K]")
    y = _f32_out(out, (N, K, 2 * H, 2 * W), x, "out")
    rc = lib.conv3x3_fwd_up2(x.data_ptr(), w.data_ptr(),
                             None if bias is None else bias.data_ptr(), y.data_ptr(),
                             N, C, K, H, W, _dtype_code(x), _stream(x))
    _raise(rc, "conv3x3_fwd_up2")
    return y


def conv3x3_bwd_data_up2(g, w, out=None, workspace=None):
    """dx [N, C, H, W] of <conv3x3(nearest_upsample_2x(x); w), g>, g being
    [N, K, 2H, 2W]."""
    _check(g, "g", 4)
    _check(w, "w", 4)
    N, K, H2, W2 = g.shape
    if H2 % 2 or W2 % 2:
        raise ValueError("g must have even height and width")
    H, W = H2 // 2, W2 // 2
    C = w.shape[1]
    if tuple(w.shape) != (K, C, 3, 3) or w.dtype != g.dtype:
        raise ValueError("w must be [K, C, 3, 3] with g's dtype")
    code = _dtype_code(g)
    dx = _f32_out(out, (N, C, H, W), g, "out")
    ws, nb = _workspace(conv3x3_up2_workspace_size(PASS_BWD_DATA, N, C, K, H, W, code),
                        workspace, g)
    rc = lib.conv3x3_bwd_data_up2(g.data_ptr(), w.data_ptr(), dx.data_ptr(), ws, nb,
                                  N, C, K, H, W, code, _stream(g))
    _raise(rc, "conv3x3_bwd_data_up2")
    return dx


def conv3x3_bwd_weight_up2(x, g, want_db=True, dw=None, db=None, workspace=None):
    """(dw, db) of <conv3x3(nearest_upsample_2x(x); w) + b, g>."""
    _check(x, "x", 4)
    _check(g, "g", 4)
    N, C, H, W = x.shape
    K = g.shape[1]
    if tuple(g.shape) != (N, K, 2 * H, 2 * W) or g.dtype != x.dtype:
        raise ValueError("g must be [N, K, 2H, 2W] with x's dtype")
    code = _dtype_code(x)
    dw = _f32_out(dw, (K, C, 3, 3), x, "dw")
    db = _f32_out(db, (K,), x, "db") if want_db else None
    ws, nb = _workspace(conv3x3_up2_workspace_size(PASS_BWD_WEIGHT, N, C, K, H, W, code),
                        workspace, x)
    rc = lib.conv3x3_bwd_weight_up2(x.data_ptr(), g.data_ptr(), dw.data_ptr(),
                                    None if db is None else db.data_ptr(), ws, nb,
                                    N, C, K, H, W, code, _stream(x))
    _raise(rc, "conv3x3_bwd_weight_up2")
    return dw, db


def conv3x3_fwd_s2(x, w, bias=None, out=None):
    """Stride-2 3x3 convolution (padding 1) of x [N, C, H, W] (H, W even):
    y [N, K, H/2, W/2]."""
    _check(x, "x", 4)
    _check(w, "w", 4)
    N, C, H, W = x.shape
    K = w.shape[0]
    if tuple(w.shape) != (K, C, 3, 3) or w.dtype != x.dtype:
        raise ValueError("w must be [K, C, 3, 3] with x's dtype")
    if bias is not None:
        _check(bias, "bias", 1)
        if bias.dtype != torch.float32 or bias.shape[0] != K:
            raise ValueError("bias must be float32 [K]")
    y = _f32_out(out, (N, K, H // 2, W // 2), x, "out")
    rc = lib.conv3x3_fwd_s2(x.data_ptr(), w.data_ptr(),
                            None if bias is None else bias.data_ptr(), y.data_ptr(),
                            N, C, K, H, W, _dtype_code(x), _stream(x))
    _raise(rc, "conv3x3_fwd_s2")
    return y


def conv3x3_bwd_data_s2(g, w, out=None):
    """dx [N, C, 2h, 2w] of <conv_s2(x; w), g> for g [N, K, h, w]."""
    _check(g, "g", 4)
    _check(w, "w", 4)
    N, K, h, wd = g.shape
    C = w.shape[1]
    if tuple(w.shape) != (K, C, 3, 3) or w.dtype != g.dtype:
        raise ValueError("w must be [K, C, 3, 3] with g's dtype")
    dx = _f32_out(out, (N, C, 2 * h, 2 * wd), g, "out")
    rc = lib.conv3x3_bwd_data_s2(g.data_ptr(), w.data_ptr(), dx.data_ptr(),
                                 N, C, K, 2 * h, 2 * wd, _dtype_code(g), _stream(g))
    _raise(rc, "conv3x3_bwd_data_s2")
    return dx


def conv3x3_bwd_weight_s2(x, g, want_db=True, dw=None, db=None, workspace=None):
    """(dw, db) of <conv_s2(x; w) + b, g>, x [N, C, H, W], g [N, K, H/2, W/2]."""
    _check(x, "x", 4)
    _check(g, "g", 4)
    N, C, H, W = x.shape
    K = g.shape[1]
    if tuple(g.shape) != (N, K, H // 2, W // 2) or g.dtype != x.dtype:
        raise ValueError("g must be [N, K, H/2, W/2] with x's dtype")
    code = _dtype_code(x)
    dw = _f32_out(dw, (K, C, 3, 3), x, "dw")
    db = _f32_out(db, (K,), x, "db") if want_db else None
    ws, nb = _workspace(conv3x3_bwd_weight_workspace_size(N, C, K, H, W, code), workspace, x)
    rc = lib.conv3x3_bwd_weight_s2(x.data_ptr(), g.data_ptr(), dw.data_ptr(),
                                   None if db is None else db.data_ptr(), ws, nb,
                                   N, C, K, H, W, code, _stream(x))
    _raise(rc, "conv3x3_bwd_weight_s2")
    return dw, db
