"""fp64 CPU oracle for the 3x3 convolution -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It loads ``liboracle_conv3x3.so``
(plain C, built from ``conv3x3_oracle.c`` by ``build.sh``) and shares nothing
with the HIP library.  The C file's header states the definition it follows
(PyTorch Conv2d semantics, read from the sourcepulse summary of the C++/CUDA
UNet project, sections "How It Works", "Quick Start & Requirements" and
"Highlighted Details") and the pins that check it.

All functions take numpy arrays or CPU torch tensors (any real dtype; they are
widened to float64, which is exact for float32 and bfloat16 values) and return
float64 numpy arrays.

The fused-activation functions (``act_*``, ``conv3x3_fwd_act``,
``conv3x3_bwd_act``) follow the reading in the C file's "fused activation"
section: activation 0 = identity, 1 = SiLU, 2 = leaky ReLU (slope 0.2) on the
biased convolution output z; the backward takes the gradient at the
activation's output and multiplies it by act'(z).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# CONV3X3_ORACLE_LIB lets the pin suite run against a deliberately broken
# build (tests/test_oracle_mutants.py); normal use never sets it.
LIB_PATH = os.environ.get("CONV3X3_ORACLE_LIB") or os.path.join(_HERE, "liboracle_conv3x3.so")

ACT_NONE, ACT_SILU, ACT_LRELU = 0, 1, 2

_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.POINTER(ctypes.c_int64)
_i = ctypes.c_int
_n = ctypes.c_int64


def build():
    """Compile the oracle with gcc."""
    subprocess.check_call(["sh", os.path.join(_HERE, "build.sh")])


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor: widen through float32 (exact for bf16)
        a = a.detach().cpu().float().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _idx(idx):
    return np.ascontiguousarray(np.asarray(idx, dtype=np.int64).ravel())


def _p(a):
    return None if a is None else a.ctypes.data_as(_D)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (code {rc})")


class Oracle:
    """One loaded build of the oracle library (the default one, or a test build)."""

    def __init__(self, path=LIB_PATH):
        lib = ctypes.CDLL(path)
        lib.oracle_conv3x3_fwd.argtypes = [_D, _D, _D, _D, _i, _i, _i, _i, _i]
        lib.oracle_conv3x3_bwd_data.argtypes = [_D, _D, _D, _i, _i, _i, _i, _i]
        lib.oracle_conv3x3_bwd_weight.argtypes = [_D, _D, _D, _D, _i, _i, _i, _i, _i]
        lib.oracle_conv3x3_fwd_at.argtypes = [_D, _D, _D, _i, _i, _i, _i, _i, _I64, _n, _D]
        lib.oracle_conv3x3_bwd_data_at.argtypes = [_D, _D, _i, _i, _i, _i, _i, _I64, _n, _D]
        lib.oracle_conv3x3_bwd_weight_at.argtypes = [_D, _D, _i, _i, _i, _i, _i, _I64, _n, _D]
        lib.oracle_conv3x3_bias_grad_at.argtypes = [_D, _i, _i, _i, _i, _I64, _n, _D]
        lib.oracle_act_forward.argtypes = [_D, _D, _n, _i]
        lib.oracle_act_grad.argtypes = [_D, _D, _D, _n, _i]
        for f in ("oracle_conv3x3_fwd", "oracle_conv3x3_bwd_data",
                  "oracle_conv3x3_bwd_weight", "oracle_conv3x3_fwd_at",
                  "oracle_conv3x3_bwd_data_at", "oracle_conv3x3_bwd_weight_at",
                  "oracle_conv3x3_bias_grad_at", "oracle_act_forward", "oracle_act_grad",
                  "oracle_num_threads"):
            getattr(lib, f).restype = _i
        self.lib = lib

    def num_threads(self):
        return self.lib.oracle_num_threads()

    def conv3x3_fwd(self, x, w, b=None):
        """y [N,K,H,W] for x [N,C,H,W], w [K,C,3,3], optional b [K]."""
        x, w, b = _f64(x), _f64(w), _f64(b)
        N, C, H, W = x.shape
        K = w.shape[0]
        assert w.shape == (K, C, 3, 3) and (b is None or b.shape == (K,))
        y = np.empty((N, K, H, W), np.float64)
        _check(self.lib.oracle_conv3x3_fwd(_p(x), _p(w), _p(b), _p(y), N, C, K, H, W), "fwd")
        return y

    def conv3x3_bwd_data(self, g, w):
        """dx [N,C,H,W] for g [N,K,H,W], w [K,C,3,3]."""
        g, w = _f64(g), _f64(w)
        N, K, H, W = g.shape
        C = w.shape[1]
        assert w.shape == (K, C, 3, 3)
        dx = np.empty((N, C, H, W), np.float64)
        _check(self.lib.oracle_conv3x3_bwd_data(_p(g), _p(w), _p(dx), N, C, K, H, W),
               "bwd_data")
        return dx

    def conv3x3_bwd_weight(self, x, g, want_db=True):
        """(dw [K,C,3,3], db [K] or None) for x [N,C,H,W], g [N,K,H,W]."""
        x, g = _f64(x), _f64(g)
        N, C, H, W = x.shape
        K = g.shape[1]
        assert g.shape == (N, K, H, W)
        dw = np.empty((K, C, 3, 3), np.float64)
        db = np.empty((K,), np.float64) if want_db else None
        _check(self.lib.oracle_conv3x3_bwd_weight(_p(x), _p(g), _p(dw), _p(db),
                                                  N, C, K, H, W), "bwd_weight")
        return dw, db

    def conv3x3_fwd_at(self, x, w, b, idx):
        """y.ravel()[idx], each element computed on its own."""
        x, w, b, idx = _f64(x), _f64(w), _f64(b), _idx(idx)
        N, C, H, W = x.shape
        K = w.shape[0]
        out = np.empty(idx.shape, np.float64)
        _check(self.lib.oracle_conv3x3_fwd_at(_p(x), _p(w), _p(b), N, C, K, H, W,
                                              idx.ctypes.data_as(_I64), idx.size, _p(out)),
               "fwd_at")
        return out

    def conv3x3_bwd_data_at(self, g, w, idx):
        """dx.ravel()[idx], each element computed on its own."""
        g, w, idx = _f64(g), _f64(w), _idx(idx)
        N, K, H, W = g.shape
        C = w.shape[1]
        out = np.empty(idx.shape, np.float64)
        _check(self.lib.oracle_conv3x3_bwd_data_at(_p(g), _p(w), N, C, K, H, W,
                                                   idx.ctypes.data_as(_I64), idx.size,
                                                   _p(out)), "bwd_data_at")
        return out

    def conv3x3_bwd_weight_at(self, x, g, idx):
        """dw.ravel()[idx], each element computed on its own."""
        x, g, idx = _f64(x), _f64(g), _idx(idx)
        N, C, H, W = x.shape
        K = g.shape[1]
        out = np.empty(idx.shape, np.float64)
        _check(self.lib.oracle_conv3x3_bwd_weight_at(_p(x), _p(g), N, C, K, H, W,
                                                     idx.ctypes.data_as(_I64), idx.size,
                                                     _p(out)), "bwd_weight_at")
        return out

    def act_forward(self, z, act):
        """act(z), elementwise, same shape."""
        z = _f64(z)
        y = np.empty_like(z)
        _check(self.lib.oracle_act_forward(_p(z), _p(y), z.size, act), "act_forward")
        return y

    def act_grad(self, gy, z, act):
        """g = gy * act'(z), elementwise, in float64."""
        gy, z = _f64(gy), _f64(z)
        assert gy.shape == z.shape
        g = np.empty_like(gy)
        _check(self.lib.oracle_act_grad(_p(gy), _p(z), _p(g), gy.size, act), "act_grad")
        return g

    def conv3x3_bias_grad_at(self, g, idx):
        """db[idx], each element computed on its own."""
        g, idx = _f64(g), _idx(idx)
        N, K, H, W = g.shape
        out = np.empty(idx.shape, np.float64)
        _check(self.lib.oracle_conv3x3_bias_grad_at(_p(g), N, K, H, W,
                                                    idx.ctypes.data_as(_I64), idx.size,
                                                    _p(out)), "bias_grad_at")
        return out


_default = None


def _o():
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            build()
        _default = Oracle(LIB_PATH)
    return _default


def num_threads():
    return _o().num_threads()


def conv3x3_fwd(x, w, b=None):
    return _o().conv3x3_fwd(x, w, b)


def conv3x3_bwd_data(g, w):
    return _o().conv3x3_bwd_data(g, w)


def conv3x3_bwd_weight(x, g, want_db=True):
    return _o().conv3x3_bwd_weight(x, g, want_db)


def conv3x3_fwd_at(x, w, b, idx):
    return _o().conv3x3_fwd_at(x, w, b, idx)


def conv3x3_bwd_data_at(g, w, idx):
    return _o().conv3x3_bwd_data_at(g, w, idx)


def conv3x3_bwd_weight_at(x, g, idx):
    return _o().conv3x3_bwd_weight_at(x, g, idx)


def conv3x3_bias_grad_at(g, idx):
    return _o().conv3x3_bias_grad_at(g, idx)


def act_forward(z, act):
    return _o().act_forward(z, act)


def act_grad(gy, z, act, bf16=False):
    """g = gy * act'(z).  bf16=True: the bfloat16 operand the bfloat16 path
    contracts, i.e. that exact product rounded once to the nearest bfloat16
    value, ties to even (round_to_bf16 below)."""
    g = _o().act_grad(gy, z, act)
    return round_to_bf16(g) if bf16 else g


def conv3x3_fwd_act(x, w, b, act):
    """(y, z): z = conv3x3_fwd(x, w, b), y = act(z)."""
    z = conv3x3_fwd(x, w, b)
    return act_forward(z, act), z


def conv3x3_bwd_act(x, w, gy, z, act, bf16=False, want_db=True):
    """(dx, dw, db) of L = <act(z), gy> with z = conv3x3_fwd(x, w, b): the
    convolution's backward on g = gy * act'(z)."""
    g = act_grad(gy, z, act, bf16)
    dx = conv3x3_bwd_data(g, w)
    dw, db = conv3x3_bwd_weight(x, g, want_db)
    return dx, dw, db


# ---------------------------------------------------------------------------
# Concatenated input (up-path skip connections).  The UNet of the sourcepulse
# summary ("How It Works") is read as the standard one: each up-path block's
# first convolution takes the channel concatenation [a ; b] of the upsampled
# features a (C0 channels) and the skip tensor b (C1 channels).  The oracle is
# that definition written out: the convolution of the concatenated tensor,
# and for backward-data the split of its input gradient at channel C0.


def _cat(x0, x1):
    return np.concatenate([_f64(x0), _f64(x1)], axis=1)


def conv3x3_fwd_cat(x0, x1, w, b=None):
    """y = conv3x3_fwd([x0 ; x1], w, b); w has C0 + C1 input channels."""
    return conv3x3_fwd(_cat(x0, x1), w, b)


def conv3x3_bwd_data_cat(g, w, C0):
    """(dx0, dx1): the gradient of <conv([x0 ; x1]; w), g> with respect to
    x0 (channels 0..C0-1 of the concatenation) and x1 (the rest)."""
    dx = conv3x3_bwd_data(g, w)
    return dx[:, :C0], dx[:, C0:]


def conv3x3_bwd_weight_cat(x0, x1, g, want_db=True):
    """(dw, db) of <conv([x0 ; x1]; w) + b, g>."""
    return conv3x3_bwd_weight(_cat(x0, x1), g, want_db)


def conv3x3_fwd_cat_at(x0, x1, w, b, idx):
    return conv3x3_fwd_at(_cat(x0, x1), w, b, idx)


def conv3x3_bwd_weight_cat_at(x0, x1, g, idx):
    return conv3x3_bwd_weight_at(_cat(x0, x1), g, idx)


# ---------------------------------------------------------------------------
# Input prologue (GroupNorm-apply + SiLU before the convolution).  The fused
# bias-and-activation kernel of the project-guide page on StyleGAN2's custom
# kernels saves a round trip through memory; the same saving on the input
# side is read as follows: a UNet residual block feeds its convolution
# a = SiLU(u), u = x * scale[n, c] + shift[n, c], where scale and shift fold a
# GroupNorm's statistics and affine parameters into one multiplier and one
# offset per sample and channel.  The convolution pads a (not x) with zeros.
# The backward passes: the gradient with respect to u is
# bwd_data(g, w) * SiLU'(u) (what the GroupNorm backward consumes), and dw is
# the plain backward-weight with the input a.  In bfloat16 mode a is a
# bfloat16 operand: the exact a rounded once to the nearest bfloat16 value
# (du stays unrounded: it is a float32 output).


def _prologue_u(x, scale, shift):
    x = _f64(x)
    s, t = _f64(scale), _f64(shift)
    N, C = x.shape[:2]
    assert s.shape == (N, C) and t.shape == (N, C)
    return x * s[:, :, None, None] + t[:, :, None, None]


def prologue_apply(x, scale, shift, bf16=False):
    """a = SiLU(x * scale[n, c] + shift[n, c]).  bf16=True: the bfloat16
    path's operand, a rounded once to the nearest bfloat16 value, ties to
    even (round_to_bf16 below)."""
    a = act_forward(_prologue_u(x, scale, shift), ACT_SILU)
    return round_to_bf16(a) if bf16 else a


def conv3x3_fwd_gnsilu(x, scale, shift, w, b=None, bf16=False):
    """y = conv3x3_fwd(SiLU(x * scale + shift), w, b) (bf16: on the rounded a)."""
    return conv3x3_fwd(prologue_apply(x, scale, shift, bf16), w, b)


def conv3x3_bwd_data_gnsilu(g, w, x, scale, shift):
    """du = gradient of <y, g> with respect to u = x * scale + shift."""
    return act_grad(conv3x3_bwd_data(g, w), _prologue_u(x, scale, shift), ACT_SILU)


def conv3x3_bwd_weight_gnsilu(x, scale, shift, g, want_db=True, bf16=False):
    """(dw, db) of <conv3x3(SiLU(x * scale + shift); w) + b, g> (bf16: on the
    rounded a)."""
    return conv3x3_bwd_weight(prologue_apply(x, scale, shift, bf16), g, want_db)


# ---------------------------------------------------------------------------
# bfloat16 outputs.  bfloat16 is the float32 exponent with an 8-bit
# significand (7 stored bits); the diffusion-fast README's "Bfloat16"
# section runs its pipeline in it.  A float32 accumulator written as
# bfloat16 is read as rounded to nearest, ties to even -- IEEE's default
# rounding -- and the oracle rounds its exact (fp64) result the same way, in
# one step (rounding through float32 first could round a value twice).


def round_to_bf16(a):
    """Round float64 values to the nearest bfloat16 value, ties to even."""
    a = np.asarray(a, dtype=np.float64)
    out = np.zeros_like(a)
    nz = a != 0
    x = a[nz]
    # spacing of bfloat16 values around x: 2^(e - 7) for |x| in [2^e, 2^(e+1)),
    # and the subnormal spacing 2^-133 below 2^-126
    e = np.floor(np.log2(np.abs(x)))
    e = np.maximum(e, -126.0)
    ulp = np.ldexp(1.0, (e - 7).astype(np.int64))
    q = x / ulp                      # exact: division by a power of two
    # np.log2 can be off by one next to a power of two: then |q| leaves
    # [128, 256) and the spacing is twice (or half) as large
    ulp = np.where(np.abs(q) >= 256.0, ulp * 2.0, ulp)
    ulp = np.where((np.abs(q) < 128.0) & (e > -126.0), ulp * 0.5, ulp)
    q = x / ulp
    out[nz] = np.round(q) * ulp      # np.round: half to even
    return out


# ---------------------------------------------------------------------------
# Nearest-neighbour 2x upsampling before the convolution (a UNet up-path
# block).  The project-guide page on StyleGAN2's custom kernels describes
# upsampling as zero insertion followed by an FIR filter; nearest-neighbour
# upsampling is that with the 2x2 box filter.  The oracle writes it as its
# plain definition -- u[n, c, i, j] = x[n, c, i // 2, j // 2] -- and the
# adjoint for backward-data: each x pixel receives the sum of the gradients
# at its four copies.


def upsample2(x):
    """u = nearest 2x upsampling of x [N, C, H, W] -> [N, C, 2H, 2W]."""
    x = _f64(x)
    return np.repeat(np.repeat(x, 2, axis=2), 2, axis=3)


def downsum2(du):
    """Adjoint of upsample2: [N, C, 2H, 2W] -> [N, C, H, W], the sum of each
    2x2 block."""
    du = _f64(du)
    N, C, H2, W2 = du.shape
    return du.reshape(N, C, H2 // 2, 2, W2 // 2, 2).sum(axis=(3, 5))


def conv3x3_fwd_up2(x, w, b=None):
    """y = conv3x3_fwd(upsample2(x), w, b), y at twice x's resolution."""
    return conv3x3_fwd(upsample2(x), w, b)


def conv3x3_bwd_data_up2(g, w):
    """dx of <conv3x3(upsample2(x); w), g>: the 2x2 block sums of the
    input gradient at the upsampled resolution."""
    return downsum2(conv3x3_bwd_data(g, w))


def conv3x3_bwd_weight_up2(x, g, want_db=True):
    """(dw, db) of <conv3x3(upsample2(x); w) + b, g>."""
    return conv3x3_bwd_weight(upsample2(x), g, want_db)


# ---------------------------------------------------------------------------
# Stride-2 3x3 convolution, zero padding 1 (a UNet's downsample block):
# y[n,k,h,w] = b[k] + sum x[n,c,2h+r-1,2w+s-1] w[k,c,r,s], output H/2 x W/2
# for even H, W -- PyTorch's Conv2d(kernel 3, stride 2, padding 1), read as
# the downsampling of the StyleGAN2 page's resampling section (filter, then
# keep every second sample).  Written as its plain definition: the stride-1
# convolution at every second output pixel.  The adjoints insert zeros: the
# gradient g of the small output placed at the even pixels of the full grid.


def zero_insert2(g):
    """[N, K, H, W] -> [N, K, 2H, 2W] with g at the even pixels, zeros
    elsewhere."""
    g = _f64(g)
    N, K, H, W = g.shape
    z = np.zeros((N, K, 2 * H, 2 * W))
    z[:, :, ::2, ::2] = g
    return z


def conv3x3_fwd_s2(x, w, b=None):
    """y = stride-2 convolution of x (H, W even): [N, K, H/2, W/2]."""
    return conv3x3_fwd(x, w, b)[:, :, ::2, ::2]


def conv3x3_bwd_data_s2(g, w):
    """dx [N, C, 2h, 2w] of <conv_s2(x; w), g> for g [N, K, h, w]."""
    return conv3x3_bwd_data(zero_insert2(g), w)


def conv3x3_bwd_weight_s2(x, g, want_db=True):
    """(dw, db) of <conv_s2(x; w) + b, g>."""
    return conv3x3_bwd_weight(x, zero_insert2(g), want_db)
