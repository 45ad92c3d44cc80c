"""Seeded synthetic inputs for the 3x3 convolution (shared by tests and bench).

This module holds shapes, value distributions and seeded draws only; it
contains none of the convolution's arithmetic, and imports neither the oracle
nor the HIP library.  Both sides of every parity check draw their inputs here.

The layers follow the UNet-shaped workloads the sources describe: a diffusion
UNet trained on ImageNet at 64x64 resolution (sourcepulse summary of the
C++/CUDA UNet project, "Quick Start & Requirements").  No dataset is used:
seeded random tensors with the stated distributions stand in for it.

Draw recipe, per layer: a CPU ``torch.Generator`` seeded with
``seed * 1000 + layer_index`` draws x, w, b, g in that order, in float32; for
bfloat16 layers x, w and g are then rounded to bfloat16 (round to nearest
even); b stays float32.  The integer-exact variant draws x, w, g from the
integers {-2..2} and b from {-2, -1.5, ..., 2}, so that every product and every
partial sum of the convolution is exactly representable in float32.
"""
from dataclasses import dataclass, replace
import math

import torch


@dataclass(frozen=True)
class Layer:
    name: str
    N: int
    C: int       # input channels
    K: int       # output channels
    H: int
    W: int
    dtype: str   # "f32" or "bf16" (x, w, g); b and all outputs are float32
    seed: int
    index: int = 0
    x_dist: str = "normal"      # "normal" -> N(0,1); "silu_normal" -> SiLU(N(0,1))
    w_bound: float = 0.0        # U(-w_bound, w_bound); 0 -> Kaiming-uniform sqrt(6/(9C))
    b_bound: float = 0.05
    g_std: float = 1.0
    cat: int = 0                # > 0: the input is [first `cat` channels ; the rest]

    @property
    def weight_bound(self):
        return self.w_bound if self.w_bound > 0 else math.sqrt(6.0 / (9 * self.C))

    @property
    def shape(self):
        return (self.N, self.C, self.K, self.H, self.W)


def _unet_sweep(dtype):
    """32 stride-1 3x3 convs of one 64x64 UNet training step: channel
    multipliers [1,2,3,4] on base 128 at resolutions 64/32/16/8, two convs per
    residual block, two blocks per level, down and up paths; up-path blocks
    take the skip concatenation as one contiguous C_in-channel input; ``cat``
    records where it splits (upsampled features first, then the skip)."""
    ch = [128, 256, 384, 512]
    res = [64, 32, 16, 8]
    layers = []
    prev = 128
    for lv in range(4):
        c = ch[lv]
        for cin in (prev, c, c, c):
            layers.append((f"down{lv}", cin, c, res[lv]))
        prev = c
    below = 512
    cats = [0] * len(layers)
    for lv in reversed(range(4)):
        c = ch[lv]
        for cin, first in ((below + c, below), (c, 0), (2 * c, c), (c, 0)):
            layers.append((f"up{lv}", cin, c, res[lv]))
            cats.append(first)
        below = c
    out = []
    for i, (nm, cin, cout, r) in enumerate(layers):
        out.append(Layer(f"{nm}_{i:02d}_{cin}to{cout}_{r}x{r}_{dtype}", 32, cin, cout, r, r,
                         dtype, 4, i, cat=cats[i]))
    return out


CONFIGS = {
    1: [Layer("small_2x64to64_32x32_f32", 2, 64, 64, 32, 32, "f32", 0, 0,
              w_bound=1.0 / math.sqrt(576.0))],
    2: [Layer("stem_32x64to64_64x64_f32", 32, 64, 64, 64, 64, "f32", 1, 0)],
    3: [Layer("mid_32x128to256_32x32_f32", 32, 128, 256, 32, 32, "f32", 2, 0,
              x_dist="silu_normal", g_std=0.1),
        Layer("mid_32x256to256_32x32_f32", 32, 256, 256, 32, 32, "f32", 2, 1,
              x_dist="silu_normal", g_std=0.1)],
    4: [Layer("bottleneck_64x512to512_16x16_bf16", 64, 512, 512, 16, 16, "bf16", 3, 0),
        Layer("bottleneck_64x512to512_8x8_bf16", 64, 512, 512, 8, 8, "bf16", 3, 1)],
    5: _unet_sweep("f32") + _unet_sweep("bf16"),
}

# Ragged and edge shapes (N, C, K, H, W) for parity beyond the UNet layers.
RAGGED_SHAPES = [
    (1, 1, 1, 1, 1), (1, 1, 1, 3, 3), (1, 3, 5, 7, 9), (2, 17, 33, 5, 13),
    (3, 64, 64, 31, 33), (1, 513, 7, 8, 8), (1, 2, 3, 2, 70), (2, 6, 40, 9, 4),
]


def small_layer(N, C, K, H, W, dtype="f32", seed=7, index=0):
    return Layer(f"shape_{N}x{C}to{K}_{H}x{W}_{dtype}", N, C, K, H, W, dtype, seed, index)


def with_dtype(layer, dtype):
    return replace(layer, dtype=dtype, name=layer.name.rsplit("_", 1)[0] + "_" + dtype)


def make_inputs(layer, integer_exact=False, with_bias=True):
    """Return dict of CPU tensors x [N,C,H,W], w [K,C,3,3], b [K] (float32 or
    None) and g [N,K,H,W]; x, w, g are float32 or bfloat16 per ``layer.dtype``."""
    gen = torch.Generator("cpu").manual_seed(layer.seed * 1000 + layer.index)
    N, C, K, H, W = layer.shape
    if integer_exact:
        x = torch.randint(-2, 3, (N, C, H, W), generator=gen).float()
        w = torch.randint(-2, 3, (K, C, 3, 3), generator=gen).float()
        b = torch.randint(-4, 5, (K,), generator=gen).float() * 0.5
        g = torch.randint(-2, 3, (N, K, H, W), generator=gen).float()
    else:
        x = torch.randn((N, C, H, W), generator=gen)
        if layer.x_dist == "silu_normal":
            x = x * torch.sigmoid(x)
        bound = layer.weight_bound
        w = (torch.rand((K, C, 3, 3), generator=gen) * 2.0 - 1.0) * bound
        b = (torch.rand((K,), generator=gen) * 2.0 - 1.0) * layer.b_bound
        g = torch.randn((N, K, H, W), generator=gen) * layer.g_std
    if layer.dtype == "bf16":
        x, w, g = x.bfloat16(), w.bfloat16(), g.bfloat16()
    elif layer.dtype != "f32":
        raise ValueError(f"unknown dtype {layer.dtype}")
    return {"x": x.contiguous(), "w": w.contiguous(),
            "b": b.contiguous() if with_bias else None, "g": g.contiguous()}


def make_prologue(layer):
    """Seeded per-sample, per-channel scale [N, C] ~ U(0.5, 1.5) and shift
    [N, C] ~ N(0, 0.5^2), float32 CPU tensors: a GroupNorm folded into one
    multiplier and one offset per sample and channel, at the magnitudes a
    trained network's normalisation produces."""
    gen = torch.Generator("cpu").manual_seed(layer.seed * 1000 + layer.index + 500)
    N, C = layer.N, layer.C
    scale = torch.rand((N, C), generator=gen) + 0.5
    shift = torch.randn((N, C), generator=gen) * 0.5
    return scale.contiguous(), shift.contiguous()


# The first convolution of the UNet: the 3-channel 64x64 image into the 128
# base channels (the shape of the diffusion UNet's stem; not one of the
# benchmark configurations, a case for the few-channel paths).
IMAGE_STEM = {dt: Layer(f"image_stem_32x3to128_64x64_{dt}", 32, 3, 128, 64, 64, dt, 6, 0)
              for dt in ("f32", "bf16")}


# The convolutions of the UNet's upsample blocks (nearest 2x, then a 3x3
# convolution keeping the channels): 8->16, 16->32 and 32->64 at N = 32.
# H, W are the input's (pre-upsampling) sizes; g is drawn at 2H x 2W.
UPSAMPLE = [Layer(f"upsample_{c}ch_{r}to{2 * r}_f32", 32, c, c, r, r, "f32", 7, i)
            for i, (c, r) in enumerate(((512, 8), (384, 16), (256, 32)))]


# The convolutions of the UNet's downsample blocks (3x3, stride 2, keeping
# the channels): 64->32, 32->16 and 16->8 at N = 32; H, W are the input's.
DOWNSAMPLE = [Layer(f"downsample_{c}ch_{r}to{r // 2}_f32", 32, c, c, r, r, "f32", 8, i)
              for i, (c, r) in enumerate(((128, 64), (256, 32), (384, 16)))]
