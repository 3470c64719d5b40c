"""Synthetic workloads: layer shapes and seeded input generators.

This module holds shapes and random-number recipes only -- none of the
quantization or convolution arithmetic -- so that the tests can feed the same
bits to the HIP path and to the CPU oracle.

The five workloads are synthetic stand-ins shaped like the networks MicroQonv
(arXiv 2609.28358) evaluates: a single 3x3 layer, a CIFAR ResNet-32 stack and
an ImageNet ResNet-18 stack (§IV-D), a YOLOv8n-shaped backbone+neck at 640x640
with FP8 E4M3 elements (§IV-E), and a 256-channel stress layer plus a 4-bit
latent-replay buffer of 10k maps of 64 channels at 8x8 (§VII).  The datasets
and pretrained weights of the paper are not used: every tensor is drawn from a
seeded generator with the stated distribution.

Layouts (the library's): activations / dX [H][W][C][N], output gradients / Y
[Ho][Wo][Cout][N] (channel-batch-first, batch fastest), weights OIHW.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

E2M1, E2M3, E4M3, E3M2 = 1, 2, 3, 5
FMT_NAMES = {E2M1: "e2m1", E2M3: "e2m3", E4M3: "e4m3", E3M2: "e3m2"}
FMT_BITS = {E2M1: 4, E2M3: 6, E4M3: 8, E3M2: 6}


@dataclass(frozen=True)
class ConvLayer:
    n: int
    c_in: int
    c_out: int
    h: int
    w: int
    k_h: int
    k_w: int
    stride_h: int = 1
    stride_w: int = 1
    pad_h: int = 0
    pad_w: int = 0

    @property
    def h_out(self) -> int:
        return (self.h + 2 * self.pad_h - self.k_h) // self.stride_h + 1

    @property
    def w_out(self) -> int:
        return (self.w + 2 * self.pad_w - self.k_w) // self.stride_w + 1

    def flops(self) -> int:
        """Dense multiply-add count x2 of one pass (padding taps included)."""
        return 2 * self.n * self.c_out * self.h_out * self.w_out * self.c_in * self.k_h * self.k_w

    def numel_x(self) -> int:
        return self.h * self.w * self.c_in * self.n

    def numel_w(self) -> int:
        return self.c_out * self.c_in * self.k_h * self.k_w

    def numel_dy(self) -> int:
        return self.h_out * self.w_out * self.c_out * self.n

    def tag(self) -> str:
        return (f"{self.c_in}->{self.c_out}@{self.h}x{self.w} k{self.k_h}x{self.k_w} "
                f"s{self.stride_h} p{self.pad_h} n{self.n}")


def conv(n, c_in, c_out, hw, k, s=1, p=0) -> ConvLayer:
    return ConvLayer(n, c_in, c_out, hw, hw, k, k, s, s, p, p)


@dataclass
class Workload:
    key: str
    name: str
    layers: list
    elem_fmts: tuple
    x_dist: str = "normal"          # normal | halfnormal | silu
    dy_sigma: float = 1.0
    lr_buffer: tuple | None = None  # (n_maps, c, h, w) of the latent-replay buffer
    cfg_index: int = 0
    notes: str = ""
    extra: dict = field(default_factory=dict)

    def flops(self) -> int:
        """fwd + dgrad + wgrad dense flops over all layers, one format."""
        return sum(3 * l.flops() for l in self.layers)


def _resnet32(n=128):
    L = [conv(n, 16, 16, 32, 3, 1, 1) for _ in range(10)]
    L += [conv(n, 16, 32, 32, 3, 2, 1)] + [conv(n, 32, 32, 16, 3, 1, 1) for _ in range(9)]
    L += [conv(n, 32, 64, 16, 3, 2, 1)] + [conv(n, 64, 64, 8, 3, 1, 1) for _ in range(9)]
    return L


def _resnet18(n=64):
    L = [conv(n, 64, 64, 56, 3, 1, 1) for _ in range(4)]
    for cin, c, hw in ((64, 128, 56), (128, 256, 28), (256, 512, 14)):
        L.append(conv(n, cin, c, hw, 3, 2, 1))
        L += [conv(n, c, c, hw // 2, 3, 1, 1) for _ in range(3)]
        L.append(conv(n, cin, c, hw, 1, 2, 0))
    return L


def _c2f(n, c_in, c, hw, r):
    """1x1 expand, 2r 3x3 convs at c/2, 1x1 fuse of (2+r)c/2 channels."""
    L = [conv(n, c_in, c, hw, 1, 1, 0)]
    L += [conv(n, c // 2, c // 2, hw, 3, 1, 1) for _ in range(2 * r)]
    L.append(conv(n, (2 + r) * c // 2, c, hw, 1, 1, 0))
    return L


def _yolov8n(n=16):
    L = []
    hw = 320
    for (cin, c, r) in ((16, 32, 1), (32, 64, 2), (64, 128, 2), (128, 256, 1)):
        L.append(conv(n, cin, c, hw, 3, 2, 1))
        hw //= 2
        L += _c2f(n, c, c, hw, r)
    L += [conv(n, 256, 128, 20, 1, 1, 0), conv(n, 512, 256, 20, 1, 1, 0)]
    L += _c2f(n, 384, 128, 40, 1)
    L += _c2f(n, 192, 64, 80, 1)
    L.append(conv(n, 64, 64, 80, 3, 2, 1))
    L += _c2f(n, 192, 128, 40, 1)
    L.append(conv(n, 128, 128, 40, 3, 2, 1))
    L += _c2f(n, 384, 256, 20, 1)
    return L


def workloads() -> dict:
    W = {
        "c1": Workload("c1", "single 3x3 conv 16->16 @16x16, N=8, stride 1, no padding",
                       [conv(8, 16, 16, 16, 3, 1, 0)], (E2M1,), "normal", 1.0, cfg_index=0),
        "c2": Workload("c2", "ResNet-32 CIFAR conv stack (30 quantized 3x3 convs), N=128",
                       _resnet32(), (E2M1,), "normal", 1.0, cfg_index=1),
        "c3": Workload("c3", "ResNet-18 ImageNet conv stack at 224 (19 quantized convs), N=64",
                       _resnet18(), (E2M1,), "halfnormal", 0.1, cfg_index=2),
        "c4": Workload("c4", "YOLOv8n-shaped backbone+neck at 640 (44 quantized convs), N=16",
                       _yolov8n(), (E4M3,), "silu", 1.0, cfg_index=3),
        "c5": Workload("c5", "stress 3x3 conv 256->256 @56x56 pad 1, N=256",
                       [conv(256, 256, 256, 56, 3, 1, 1)], (E2M1, E2M3, E4M3), "normal", 1.0,
                       lr_buffer=(10000, 64, 8, 8), cfg_index=4),
    }
    return W


# ---------------------------------------------------------------------------
# seeded generators (CPU, fp32)
# ---------------------------------------------------------------------------

def seed_for(cfg_index: int, layer: int, t: int) -> int:
    """t: 1 = X, 2 = W, 3 = dY, 4 = stochastic-rounding seed, 5 = replay buffer."""
    return 1000 * (cfg_index + 1) + 10 * layer + t


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(seed)
    return g


def gen_x(layer: ConvLayer, dist: str, seed: int) -> torch.Tensor:
    """Activation in [H][W][Cin][N]."""
    x = torch.randn(layer.h, layer.w, layer.c_in, layer.n, generator=_gen(seed))
    if dist == "halfnormal":
        x = x.abs_()
    elif dist == "silu":
        x = torch.nn.functional.silu(x)
    elif dist != "normal":
        raise ValueError(dist)
    return x.contiguous()


def gen_w(layer: ConvLayer, seed: int) -> torch.Tensor:
    """Kaiming-normal weights, OIHW: std = sqrt(2 / (Cin*Kh*Kw))."""
    std = math.sqrt(2.0 / (layer.c_in * layer.k_h * layer.k_w))
    w = torch.randn(layer.c_out, layer.c_in, layer.k_h, layer.k_w, generator=_gen(seed))
    return (w * std).contiguous()


def gen_dy(layer: ConvLayer, sigma: float, seed: int) -> torch.Tensor:
    """Output gradient in [Ho][Wo][Cout][N], N(0, sigma^2)."""
    dy = torch.randn(layer.h_out, layer.w_out, layer.c_out, layer.n, generator=_gen(seed))
    return (dy * sigma).contiguous()


def gen_lr_maps(n_maps: int, c: int, h: int, w: int, seed: int) -> torch.Tensor:
    """Post-ReLU latent maps (half-normal) in [H][W][C][N]."""
    x = torch.randn(h, w, c, n_maps, generator=_gen(seed)).abs_()
    return x.contiguous()


def gen_tensor(shape, dist: str, seed: int, sigma: float = 1.0) -> torch.Tensor:
    """Generic seeded tensor of the given shape."""
    x = torch.randn(*shape, generator=_gen(seed))
    if dist == "halfnormal":
        x = x.abs_()
    elif dist == "silu":
        x = torch.nn.functional.silu(x)
    elif dist == "uniform":
        x = torch.rand(*shape, generator=_gen(seed)) * 2 - 1
    return (x * sigma).contiguous()


# Grid-aligned inputs for GEMM checks that must hold bit for bit.  Every 8x8
# block of a tensor holds one element of the format's largest magnitude (at
# a fixed in-block position per tensor) and small grid values elsewhere,
# all times 448 * 2^k.  With the tensor maximum in every block, a
# microscaling quantizer of the two-level kind gives a power-of-two tensor
# scale and the largest block scale in every block, so the elements sit on
# the grid unchanged.  The fixed positions never pair two largest elements
# in a product of the three GEMMs (the weight's sits at in-block (c_out 0,
# c_in 0), the activation's at (c_in 1, n 1), the gradient's at (c_out 1,
# n 0)), which keeps every output's sum of |products| small.
EXACT_LARGEST = {E2M1: 6.0, E2M3: 7.5, E4M3: 448.0}
EXACT_SMALL = {E2M1: (0.5, 1.0), E2M3: (0.5, 1.0), E4M3: (64.0, 128.0)}
EXACT_POW2 = {"x": -8, "w": -10, "dy": -6}


def _exact_fill(shape, fmt, seed):
    g = _gen(seed)
    small = EXACT_SMALL[fmt]
    pick = torch.randint(0, 5, shape, generator=g)   # 0, +-small[0], +-small[1]
    mag = torch.tensor([0.0, small[0], small[0], small[1], small[1]])[pick]
    sign = torch.where(torch.randint(0, 2, shape, generator=g) == 0, 1.0, -1.0)
    return mag * sign, torch.where(torch.randint(0, 2, shape, generator=g) == 0, 1.0, -1.0)


def gen_exact(layer: ConvLayer, which: str, fmt: int, seed: int) -> torch.Tensor:
    """which: "x" ([H][W][Cin][N]), "w" (OIHW) or "dy" ([Ho][Wo][Cout][N])."""
    if which == "x":
        shape = (layer.h, layer.w, layer.c_in, layer.n)
    elif which == "dy":
        shape = (layer.h_out, layer.w_out, layer.c_out, layer.n)
    else:
        shape = (layer.c_out, layer.c_in, layer.k_h, layer.k_w)
    v, sgn = _exact_fill(shape, fmt, seed)
    big = EXACT_LARGEST[fmt]
    if which == "x":
        v[:, :, 1::8, 1::8] = big * sgn[:, :, 1::8, 1::8]
    elif which == "dy":
        v[:, :, 1::8, 0::8] = big * sgn[:, :, 1::8, 0::8]
    else:
        v[0::8, 0::8, :, :] = big * sgn[0::8, 0::8, :, :]
    return (v * (448.0 * 2.0 ** EXACT_POW2[which])).contiguous()


def exact_quantum(which: str, fmt: int) -> float:
    """Step of the tensor's dequantized values (every value is a multiple)."""
    return EXACT_SMALL[fmt][0] * 448.0 * 2.0 ** EXACT_POW2[which]
