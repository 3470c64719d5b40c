"""Byte and quantization accounting -- TEST INFRASTRUCTURE ONLY (part of the oracle).

Restates the storage arithmetic of "MicroQonv: Reshaping Convolution Tensors
for Efficient Microscaling in Training and Inference" (arXiv 2609.28358):

* bits per stored element = element bits + block-scale bits / block size
  (+ the fp32 tensor scale, 32 bits per tensor) -- §II-D, §IV-B, §VI-A
* Table I's backward memory-movement ratio against FP32 storage
* Table V's FP32 tensor sizes, re-derived from the layer inventories of the
  two classification networks at batch 32 -- §V-A, Table V
* the im2col expansion factor Kh*Kw*Ho*Wo/(H*W) of the quantize-after-im2col
  flow -- §V-B

The network inventories are the standard CIFAR ResNet-32 (6n+2 layers, n=5,
widths 16/32/64) and ImageNet ResNet-18 (He et al., "Deep Residual Learning
for Image Recognition", CVPR 2016, §4.2 and Table 1).  Only their shapes are
used.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Conv:
    c_in: int
    c_out: int
    h: int          # input spatial size (square)
    k: int
    stride: int
    pad: int

    @property
    def h_out(self) -> int:
        return (self.h + 2 * self.pad - self.k) // self.stride + 1

    def act_elems(self, n: int) -> int:
        """Input activation elements of the layer (what is kept for backward)."""
        return n * self.c_in * self.h * self.h

    def im2col_elems(self, n: int) -> int:
        """Entries of the explicit im2col matrix X' (K x J)."""
        return n * self.k * self.k * self.c_in * self.h_out * self.h_out

    def weight_elems(self) -> int:
        return self.c_out * self.c_in * self.k * self.k


def bits_per_element(elem_bits: int, scale_bits: int = 8, block: int = 64) -> float:
    """Storage bits per element of a microscaled tensor, ignoring the single
    fp32 tensor scale."""
    return elem_bits + scale_bits / block


def fp32_ratio(elem_bits: int, scale_bits: int = 8, block: int = 64) -> float:
    """FP32 storage divided by microscaled storage."""
    return 32.0 / bits_per_element(elem_bits, scale_bits, block)


# Table I's x7.53 is 32 / 4.25, i.e. a scale overhead of 0.25 bit per element
# (for instance an 8-bit scale per 32 elements, or 16 scale bits per 64-element
# block); an 8-bit E4M3 scale per 8x8 block costs 0.125 bit (x7.76).
TABLE1_OVERHEAD_BITS = 0.25


def resnet32_cifar() -> tuple[list[Conv], tuple[int, int]]:
    """All 31 convolutions (stem + 3 stages x 5 blocks x 2) and the FC layer
    (in_features, out_features) of ResNet-32 for 32x32 inputs, 100 classes.
    Shortcuts are parameter-free (option A), as in the CIFAR networks."""
    convs = [Conv(3, 16, 32, 3, 1, 1)]
    c, h = 16, 32
    for stage, width in enumerate((16, 32, 64)):
        for blk in range(5):
            stride = 2 if (stage > 0 and blk == 0) else 1
            convs.append(Conv(c, width, h, 3, stride, 1))
            h = convs[-1].h_out
            convs.append(Conv(width, width, h, 3, 1, 1))
            c = width
    return convs, (64, 100)


def resnet18_imagenet() -> tuple[list[Conv], tuple[int, int]]:
    """The 20 convolutions of ResNet-18 (7x7 stem, 16 3x3 convs, 3 1x1
    projection shortcuts) and its FC layer, for 224x224 inputs."""
    convs = [Conv(3, 64, 224, 7, 2, 3)]
    c, h = 64, 56  # after the 3x3/2 max-pool
    for stage, width in enumerate((64, 128, 256, 512)):
        for blk in range(2):
            stride = 2 if (stage > 0 and blk == 0) else 1
            conv1 = Conv(c, width, h, 3, stride, 1)
            convs.append(conv1)
            if stride != 1 or c != width:
                convs.append(Conv(c, width, h, 1, stride, 0))
            h = conv1.h_out
            convs.append(Conv(width, width, h, 3, 1, 1))
            c = width
    return convs, (512, 1000)


def stack_fp32_sizes(convs: list[Conv], fc: tuple[int, int], n: int) -> dict:
    """FP32 bytes of the activations kept for backward (every conv input plus
    the FC input) and of all weights (conv + FC weights and FC bias)."""
    act = sum(cv.act_elems(n) for cv in convs) + n * fc[0]
    wts = sum(cv.weight_elems() for cv in convs) + fc[0] * fc[1] + fc[1]
    return {"act_elems": act, "act_bytes": 4 * act, "weight_elems": wts, "weight_bytes": 4 * wts}


def im2col_expansion(convs: list[Conv], n: int) -> float:
    """Entries of all explicit im2col matrices over activation elements."""
    return sum(cv.im2col_elems(n) for cv in convs) / sum(cv.act_elems(n) for cv in convs)


def expansion_factor(cv: Conv) -> float:
    """Exact per-layer expansion Kh*Kw*Ho*Wo/(H*W)."""
    return cv.k * cv.k * cv.h_out * cv.h_out / (cv.h * cv.h)
