"""Byte accounting pins (CPU only): Table I's x7.53 and Table V's FP32 sizes.

MicroQonv (arXiv 2609.28358): Table I (backward memory movement of FP32
storage against 4-bit microscaling), Table V (tensor sizes of the DRAM
simulation at batch 32), §V-B (im2col expansion), §VI-A (3.125 bits per
post-ReLU pixel).
"""
import json
import os

import pytest

from oracle import accounting as A

GOLD = os.path.join(os.path.dirname(__file__), "golden")
T1 = json.load(open(os.path.join(GOLD, "table1.json")))
T5 = json.load(open(os.path.join(GOLD, "table5.json")))
FACTS = json.load(open(os.path.join(GOLD, "format_facts.json")))


def test_table1_fp32_ratio():
    dacapo = T1["backward_memory_movement_vs_microqonv"]["dacapo"]["A"]
    r = 32.0 / (4 + A.TABLE1_OVERHEAD_BITS)
    assert round(r, 2) == dacapo
    # an 8-bit E4M3 scale per 8x8 block costs 0.125 bit per element: x7.76
    assert A.fp32_ratio(4, 8, 64) == pytest.approx(32 / 4.125)
    assert A.bits_per_element(4, 8, 64) == 4.125


def test_table1_im2col_ratio():
    # storing the quantized im2col tensor of a 3x3, stride-1, pad-1 layer costs
    # Kh*Kw = 9 times the activation
    cv = A.Conv(16, 16, 32, 3, 1, 1)
    assert A.expansion_factor(cv) == T1["backward_memory_movement_vs_microqonv"]["cuyckens"]["A"]


def test_post_relu_bits_per_pixel():
    f = FACTS["post_relu_fp4_bits_per_pixel"]
    assert A.bits_per_element(f["element_bits"], f["scale_bits"], f["block"]) == f["value"]
    g = FACTS["replay_sample_gain"]
    assert g["vs_bits"] / f["value"] == pytest.approx(g["value"], rel=0.03)


def test_table5_resnet32_fp32_sizes():
    convs, fc = A.resnet32_cifar()
    assert len(convs) == 31
    sz = A.stack_fp32_sizes(convs, fc, T5["batch"])
    assert round(sz["act_bytes"] / 1e6, 2) == T5["r32_cifar100"]["activations_MB"]["dacapo"]
    assert round(sz["weight_bytes"] / 1e6, 2) == T5["r32_cifar100"]["weights_MB"]["dacapo"]


def test_table5_resnet18_fp32_sizes():
    convs, fc = A.resnet18_imagenet()
    assert len(convs) == 20
    sz = A.stack_fp32_sizes(convs, fc, T5["batch"])
    assert round(sz["act_bytes"] / 1e6, 2) == pytest.approx(T5["r18_imagenet"]["activations_MB"]["dacapo"],
                                                           abs=0.011)
    assert round(sz["weight_bytes"] / 1e6, 2) == T5["r18_imagenet"]["weights_MB"]["dacapo"]


def test_table5_resnet32_im2col_expansion():
    # quantize-after-im2col stores X' (Cuyckens ext.), MicroQonv stores X: the
    # ratio of their activation sizes in Table V is the expansion factor
    convs, _ = A.resnet32_cifar()
    e = A.im2col_expansion(convs, T5["batch"])
    mb = T5["r32_cifar100"]["activations_MB"]
    assert e == pytest.approx(mb["cuyckens"] / mb["microqonv"], rel=2e-3)
    # "around x8.5" in §V-B
    assert round(e, 1) == 8.5


def test_table5_quantized_weight_size_unpinned_report():
    # Table V's quantized weight size (0.244 MB) implies ~4.17 bits/element for
    # the R32 weights, between the 4.125 of an 8-bit scale per 64 elements and
    # Table I's 4.25: reported, not pinned.
    convs, fc = A.resnet32_cifar()
    sz = A.stack_fp32_sizes(convs, fc, T5["batch"])
    implied = T5["r32_cifar100"]["weights_MB"]["microqonv"] * 1e6 * 8 / sz["weight_elems"]
    assert 4.0 < implied < 4.3
