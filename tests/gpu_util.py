"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and the CPU oracle on the same seeded inputs, and compare.

Pass criteria: quantized codes, block scales, tensor scale and amax are
bit-identical; every GEMM output satisfies |gpu - ref| <= 2e-3 * S with
S = sum |a*b| over the exact dequantized operands (fp64 oracle)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import microscaling_quantized_convolution_mx_amd as mx
import oracle as O

TOL = 2e-3
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_quantize(d, role, src: torch.Tensor, rounding=mx.MX_RNE, seed=0, amax=None, dev_src=None):
    q = mx.QTensor(d, role, DEV)
    if amax is not None:
        q.amax.fill_(amax)
    s = dev_src if dev_src is not None else src.to(DEV)
    mx.mx_quantize_cbf(d, role, s, q, rounding, seed, amax_given=amax is not None)
    return q


# the oracle numbers the formats on its own
OFMT = {mx.MX_E2M1: O.E2M1, mx.MX_E2M3: O.E2M3, mx.MX_E4M3: O.E4M3, mx.MX_E3M2: O.E3M2,
        mx.MX_UE2M1: O.UE2M1}


def ofmt(fmt: int) -> int:
    """The oracle's number of the library's element format fmt."""
    return OFMT[fmt]


def oracle_quantize(d, role, src: torch.Tensor, rounding=mx.MX_RNE, seed=0, amax=None):
    return O.quantize(role, ofmt(mx.role_fmt(d, role)), src.numpy(), rounding, seed, amax)


def f32_bits(v: float) -> int:
    return int(np.array([v], dtype=np.float32).view(np.uint32)[0])


def assert_quant_equal(gq: mx.QTensor, oq, what=""):
    torch.cuda.synchronize()
    codes = gq.codes[:gq.code_bytes].cpu().numpy()
    scales = gq.scales[:gq.nblocks].cpu().numpy()
    t = gq.tensor_scale.item()
    amax = gq.amax.item()
    if np.isnan(oq.t):
        assert np.isnan(t), what
    else:
        assert f32_bits(t) == f32_bits(oq.t), f"{what}: T {t!r} vs {oq.t!r}"
    if np.isnan(oq.amax) or np.isinf(oq.amax):
        assert not np.isfinite(amax), what
    else:
        assert f32_bits(amax) == f32_bits(oq.amax), f"{what}: amax {amax!r} vs {oq.amax!r}"
    assert scales.size == oq.scales.size
    bad = np.flatnonzero(scales != oq.scales)
    assert bad.size == 0, f"{what}: {bad.size} scales differ, first block {bad[:5]}"
    packed = oq.packed()
    bad = np.flatnonzero(codes != packed)
    assert bad.size == 0, f"{what}: {bad.size} code bytes differ, first at {bad[:5]}"


def assert_close(got: np.ndarray, ref: np.ndarray, s: np.ndarray, what=""):
    got = got.astype(np.float64)
    err = np.abs(got - ref)
    bound = TOL * s
    bad = ~(err <= bound)
    if bad.any():
        i = np.flatnonzero(bad.ravel())
        ratio = err.ravel()[i] / np.maximum(s.ravel()[i], 1e-300)
        raise AssertionError(f"{what}: {i.size} of {got.size} outputs outside 2e-3*S; "
                             f"first idx {i[:5]}, err/S {ratio[:5]}, got {got.ravel()[i[:3]]}, "
                             f"ref {ref.ravel()[i[:3]]}")


def conv_buffers(d):
    """Output buffers of the three GEMMs and the weight-gradient workspace,
    filled with NaN: an output the kernels never write, or a split partial
    the reduce reads without the GEMM having written it, shows up as NaN."""
    y = torch.full((d.h_out, d.w_out, d.c_out, d.n), float("nan"), device=DEV)
    dx = torch.full((d.h, d.w, d.c_in, d.n), float("nan"), device=DEV)
    dw = torch.full((d.c_out, d.c_in, d.k_h, d.k_w), float("nan"), device=DEV)
    ws = torch.full((max(mx.mx_wgrad_workspace_bytes(d) // 4, 4),), float("nan"), device=DEV)
    return y, dx, dw, ws


def run_layer(d, x, w, dy, seed_sr, ops=("fwd", "dgrad", "wgrad")):
    """Quantize X, W, dY on the GPU and run the requested GEMMs.
    Returns the quantized tensors and the fp32 outputs (device)."""
    qx = gpu_quantize(d, mx.MX_ROLE_ACT, x)
    qw = gpu_quantize(d, mx.MX_ROLE_WEIGHT, w)
    qdy = gpu_quantize(d, mx.MX_ROLE_GRAD, dy, mx.MX_SR, seed_sr)
    y, dx, dw, ws = conv_buffers(d)
    if "fwd" in ops:
        mx.mx_conv_fwd(d, qw, qx, y)
    if "dgrad" in ops:
        mx.mx_conv_dgrad(d, qw, qdy, dx)
    if "wgrad" in ops:
        mx.mx_conv_wgrad(d, qdy, qx, dw, ws)
    torch.cuda.synchronize()
    return (qx, qw, qdy), (y, dx, dw)


def oracle_conv(d):
    return O.conv(d.n, d.c_in, d.c_out, d.h, d.w, d.k_h, d.k_w, d.stride_h, d.stride_w,
                  d.pad_h, d.pad_w)
