"""GPU parity of the original-microscaling variant: E8M0 power-of-two scale
per 32x32 square block, E2M1 elements, no tensor scale (MicroQonv, arXiv
2609.28358, §II-D; §IV-B: the method holds for any block scale), with the
GEMMs on gfx950's scaled FP4 MFMA.

Codes and scales are bit-exact against the oracle; dequantization is
bit-exact; every GEMM output lies within 2e-3 * sum|a*b| of the oracle's
fp64 GEMM on the same quantized tensors, and with an identity weight the
forward and data-gradient GEMMs reproduce the dequantized operand exactly."""
import numpy as np
import pytest
import torch

import microscaling_quantized_convolution_mx_amd as mx
import oracle as O
from microscaling_quantized_convolution_mx_amd import workloads as WL
from gpu_util import DEV, assert_close, conv_buffers, gpu_quantize, oracle_conv, run_layer, say

pytestmark = pytest.mark.gpu

ROLES = [(mx.MX_ROLE_ACT, mx.MX_RNE), (mx.MX_ROLE_WEIGHT, mx.MX_RNE), (mx.MX_ROLE_GRAD, mx.MX_SR),
         (mx.MX_ROLE_GRAD, mx.MX_RNE), (mx.MX_ROLE_WEIGHT, mx.MX_SR), (mx.MX_ROLE_ACT, mx.MX_SR)]
ORACLE_ROLE = {mx.MX_ROLE_ACT: O.ACT, mx.MX_ROLE_WEIGHT: O.WEIGHT, mx.MX_ROLE_GRAD: O.GRAD}


def mx_desc(n, ci, co, h, w, k, s, p):
    return mx.desc(n, ci, co, h, w, k, k, s, s, p, p, block=32)


def src_for(d, role, seed):
    lay = WL.ConvLayer(d.n, d.c_in, d.c_out, d.h, d.w, d.k_h, d.k_w, d.stride_h, d.stride_w, d.pad_h, d.pad_w)
    if role == mx.MX_ROLE_ACT:
        return WL.gen_x(lay, "normal", seed)
    if role == mx.MX_ROLE_WEIGHT:
        return WL.gen_w(lay, seed)
    return WL.gen_dy(lay, 1.0, seed)


def oracle_mx(role, src, rounding=mx.MX_RNE, seed=0):
    return O.quantize_mx(ORACLE_ROLE[role], O.E2M1, src.numpy(), rounding, seed)


def assert_mx_equal(gq, oq, what=""):
    torch.cuda.synchronize()
    assert gq.tensor_scale.item() == 1.0, what
    scales = gq.scales[:gq.nblocks].cpu().numpy()
    bad = np.flatnonzero(scales != oq.scales)
    assert bad.size == 0, f"{what}: {bad.size} of {scales.size} scales differ, first {bad[:5]}"
    codes = gq.codes[:gq.code_bytes].cpu().numpy()
    bad = np.flatnonzero(codes != oq.packed())
    assert bad.size == 0, f"{what}: {bad.size} code bytes differ, first at {bad[:5]}"


QSHAPES = [
    # n, c_in, c_out, h, w, k, stride, pad
    (32, 32, 32, 3, 3, 3, 1, 1),
    (64, 96, 64, 5, 3, 3, 2, 1),
    (96, 32, 160, 2, 2, 1, 1, 0),
]


@pytest.mark.parametrize("shape", QSHAPES)
@pytest.mark.parametrize("role,rounding", ROLES)
def test_quantize_bit_exact(shape, role, rounding):
    d = mx_desc(*shape)
    say("mx quantize", shape, role, rounding)
    src = src_for(d, role, seed=17 + QSHAPES.index(shape) * 7 + role)
    assert_mx_equal(gpu_quantize(d, role, src, rounding, seed=99), oracle_mx(role, src, rounding, 99),
                    f"role {role} rounding {rounding}")


def test_quantize_special_blocks():
    # an all-zero block, a block with NaN, one with Inf, fp32 subnormals,
    # signed zeros and huge values, side by side
    d = mx.desc(64, 64, 64, 2, 2, 1, 1, block=32)   # X and dY of one shape
    g = torch.Generator().manual_seed(8)
    x = torch.randn(2, 2, 64, 64, generator=g)
    x[0, 0, :32, :32] = 0.0
    x[0, 0, 32:, :32] = -0.0
    x[0, 1, 5, 40] = float("nan")
    x[1, 0, 40, 3] = float("-inf")
    x[1, 1, :32, :32] *= 1e-40
    x[1, 1, 32:, 32:] *= 3e37
    say("mx quantize special blocks")
    for role, rnd in ((mx.MX_ROLE_ACT, mx.MX_RNE), (mx.MX_ROLE_GRAD, mx.MX_SR)):
        oq = oracle_mx(role, x, rnd, 5)
        assert 0xFF in oq.scales and 0 in oq.scales
        assert_mx_equal(gpu_quantize(d, role, x, rnd, seed=5), oq, f"special role {role}")


@pytest.mark.parametrize("role,rounding", ROLES[:3])
def test_dequantize_bit_exact(role, rounding):
    d = mx_desc(64, 64, 96, 5, 3, 3, 1, 1)
    say("mx dequantize", role)
    src = src_for(d, role, 31)
    gq = gpu_quantize(d, role, src, rounding, 3)
    out = torch.empty(src.shape, device=DEV)
    mx.mx_dequantize(d, role, gq, out)
    torch.cuda.synchronize()
    ref = oracle_mx(role, src, rounding, 3).dequantize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


SHAPES = [
    # n, ci, co, h, w, kh, kw, sh, sw, ph, pw
    (32, 32, 32, 8, 8, 3, 3, 1, 1, 1, 1),
    (32, 64, 96, 9, 7, 3, 3, 2, 2, 1, 1),      # stride 2, ragged rows and columns
    (64, 32, 64, 6, 6, 1, 1, 2, 2, 0, 0),      # 1x1 stride-2 shortcut
    (32, 32, 32, 5, 5, 5, 5, 1, 1, 2, 2),
    (32, 64, 32, 7, 8, 3, 2, 2, 1, 0, 1),      # rectangular kernel, mixed strides
    (32, 288, 320, 6, 6, 3, 3, 1, 1, 1, 1),    # two row tiles; odd k-block counts
    (64, 32, 32, 32, 32, 1, 1, 1, 1, 0, 0),    # 256 column tiles
    (32, 256, 256, 12, 12, 3, 3, 1, 1, 1, 1),  # wgrad split over K
    (32, 32, 32, 4, 4, 3, 3, 1, 1, 3, 3),      # padding wider than the kernel reach
    (32, 64, 32, 16, 16, 3, 3, 2, 2, 1, 1),    # dgrad phases of 4, 2, 2 and 1 taps
]


@pytest.mark.parametrize("shape", SHAPES)
def test_conv_mx(shape):
    say("mx conv", shape)
    lay = WL.ConvLayer(*shape)
    seed = 300 + SHAPES.index(shape)
    x, w, dy = WL.gen_x(lay, "normal", seed), WL.gen_w(lay, seed + 1), WL.gen_dy(lay, 1.0, seed + 2)
    d = mx.desc_from_layer(lay, mx.MX_E2M1, block=32)
    (qx, qw, qdy), (y, dx, dw) = run_layer(d, x, w, dy, seed_sr=7)
    ox = oracle_mx(mx.MX_ROLE_ACT, x)
    ow = oracle_mx(mx.MX_ROLE_WEIGHT, w)
    ody = oracle_mx(mx.MX_ROLE_GRAD, dy, mx.MX_SR, 7)
    assert_mx_equal(qx, ox, "X")
    assert_mx_equal(qdy, ody, "dY")
    cv = oracle_conv(d)
    ref, s = O.conv_fwd(cv, ow.exact(), ox.exact())
    assert_close(y.cpu().numpy(), ref, s, "fwd")
    ref, s = O.conv_dgrad(cv, ow.exact(), ody.exact())
    assert_close(dx.cpu().numpy(), ref, s, "dgrad")
    ref, s = O.conv_wgrad(cv, ody.exact(), ox.exact())
    assert_close(dw.cpu().numpy(), ref, s, "wgrad")


# Shapes on which the launch takes the 256x256 tile (M above 128 and at
# least 1024 such tiles, or for wgrad a full round of splits), with M and N
# not multiples of 256; the small shapes above all take the 128x128 tile.
# Quantized tensors are compared in full, the GEMMs on sampled outputs.
BIG = [
    # n, ci, co, h, w, kh, kw, sh, sw, ph, pw
    (256, 32, 160, 32, 32, 3, 3, 1, 1, 1, 1),   # fwd and wgrad: 160 rows of the tile, wgrad 288 columns of 512
    (256, 160, 32, 32, 32, 3, 3, 1, 1, 1, 1),   # dgrad: 160 rows of the tile
]


def sample_points(n, rng, npts=16384):
    if n <= npts:
        return np.arange(n, dtype=np.int64)
    return np.unique(np.concatenate([rng.integers(0, n, npts), [0, n - 1, n // 2]])).astype(np.int64)


@pytest.mark.parametrize("shape", BIG)
def test_conv_mx_large_tile(shape):
    say("mx conv, large tile", shape)
    lay = WL.ConvLayer(*shape)
    seed = 500 + BIG.index(shape)
    x, w, dy = WL.gen_x(lay, "normal", seed), WL.gen_w(lay, seed + 1), WL.gen_dy(lay, 1.0, seed + 2)
    d = mx.desc_from_layer(lay, mx.MX_E2M1, block=32)
    (qx, qw, qdy), (y, dx, dw) = run_layer(d, x, w, dy, seed_sr=9)
    ox = oracle_mx(mx.MX_ROLE_ACT, x)
    ow = oracle_mx(mx.MX_ROLE_WEIGHT, w)
    ody = oracle_mx(mx.MX_ROLE_GRAD, dy, mx.MX_SR, 9)
    assert_mx_equal(qx, ox, "X")
    assert_mx_equal(qw, ow, "W")
    assert_mx_equal(qdy, ody, "dY")
    cv = oracle_conv(d)
    rng = np.random.default_rng(seed)
    xe, we, dye = ox.exact(), ow.exact(), ody.exact()
    for name, out, fn, a, b, npts in (("fwd", y, O.conv_fwd_points, we, xe, 16384),
                                      ("dgrad", dx, O.conv_dgrad_points, we, dye, 16384),
                                      ("wgrad", dw, O.conv_wgrad_points, dye, xe, 2048)):
        assert not torch.isnan(out).any(), f"{name}: outputs left unwritten"
        idx = sample_points(out.numel(), rng, npts)
        ref, sabs = fn(cv, a, b, idx)
        assert_close(out.reshape(-1)[torch.from_numpy(idx).to(DEV)].cpu().numpy(), ref, sabs, name)


def test_identity_weight_is_exact():
    # W = I quantizes exactly (scale 2^-2, code 4.0), so a 1x1 fwd returns the
    # dequantized X and a 1x1 dgrad the dequantized dY, bit for bit: every
    # code and scale reaches the MFMA through the right lane
    c, n, hw = 64, 64, 8
    d = mx.desc(n, c, c, hw, hw, 1, 1, block=32)
    say("mx identity")
    g = torch.Generator().manual_seed(12)
    x = torch.randn(hw, hw, c, n, generator=g) * torch.exp2(torch.randint(-8, 8, (hw, hw, c, n), generator=g).float())
    w = torch.eye(c).reshape(c, c, 1, 1)
    qx = gpu_quantize(d, mx.MX_ROLE_ACT, x)
    qw = gpu_quantize(d, mx.MX_ROLE_WEIGHT, w)
    qdy = gpu_quantize(d, mx.MX_ROLE_GRAD, x, mx.MX_SR, 4)
    y = torch.full((hw, hw, c, n), float("nan"), device=DEV)
    dx = torch.full((hw, hw, c, n), float("nan"), device=DEV)
    mx.mx_conv_fwd(d, qw, qx, y)
    mx.mx_conv_dgrad(d, qw, qdy, dx)
    torch.cuda.synchronize()
    assert np.array_equal(oracle_mx(mx.MX_ROLE_WEIGHT, w).exact()[:, :, 0, 0], np.eye(c))
    assert np.array_equal(y.cpu().numpy(), oracle_mx(mx.MX_ROLE_ACT, x).dequantize())
    assert np.array_equal(dx.cpu().numpy(), oracle_mx(mx.MX_ROLE_GRAD, x, mx.MX_SR, 4).dequantize())


def test_empty_batch():
    d = mx.desc(0, 32, 32, 6, 6, 3, 3, 1, 1, 1, 1, block=32)
    say("mx empty batch")
    qx, qw, qdy = (mx.QTensor(d, r, DEV) for r in (0, 1, 2))
    w = WL.gen_w(WL.ConvLayer(32, 32, 32, 6, 6, 3, 3, 1, 1, 1, 1), 3).to(DEV)
    mx.mx_quantize_cbf(d, mx.MX_ROLE_WEIGHT, w, qw)
    for q, role in ((qx, 0), (qdy, 2)):
        mx.mx_quantize_cbf(d, role, torch.empty(0, device=DEV), q)
    y, dx, dw, ws = conv_buffers(d)
    dw.fill_(float("nan"))
    mx.mx_conv_fwd(d, qw, qx, y)
    mx.mx_conv_dgrad(d, qw, qdy, dx)
    mx.mx_conv_wgrad(d, qdy, qx, dw, ws)
    torch.cuda.synchronize()
    assert (dw == 0).all()
