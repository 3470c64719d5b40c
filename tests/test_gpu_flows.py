"""The quantize-after-im2col baseline on the GPU (MicroQonv, arXiv
2609.28358, §III-C and Table I: the extrapolation of Cuyckens et al. to
convolutions, which writes the expanded activation X' and quantizes it).

  - mx_im2col_cbf writes X' [Ho][Wo][Kh][Kw][C][N] exactly: each row is X at
    one position, or zeros in the padding (checked against X' gathered on
    the host from X, bit for bit);
  - quantized as a 1x1 activation with C' = Kh*Kw*C channels, X' gives for
    every tap the very blocks of Xq (same tensor scale, same block scales
    and codes): in the channel-batch-first layout quantizing after im2col
    reproduces MicroQonv's single quantization, only nine times over;
  - the GEMMs of the baseline (the 1x1 calls on X') meet the oracle's bound."""
import numpy as np
import pytest
import torch

import microscaling_quantized_convolution_mx_amd as mx
import oracle as O
from microscaling_quantized_convolution_mx_amd import workloads as WL
from gpu_util import DEV, assert_close, gpu_quantize, oracle_conv, say

pytestmark = pytest.mark.gpu

IM2COL_SHAPES = [
    (8, 16, 16, 16, 16, 3, 3, 1, 1, 1, 1),
    (8, 16, 8, 9, 10, 3, 3, 2, 2, 1, 1),
    (16, 8, 24, 6, 6, 1, 1, 2, 2, 0, 0),
    (8, 8, 8, 5, 5, 5, 5, 1, 1, 2, 2),
]


def host_im2col(x: np.ndarray, d) -> np.ndarray:
    h, w, c, n = x.shape
    out = np.zeros((d.h_out, d.w_out, d.k_h, d.k_w, c, n), dtype=np.float32)
    for oy in range(d.h_out):
        for ox in range(d.w_out):
            for kh in range(d.k_h):
                for kw in range(d.k_w):
                    iy, ix = oy * d.stride_h - d.pad_h + kh, ox * d.stride_w - d.pad_w + kw
                    if 0 <= iy < h and 0 <= ix < w:
                        out[oy, ox, kh, kw] = x[iy, ix]
    return out


def one_by_one(d):
    """The 1x1 descriptor of the baseline GEMMs over X'."""
    return mx.desc(d.n, d.k_h * d.k_w * d.c_in, d.c_out, d.h_out, d.w_out, 1, 1, elem_fmt=d.elem_fmt)


@pytest.mark.parametrize("shape", IM2COL_SHAPES)
def test_im2col_cbf_exact(shape):
    say("im2col", shape)
    lay = WL.ConvLayer(*shape)
    d = mx.desc_from_layer(lay, mx.MX_E2M1)
    x = WL.gen_x(lay, "normal", 31)
    xc = torch.full((d.h_out, d.w_out, d.k_h, d.k_w, d.c_in, d.n), float("nan"), device=DEV)
    mx.mx_im2col_cbf(d, x.to(DEV), xc)
    torch.cuda.synchronize()
    ref = host_im2col(x.numpy(), d)
    assert np.array_equal(xc.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("fmt", [mx.MX_E2M1, mx.MX_E2M3, mx.MX_E4M3])
def test_quantize_after_im2col_repeats_the_single_quantization(fmt):
    # 3x3, stride 1, pad 1: every element of X appears in X', so amax(X') = amax(X)
    lay = WL.ConvLayer(16, 16, 24, 10, 12, 3, 3, 1, 1, 1, 1)
    say("quantize after im2col", fmt)
    d = mx.desc_from_layer(lay, fmt)
    d1 = one_by_one(d)
    x = WL.gen_x(lay, "normal", 41)
    qx = gpu_quantize(d, mx.MX_ROLE_ACT, x)
    xc = torch.empty(d.h_out, d.w_out, d.k_h, d.k_w, d.c_in, d.n, device=DEV)
    mx.mx_im2col_cbf(d, x.to(DEV), xc)
    qxc = mx.QTensor(d1, mx.MX_ROLE_ACT, DEV)
    mx.mx_quantize_cbf(d1, mx.MX_ROLE_ACT, xc, qxc)
    torch.cuda.synchronize()
    assert torch.equal(qx.tensor_scale.view(torch.int32), qxc.tensor_scale.view(torch.int32))
    bb = {mx.MX_E2M1: 32, mx.MX_E2M3: 48, mx.MX_E4M3: 64}[fmt]
    cb, nb = d.c_in // 8, d.n // 8
    codes = qx.codes[:qx.code_bytes].cpu().numpy().reshape(d.h, d.w, cb, nb, bb)
    scales = qx.scales[:qx.nblocks].cpu().numpy().reshape(d.h, d.w, cb, nb)
    ccodes = qxc.codes[:qxc.code_bytes].cpu().numpy().reshape(d.h_out, d.w_out, d.k_h, d.k_w, cb, nb, bb)
    cscales = qxc.scales[:qxc.nblocks].cpu().numpy().reshape(d.h_out, d.w_out, d.k_h, d.k_w, cb, nb)
    for oy in range(d.h_out):
        for ox in range(d.w_out):
            for kh in range(3):
                for kw in range(3):
                    iy, ix = oy - 1 + kh, ox - 1 + kw
                    if 0 <= iy < d.h and 0 <= ix < d.w:
                        assert np.array_equal(ccodes[oy, ox, kh, kw], codes[iy, ix])
                        assert np.array_equal(cscales[oy, ox, kh, kw], scales[iy, ix])
                    else:
                        assert not cscales[oy, ox, kh, kw].any()


def test_baseline_gemms_meet_the_oracle_bound():
    lay = WL.ConvLayer(16, 16, 24, 10, 12, 3, 3, 1, 1, 1, 1)
    say("baseline GEMMs")
    d = mx.desc_from_layer(lay, mx.MX_E2M1)
    d1 = one_by_one(d)
    x, w, dy = WL.gen_x(lay, "normal", 51), WL.gen_w(lay, 52), WL.gen_dy(lay, 1.0, 53)
    # W' [C_out][(kh, kw, ci)][1][1]: the same elements, so the same quantized values
    w1 = w.permute(0, 2, 3, 1).reshape(d.c_out, d1.c_in, 1, 1).contiguous()
    xc = torch.empty(d.h_out, d.w_out, d.k_h, d.k_w, d.c_in, d.n, device=DEV)
    mx.mx_im2col_cbf(d, x.to(DEV), xc)
    qxc = mx.QTensor(d1, mx.MX_ROLE_ACT, DEV)
    mx.mx_quantize_cbf(d1, mx.MX_ROLE_ACT, xc, qxc)
    qw1 = gpu_quantize(d1, mx.MX_ROLE_WEIGHT, w1)
    qdy = gpu_quantize(d1, mx.MX_ROLE_GRAD, dy, mx.MX_SR, 7)
    y = torch.empty(d.h_out, d.w_out, d.c_out, d.n, device=DEV)
    dw1 = torch.empty(d.c_out, d1.c_in, 1, 1, device=DEV)
    ws = torch.empty(max(mx.mx_wgrad_workspace_bytes(d1) // 4, 4), device=DEV)
    mx.mx_conv_fwd(d1, qw1, qxc, y)
    mx.mx_conv_wgrad(d1, qdy, qxc, dw1, ws)
    torch.cuda.synchronize()
    # the oracle on the original layer (MicroQonv's single quantization)
    ox = O.quantize(O.ACT, d.elem_fmt, x.numpy())
    ow = O.quantize(O.WEIGHT, d.elem_fmt, w.numpy())
    ody = O.quantize(O.GRAD, d.elem_fmt, dy.numpy(), O.SR, 7)
    cv = oracle_conv(d)
    ref, s = O.conv_fwd(cv, ow.exact(), ox.exact())
    assert_close(y.cpu().numpy(), ref, s, "baseline fwd")
    ref, s = O.conv_wgrad(cv, ody.exact(), ox.exact())
    dw = dw1.reshape(d.c_out, d.k_h, d.k_w, d.c_in).permute(0, 3, 1, 2).cpu().numpy()
    assert_close(dw, ref, s, "baseline wgrad")
