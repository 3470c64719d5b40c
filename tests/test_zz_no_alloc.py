"""mx_conv_wgrad_noalloc: the weight gradient for callers that cannot
allocate, with its split partials in the library's static per-GPU array.

Checked through the C ABI against mx_conv_wgrad (caller workspace) on the
same quantized inputs: the two use the same kernels, split plan and
reduction order, so the results must be identical bit for bit, and both
within the oracle's bound (2e-3 * sum|a*b|, MicroQonv §IV-B weight gradient).
Two calls in a row, the second on a smaller layer, show that the array
keeps nothing between calls that could change a result.  A layer whose
workspace exceeds the array is rejected before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import microscaling_quantized_convolution_mx_amd as mx
import oracle as O
from microscaling_quantized_convolution_mx_amd import workloads as WL
from gpu_util import DEV, assert_close, conv_buffers, gpu_quantize, oracle_conv, oracle_quantize, say

pytestmark = pytest.mark.gpu


def run_both(lay, fmt, seed):
    d = mx.desc_from_layer(lay, fmt)
    x = WL.gen_x(lay, "normal", seed)
    dy = WL.gen_dy(lay, 1.0, seed + 1)
    qx = gpu_quantize(d, mx.MX_ROLE_ACT, x)
    qdy = gpu_quantize(d, mx.MX_ROLE_GRAD, dy, mx.MX_SR, seed + 2)
    _, _, dw_ref, ws = conv_buffers(d)
    dw = torch.full_like(dw_ref, float("nan"))
    assert mx.mx_wgrad_workspace_bytes(d) <= mx.NOALLOC_SCRATCH_BYTES
    mx.mx_conv_wgrad(d, qdy, qx, dw_ref, ws)
    L = mx.lib()
    rc = L.mx_conv_wgrad_noalloc(ctypes.byref(d), ctypes.byref(qdy.c()), ctypes.byref(qx.c()), dw.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream)
    assert rc == 0, mx.status_str(rc)
    torch.cuda.synchronize()
    return d, x, dy, dw, dw_ref



def test_noalloc_wgrad_two_calls():
    # first the stress layer's shape with a smaller batch (many splits, the
    # 256x256 E2M1 tile), then a smaller ragged layer on the generic tile
    cases = [(WL.ConvLayer(64, 256, 256, 28, 28, 3, 3, 1, 1, 1, 1), mx.MX_E2M1, 300),
             (WL.ConvLayer(16, 24, 40, 9, 7, 3, 3, 2, 2, 1, 1), mx.MX_E4M3, 310)]
    for lay, fmt, seed in cases:
        say("noalloc wgrad", lay.tag(), fmt)
        d, x, dy, dw, dw_ref = run_both(lay, fmt, seed)
        assert bool(torch.isfinite(dw).all())
        assert torch.equal(dw.view(torch.int32), dw_ref.view(torch.int32)), "differs from mx_conv_wgrad"
        ox = oracle_quantize(d, mx.MX_ROLE_ACT, x)
        ody = oracle_quantize(d, mx.MX_ROLE_GRAD, dy, mx.MX_SR, seed + 2)
        cv = oracle_conv(d)
        n = dw.numel()
        idx = np.unique(np.concatenate([np.random.default_rng(seed).integers(0, n, 512), [0, n - 1]])).astype(np.int64)
        ref, s = O.conv_wgrad_points(cv, ody.exact(), ox.exact(), idx)
        assert_close(dw.view(-1)[torch.from_numpy(idx).to(DEV)].cpu().numpy(), ref, s, "noalloc wgrad")


def test_noalloc_rejects_layers_beyond_the_array():
    # a layer whose split partials exceed the static array: rejected on the
    # host (MX_ERR_WORKSPACE), nothing enqueued
    big = None
    for c in (512, 1024, 2048):
        d = mx.desc(256, c, c, 14, 14, 3, 3, pad_h=1, pad_w=1)
        if mx.mx_wgrad_workspace_bytes(d) > mx.NOALLOC_SCRATCH_BYTES:
            big = d
            break
    assert big is not None
    q = mx.mx_qtensor(256, 256, 256, 256)  # aligned stand-ins: never dereferenced
    rc = mx.lib().mx_conv_wgrad_noalloc(ctypes.byref(big), ctypes.byref(q), ctypes.byref(q), 256, None)
    assert rc == -6
