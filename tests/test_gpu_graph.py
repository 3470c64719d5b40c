"""The entry points allocate nothing and only enqueue kernels, so a whole layer
(quantize X, W, dY; fwd; dgrad; wgrad; dequantize) can be captured in a HIP
graph.  The graph is replayed several times with eager work and
synchronizations in between, and every replay must reproduce the eager
results bit for bit."""
import pytest
import torch

import microscaling_quantized_convolution_mx_amd as mx
from microscaling_quantized_convolution_mx_amd import workloads as WL
from gpu_util import DEV, conv_buffers, say

pytestmark = pytest.mark.gpu


def test_layer_graph_replays_match_eager():
    lay = WL.ConvLayer(32, 32, 64, 12, 12, 3, 3, 1, 1, 1, 1)
    d = mx.desc_from_layer(lay, mx.MX_E2M1)
    x = WL.gen_x(lay, "normal", 1).to(DEV)
    w = WL.gen_w(lay, 2).to(DEV)
    dy = WL.gen_dy(lay, 1.0, 3).to(DEV)
    qx, qw, qdy = (mx.QTensor(d, r, DEV) for r in (0, 1, 2))
    y, dx, dw, ws = conv_buffers(d)
    xdq = torch.empty_like(x)
    # the stored results only: the scales buffers continue with the
    # quantizer's scratch, whose unused bytes are not results
    outs = (y, dx, dw, xdq, qx.codes, qdy.codes, qw.scales[:qw.nblocks], qdy.scales[:qdy.nblocks],
            qx.tensor_scale, qx.amax)
    names = ("y", "dx", "dw", "xdq", "x codes", "dy codes", "w scales", "dy scales", "x T", "x amax")

    def layer(stream):
        mx.mx_quantize_cbf(d, 0, x, qx, stream=stream)
        mx.mx_quantize_cbf(d, 1, w, qw, stream=stream)
        mx.mx_quantize_cbf(d, 2, dy, qdy, mx.MX_SR, 99, stream=stream)
        mx.mx_conv_fwd(d, qw, qx, y, stream=stream)
        mx.mx_conv_dgrad(d, qw, qdy, dx, stream=stream)
        mx.mx_conv_wgrad(d, qdy, qx, dw, ws, stream=stream)
        mx.mx_dequantize(d, 0, qx, xdq, stream=stream)

    say("graph: eager reference")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        layer(s)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            layer(s)
    torch.cuda.synchronize()
    for rep in range(4):
        say("graph replay", rep)
        for t in outs:
            t.fill_(float("nan")) if t.dtype == torch.float32 else t.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for r, t, nm in zip(ref, outs, names):
            assert torch.equal(r, t), f"replay {rep}: {nm}"
        # eager work between replays
        z = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        assert torch.isfinite(z)
