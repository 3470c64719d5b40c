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


# the layers whose kernels the timed bench steps capture: a mid-sized layer;
# the first ResNet-32 layer (W small enough for the one-launch quantizer,
# small-tile GEMMs, split-K reduce); a 256-channel layer on the 256x256
# decode-at-read tiles; the E8M0 32x32-block format on the scaled MFMA
LAYERS = [
    ((32, 32, 64, 12, 12, 3, 3, 1, 1, 1, 1), 8),
    ((128, 16, 16, 32, 32, 3, 3, 1, 1, 1, 1), 8),
    ((64, 256, 256, 14, 14, 3, 3, 1, 1, 1, 1), 8),
    ((64, 64, 64, 12, 12, 3, 3, 1, 1, 1, 1), 32),
]


@pytest.mark.parametrize("shape,block", LAYERS, ids=["mid", "resnet32-first", "c256", "e8m0"])
def test_layer_graph_replays_match_eager(shape, block):
    lay = WL.ConvLayer(*shape)
    d = mx.desc_from_layer(lay, mx.MX_E2M1, block=block)
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
    if block == 32:  # no tensor amax in the E8M0 format: not written
        outs, names = outs[:-1], names[:-1]

    def layer(stream):
        mx.mx_quantize_cbf(d, 0, x, qx, stream=stream)
        mx.mx_quantize_cbf(d, 1, w, qw, stream=stream)
        mx.mx_quantize_cbf(d, 2, dy, qdy, mx.MX_SR, 99, stream=stream)
        mx.mx_conv_fwd(d, qw, qx, y, stream=stream)
        mx.mx_conv_dgrad(d, qw, qdy, dx, stream=stream)
        mx.mx_conv_wgrad(d, qdy, qx, dw, ws, stream=stream)
        mx.mx_dequantize(d, 0, qx, xdq, stream=stream)

    say("graph: eager reference", shape, block)
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


def test_layer_dag_on_three_streams_matches_serial():
    # the schedule bench.py times: within a layer the three quantizations
    # run on three streams, then fwd (X, W), dgrad (W, dY) and wgrad (dY, X)
    # on the streams of their first operand, each after the quantizations it
    # reads; captured into one graph and replayed against the serial results
    lay = WL.ConvLayer(128, 16, 16, 32, 32, 3, 3, 1, 1, 1, 1)
    d = mx.desc_from_layer(lay, mx.MX_E2M1)
    x = WL.gen_x(lay, "normal", 4).to(DEV)
    w = WL.gen_w(lay, 5).to(DEV)
    dy = WL.gen_dy(lay, 1.0, 6).to(DEV)
    qx, qw, qdy = (mx.QTensor(d, r, DEV) for r in (0, 1, 2))
    y, dx, dw, ws = conv_buffers(d)
    xdq = torch.empty_like(x)
    outs = (y, dx, dw, xdq, qx.codes, qw.codes, qdy.codes)
    say("graph dag: serial reference")
    s0 = torch.cuda.Stream()
    with torch.cuda.stream(s0):
        mx.mx_quantize_cbf(d, 0, x, qx, stream=s0)
        mx.mx_quantize_cbf(d, 1, w, qw, stream=s0)
        mx.mx_quantize_cbf(d, 2, dy, qdy, mx.MX_SR, 7, stream=s0)
        mx.mx_conv_fwd(d, qw, qx, y, stream=s0)
        mx.mx_conv_dgrad(d, qw, qdy, dx, stream=s0)
        mx.mx_conv_wgrad(d, qdy, qx, dw, ws, stream=s0)
        mx.mx_dequantize(d, 0, qx, xdq, stream=s0)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    ev = [torch.cuda.Event() for _ in range(6)]

    def dag():
        fork, ex, ew, edy, j1, j2 = ev
        fork.record(s0)
        s1.wait_event(fork)
        s2.wait_event(fork)
        mx.mx_quantize_cbf(d, 0, x, qx, stream=s0)
        ex.record(s0)
        mx.mx_quantize_cbf(d, 1, w, qw, stream=s1)
        ew.record(s1)
        mx.mx_quantize_cbf(d, 2, dy, qdy, mx.MX_SR, 7, stream=s2)
        edy.record(s2)
        s0.wait_event(ew)
        mx.mx_conv_fwd(d, qw, qx, y, stream=s0)
        s1.wait_event(edy)
        mx.mx_conv_dgrad(d, qw, qdy, dx, stream=s1)
        s2.wait_event(ex)
        mx.mx_conv_wgrad(d, qdy, qx, dw, ws, stream=s2)
        mx.mx_dequantize(d, 0, qx, xdq, stream=s0)
        j1.record(s1)
        j2.record(s2)
        s0.wait_event(j1)
        s0.wait_event(j2)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s0):
        with torch.cuda.graph(g, stream=s0):
            dag()
    torch.cuda.synchronize()
    for rep in range(4):
        say("graph dag replay", rep)
        for t in outs:
            t.fill_(float("nan")) if t.dtype == torch.float32 else t.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for r, t in zip(ref, outs):
            assert torch.equal(r, t), f"replay {rep}"
        z = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        assert torch.isfinite(z)
