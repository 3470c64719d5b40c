"""Benchmark of the MicroQonv microscaling convolution hot path on one MI355X.

One step = one pass of the whole hot path over one batch of the workload:
for every quantized conv layer of the stack
  S1+S2  quantize X (activation, RNE), W (weight, RNE), dY (gradient, SR)
  S4     forward          Y  = W . im2col(Xq)
  S5     data gradient    dX = col2im(Wq^T . dYq)
  S6     weight gradient  dW = dYq . im2col(Xq)^T
  S7     dequantize Xq (fake-quantized fp32 activation)
and, for the workload that has one, S8: the latent-replay buffer quantized
(S1+S2) and dequantized (S7).  Inputs are seeded synthetic tensors already
resident in device memory when the timed region starts.

value = sum of the dense fwd+dgrad+wgrad flops of all layers / step time
(quantization and dequantization time included in the step time).

Prints one JSON line (see the keys below).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12                    # bytes/s, MI355X HBM3E
PEAK_MFMA = {"bf16": 2.5e15, "f16": 2.5e15, "fp4": 10.1e15}  # dense flop/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c5",
                    help="c1..c5 (default c5: the 256-channel stress layer in its three element formats, "
                         "plus the replay buffer)")
    ap.add_argument("--fmt", default=None, help="element format override: e2m1|e2m3|e4m3")
    ap.add_argument("--act-fmt", default=None, choices=["e3m2", "e2m3"],
                    help="MicroQonv+: activations in this FP6 format, weights and gradients in the "
                         "element format (E2M1)")
    ap.add_argument("--block", type=int, default=8, choices=[8, 32],
                    help="8: E4M3 scale per 8x8 block + fp32 tensor scale; 32: E8M0 scale per 32x32 block "
                         "(original microscaling, E2M1, scaled FP4 MFMA)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate budget of the CPU-baseline sample")
    ap.add_argument("--producer-amax", action="store_true",
                    help="chain the stack: where a layer's input has the previous layer's output shape, X is that "
                         "output, quantized in one pass with the amax its fwd produced (mx_conv_fwd_amax)")
    ap.add_argument("--flow", default=None, choices=["microqonv", "im2col-square", "dacapo"],
                    help="time only the activation path (fwd + wgrad) of one flow: MicroQonv's single quantization, "
                         "quantize-after-im2col (X' written and square-quantized once), or DaCapo-style "
                         "(X' formed and quantized again for the backward)")
    ap.add_argument("--replay-compact", action="store_true",
                    help="store the latent-replay buffer in the compact 3-bit codes (MX_UE2M1, 3.125 b/element)")
    ap.add_argument("--eager", action="store_true",
                    help="launch the calls one by one, in order, in the timed region instead of replaying the "
                         "step as one captured HIP graph (the default; per-call timing always comes from an "
                         "eager pass)")
    ap.add_argument("--graph", action="store_true", help="the default; kept for old command lines")
    ap.add_argument("--serial", action="store_true",
                    help="issue every call on one stream, in order (default: within a layer, the three "
                         "quantizations and then fwd / dgrad / wgrad run on three streams, each call after "
                         "the quantizations it reads; layers stay in order)")
    ap.add_argument("--copy-calib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--library-gemm", action="store_true",
                    help="only time the vendor dense GEMM (torch.matmul: hipBLASLt) in fp16 and bf16 on the "
                         "workload's first layer's three GEMM shapes and on 8192^3, as context for the MX GEMMs "
                         "(same flops, 16-bit operands, no decode, no gather)")
    ap.add_argument("--verbose", action="store_true")
    return ap.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "microscaling_quantized_convolution_mx_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


class Call:
    """One prepared C-ABI call: the function and its ctypes arguments are
    built once, so that the timed loop only pays for the call itself."""

    __slots__ = ("fn", "args", "op", "group", "flops", "bytes", "name")

    def __init__(self, fn, args, op, group, flops, nbytes, name):
        self.fn, self.args, self.op, self.group = fn, args, op, group
        self.flops, self.bytes, self.name = flops, nbytes, name

    def __call__(self):
        rc = self.fn(*self.args)
        if rc != 0:
            raise RuntimeError(f"{self.name}: status {rc}")


def flow_calls(flow, L, mx, torch, D, d, lay, x, w, dy, sr_seed, fmt, fname, qb, stream, keep, dev):
    """The activation path (fwd + wgrad) of one layer under one flow.  W and dY
    are quantized here, outside the timed step (they are the same in every
    flow).  The baseline flows run the GEMMs as 1x1 convolutions over X'
    [Ho][Wo][(Kh, Kw, C)][N] (mx_im2col_cbf)."""
    shape = lay.tag()
    nx, nw, ny = lay.numel_x(), lay.numel_w(), lay.numel_dy()
    f = lay.flops()
    if flow == "microqonv":
        g, xs = d, x
    else:
        g = mx.desc(d.n, d.k_h * d.k_w * d.c_in, d.c_out, d.h_out, d.w_out, 1, 1, elem_fmt=fmt)
        w = w.permute(0, 2, 3, 1).reshape(d.c_out, g.c_in, 1, 1).contiguous()
        xs = torch.empty(d.h_out, d.w_out, d.k_h, d.k_w, d.c_in, d.n, device=dev)
    qx, qw, qdy = (mx.QTensor(g, r, dev) for r in (mx.MX_ROLE_ACT, mx.MX_ROLE_WEIGHT, mx.MX_ROLE_GRAD))
    mx.mx_quantize_cbf(g, mx.MX_ROLE_WEIGHT, w, qw)
    mx.mx_quantize_cbf(g, mx.MX_ROLE_GRAD, dy, qdy, mx.MX_SR, sr_seed)
    y = torch.empty(lay.h_out, lay.w_out, lay.c_out, lay.n, device=dev)
    dw = torch.empty(g.c_out, g.c_in, g.k_h, g.k_w, device=dev)
    wsb = mx.mx_wgrad_workspace_bytes(g)
    wsf = torch.empty(max(wsb // 4, 4), device=dev)
    cq = [q.c() for q in (qx, qw, qdy)]
    keep += [g, w, xs, qx, qw, qdy, y, dw, wsf, cq]
    nxc = xs.numel() if flow != "microqonv" else nx
    q_x = Call(L.mx_quantize_cbf, (D(g), mx.MX_ROLE_ACT, xs.data_ptr(), D(cq[0]), mx.MX_RNE, 0, 0, stream),
               "quantize", ("quantize_act", shape, fname), 0, nxc * (8 + qb), "quantize X" if flow == "microqonv" else "quantize X'")
    fwd = Call(L.mx_conv_fwd, (D(g), D(cq[1]), D(cq[0]), y.data_ptr(), stream),
               "fwd", ("conv_fwd", shape, fname), f, (nw + nxc) * qb + 4 * ny, "fwd")
    wgrad = Call(L.mx_conv_wgrad, (D(g), D(cq[2]), D(cq[0]), dw.data_ptr(), wsf.data_ptr(), wsb, stream),
                 "wgrad", ("conv_wgrad", shape, fname), f, (ny + nxc) * qb + 4 * nw, "wgrad")
    if flow == "microqonv":
        return [q_x, fwd, wgrad]

    def im2col():
        return Call(L.mx_im2col_cbf, (D(d), x.data_ptr(), xs.data_ptr(), stream),
                    "im2col", ("im2col", shape, fname), 0, 4 * (nx + nxc), "im2col")
    if flow == "im2col-square":
        return [im2col(), q_x, fwd, wgrad]
    # dacapo: X kept in fp32; X' formed and quantized in the forward and again in the backward
    q_x2 = Call(q_x.fn, q_x.args, "quantize", ("quantize_act", shape, fname), 0, nxc * (8 + qb), "quantize X' (backward)")
    return [im2col(), q_x, fwd, im2col(), q_x2, wgrad]


def fmt_list(a, wl, mx):
    """Element formats of one step: all of the workload's (the stress layer
    runs E2M1, E2M3 and E4M3), or the one --fmt names.  The variants
    (--block 32, --act-fmt, --flow, --producer-amax) run one format."""
    names = {"e2m1": mx.MX_E2M1, "e2m3": mx.MX_E2M3, "e4m3": mx.MX_E4M3, "e3m2": mx.MX_E3M2}
    if a.fmt:
        return [names[a.fmt]]
    if a.block == 32 or a.act_fmt or a.flow or a.producer_amax:
        return [wl.elem_fmts[0]]
    return list(wl.elem_fmts)


def mfma_dtype(block, fmt, mx):
    """Operand type of the GEMMs' MFMA: fp4 (scaled, 32x32 E8M0 blocks), else
    the exact decode to fp16 (E4M3 with a 2^-2 exponent shift on the 256x256
    tile; its smaller tiles decode to bf16, at the same dense peak)."""
    return "fp4" if block == 32 else "f16"


def library_gemm(a, torch, dev, WL):
    """Dense 16-bit GEMM rates of the vendor library on the MX GEMMs' shapes:
    fwd C_out x (N Ho Wo) x (C_in Kh Kw), wgrad C_out x (C_in Kh Kw) x (N Ho Wo),
    and a square 8192 GEMM.  One JSON line per case."""
    lay = WL.workloads()[a.workload].layers[0]
    cols = lay.n * lay.h_out * lay.w_out
    kk = lay.c_in * lay.k_h * lay.k_w
    cases = [("square", 8192, 8192, 8192), ("fwd", lay.c_out, cols, kk), ("wgrad", lay.c_out, kk, cols)]
    for dt in (torch.float16, torch.bfloat16):
        for name, m, n, k in cases:
            x = torch.randn(m, k, device=dev, dtype=dt)
            y = torch.randn(k, n, device=dev, dtype=dt)
            for _ in range(3):
                z = torch.matmul(x, y)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 10
            e0.record()
            for _ in range(reps):
                z = torch.matmul(x, y)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            tf = 2.0 * m * n * k / (us * 1e-6) / 1e12
            print(json.dumps({"library_gemm": name, "dtype": str(dt).replace("torch.", ""), "m": m, "n": n, "k": k,
                              "us": round(us, 1), "tflops": round(tf, 1), "frac_of_2p5_pflops": round(tf / 2500, 4)}),
                  flush=True)
            del x, y, z
            torch.cuda.empty_cache()


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU: the hot path is the single-GPU "
                                   "kernel set (multi-GPU sharding is a design note only); "
                                   "run with --gpus 1"}))
        sys.exit(2)

    import torch
    import microscaling_quantized_convolution_mx_amd as mx
    from microscaling_quantized_convolution_mx_amd import workloads as WL

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if a.library_gemm:
        library_gemm(a, torch, dev, WL)
        return

    if a.copy_calib:
        n = a.copy_calib * (1 << 20) // 4
        src = torch.ones(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes_each_way": n * 4, "launches": 3}))
        return

    L = mx.lib()
    wl = WL.workloads()[a.workload]
    fmts_by_name = {"e2m1": mx.MX_E2M1, "e2m3": mx.MX_E2M3, "e4m3": mx.MX_E4M3, "e3m2": mx.MX_E3M2}
    fmts = fmt_list(a, wl, mx)
    afmt = fmts_by_name[a.act_fmt] if a.act_fmt else 0   # 0: activations in the element format too
    if afmt and a.flow:
        raise SystemExit("--act-fmt applies to the MicroQonv step, not to --flow")
    if a.block == 32 and (afmt or a.flow or a.producer_amax or fmts != [mx.MX_E2M1]):
        raise SystemExit("--block 32 runs the E2M1 MicroQonv step only")
    sb = 1 / (a.block * a.block)                   # scale bytes per element
    rd = 8 if a.block == 8 else 4                  # fp32 source bytes read per element: amax pass + pass, or once
    stream = torch.cuda.current_stream().cuda_stream

    D = ctypes.byref
    calls: list[Call] = []
    keep = []                         # keeps every buffer and ctypes struct alive
    ws_bytes = max(mx.mx_wgrad_workspace_bytes(mx.desc_from_layer(l, f, afmt, a.block))
                   for l in wl.layers for f in fmts)
    ws = torch.empty(max(ws_bytes // 4, 4), device=dev)
    keep.append(ws)

    t_gen = time.time()
    inputs = {}  # layer index -> (x, w, dy) on the device, shared by the formats
    flow_stats = {"activation_elements": 0, "quantized_elements": 0, "stored_activation_bytes": 0.0}
    n_chained = 0
    layer_starts = []  # index of each (format, layer)'s first call (the 7-call MicroQonv step)
    for fmt in fmts:
        fname = WL.FMT_NAMES[fmt]
        qb = mx.CODE_BITS[fmt] / 8 + sb                # quantized bytes per element (codes + block scales)
        qbx = mx.CODE_BITS[afmt or fmt] / 8 + sb       # the same for the activation X
        prev = None  # --producer-amax: (descriptor, y, fwd Call) of the previous layer
        for li, lay in enumerate(wl.layers):
            d = mx.desc_from_layer(lay, fmt, afmt, a.block)
            if li not in inputs:
                inputs[li] = (WL.gen_x(lay, wl.x_dist, WL.seed_for(wl.cfg_index, li, 1)).to(dev),
                              WL.gen_w(lay, WL.seed_for(wl.cfg_index, li, 2)).to(dev),
                              WL.gen_dy(lay, wl.dy_sigma, WL.seed_for(wl.cfg_index, li, 3)).to(dev))
            x, w, dy = inputs[li]
            sr_seed = WL.seed_for(wl.cfg_index, li, 4)
            shape = lay.tag()
            nx, nw, ny = lay.numel_x(), lay.numel_w(), lay.numel_dy()
            f = lay.flops()
            if a.flow:
                calls += flow_calls(a.flow, L, mx, torch, D, d, lay, x, w, dy, sr_seed, fmt, fname, qb, stream, keep, dev)
                nxc = lay.h_out * lay.w_out * lay.k_h * lay.k_w * lay.c_in * lay.n
                flow_stats["activation_elements"] += nx
                flow_stats["quantized_elements"] += {"microqonv": nx, "im2col-square": nxc, "dacapo": 2 * nxc}[a.flow]
                flow_stats["stored_activation_bytes"] += {"microqonv": nx * qb, "im2col-square": nxc * qb,
                                                          "dacapo": nx * 4.0}[a.flow]
                continue
            qx, qw, qdy = (mx.QTensor(d, r, dev) for r in (mx.MX_ROLE_ACT, mx.MX_ROLE_WEIGHT, mx.MX_ROLE_GRAD))
            y = torch.empty(lay.h_out, lay.w_out, lay.c_out, lay.n, device=dev)
            dx = torch.empty(lay.h, lay.w, lay.c_in, lay.n, device=dev)
            dw = torch.empty(lay.c_out, lay.c_in, lay.k_h, lay.k_w, device=dev)
            xdq = torch.empty_like(x)
            cq = [q.c() for q in (qx, qw, qdy)]
            keep += [d, qx, qw, qdy, y, dx, dw, xdq, cq]
            # --producer-amax: where the previous layer's output has this
            # layer's input shape, X is that output, its fwd writes max|y|
            # into qx.amax and X is quantized in one pass (amax given)
            chained = (a.producer_amax and prev is not None
                       and (prev[0].h_out, prev[0].w_out, prev[0].c_out, prev[0].n) == (lay.h, lay.w, lay.c_in, lay.n))
            if chained:
                pd, py, pcall = prev
                # the previous fwd's amax buffer: word 0 is the amax this layer's X is quantized with
                abuf = torch.empty(mx.mx_fwd_amax_bytes(pd) // 4, device=dev)
                keep.append(abuf)
                qx.amax = abuf[:1]
                cq[0] = qx.c()
                pcall.fn = L.mx_conv_fwd_amax
                pcall.args = pcall.args[:-1] + (abuf.data_ptr(), stream)
                pcall.name = "fwd (+amax)"
                x_src, x_given, x_bytes = py.data_ptr(), 1, nx * (4 + qbx)
                n_chained += 1
            else:
                x_src, x_given, x_bytes = x.data_ptr(), 0, nx * (rd + qbx)
            calls += [
                Call(L.mx_quantize_cbf, (D(d), mx.MX_ROLE_ACT, x_src, D(cq[0]), mx.MX_RNE, 0, x_given, stream),
                     "quantize", ("quantize_act", shape, fname), 0, x_bytes, "quantize X"),
                Call(L.mx_quantize_cbf, (D(d), mx.MX_ROLE_WEIGHT, w.data_ptr(), D(cq[1]), mx.MX_RNE, 0, 0, stream),
                     "quantize", ("quantize_weight", shape, fname), 0, nw * (rd + qb), "quantize W"),
                Call(L.mx_quantize_cbf, (D(d), mx.MX_ROLE_GRAD, dy.data_ptr(), D(cq[2]), mx.MX_SR, sr_seed, 0,
                                         stream),
                     "quantize", ("quantize_grad", shape, fname), 0, ny * (rd + qb), "quantize dY"),
                Call(L.mx_conv_fwd, (D(d), D(cq[1]), D(cq[0]), y.data_ptr(), stream),
                     "fwd", ("conv_fwd", shape, fname), f, nw * qb + nx * qbx + 4 * ny, "fwd"),
                Call(L.mx_conv_dgrad, (D(d), D(cq[1]), D(cq[2]), dx.data_ptr(), stream),
                     "dgrad", ("conv_dgrad", shape, fname), f, (nw + ny) * qb + 4 * nx, "dgrad"),
                Call(L.mx_conv_wgrad, (D(d), D(cq[2]), D(cq[0]), dw.data_ptr(), ws.data_ptr(), ws_bytes, stream),
                     "wgrad", ("conv_wgrad", shape, fname), f, ny * qb + nx * qbx + 4 * nw, "wgrad"),
                Call(L.mx_dequantize, (D(d), mx.MX_ROLE_ACT, D(cq[0]), xdq.data_ptr(), stream),
                     "dequantize", ("dequantize_act", shape, fname), 0, nx * (qbx + 4), "dequantize X"),
            ]
            prev = (d, y, calls[-4])
            layer_starts.append(len(calls) - 7)
    keep.append(inputs)
    if wl.lr_buffer is not None and not a.flow:
        nmaps, c, h, w_ = wl.lr_buffer
        lr_fmt = mx.MX_UE2M1 if a.replay_compact else mx.MX_E2M1
        d = mx.desc(nmaps, c, c, h, w_, 1, 1, elem_fmt=lr_fmt)
        maps = WL.gen_lr_maps(nmaps, c, h, w_, WL.seed_for(wl.cfg_index, 0, 5)).to(dev)
        q = mx.QTensor(d, mx.MX_ROLE_ACT, dev)
        back = torch.empty_like(maps)
        cq = q.c()
        keep += [d, maps, q, back, cq]
        n_el = maps.numel()
        qb4 = (3 if a.replay_compact else 4) / 8 + 1 / 64
        shape = f"replay buffer {nmaps}x{c}@{h}x{w_}"
        lrn = "ue2m1" if a.replay_compact else "e2m1"
        calls += [
            Call(L.mx_quantize_cbf, (D(d), mx.MX_ROLE_ACT, maps.data_ptr(), D(cq), mx.MX_RNE, 0, 0, stream),
                 "quantize", ("quantize_replay", shape, lrn), 0, n_el * (8 + qb4), "quantize replay buffer"),
            Call(L.mx_dequantize, (D(d), mx.MX_ROLE_ACT, D(cq), back.data_ptr(), stream),
                 "dequantize", ("dequantize_replay", shape, lrn), 0, n_el * (qb4 + 4), "dequantize replay buffer"),
        ]
    torch.cuda.synchronize()
    t_gen = time.time() - t_gen

    total_flops = sum(c.flops for c in calls)

    # Layer DAG on three streams (lanes): lane 0 quantizes X, runs fwd and
    # dequantizes X; lane 1 quantizes W and runs dgrad; lane 2 quantizes dY
    # and runs wgrad.  fwd waits for W, dgrad for dY, wgrad for X; each layer
    # (of each format) forks from lane 0 and joins back into it, so layers run
    # in order, as the layers of a network would.  Calls outside the layers
    # (the replay buffer) run on lane 0 after them.  (graph replay only:
    # issued eagerly, the event calls between the launches cost more host
    # time than the overlap saves)
    dag = (not a.serial and not a.eager and not a.flow and n_chained == 0
           and len(layer_starts) == len(wl.layers) * len(fmts))
    LANE = (0, 1, 2, 0, 1, 2, 0)
    lanes = [torch.cuda.current_stream(), torch.cuda.Stream(), torch.cuda.Stream()]
    in_layer = set()
    for st in layer_starts:
        in_layer.update(range(st, st + 7))
    dag_ev = [[torch.cuda.Event() for _ in range(6)] for _ in layer_starts]

    def set_stream(h):
        for c in calls:
            c.args = c.args[:-1] + (h,)

    def set_lanes(main):
        # lane streams: `main` for lane 0 (the stream the step is issued on)
        handles = [main.cuda_stream, lanes[1].cuda_stream, lanes[2].cuda_stream]
        set_stream(main.cuda_stream)
        for st in layer_starts:
            for k in range(7):
                c = calls[st + k]
                c.args = c.args[:-1] + (handles[LANE[k]],)

    def run_step_dag(main):
        l1, l2 = lanes[1], lanes[2]
        for li, st in enumerate(layer_starts):
            fork, ex, ew, edy, j1, j2 = dag_ev[li]
            fork.record(main)
            l1.wait_event(fork)
            l2.wait_event(fork)
            calls[st]()               # quantize X   (lane 0)
            ex.record(main)
            calls[st + 1]()           # quantize W   (lane 1)
            ew.record(l1)
            calls[st + 2]()           # quantize dY  (lane 2)
            edy.record(l2)
            main.wait_event(ew)
            calls[st + 3]()           # fwd: X, W    (lane 0)
            l1.wait_event(edy)
            calls[st + 4]()           # dgrad: W, dY (lane 1)
            l2.wait_event(ex)
            calls[st + 5]()           # wgrad: dY, X (lane 2)
            calls[st + 6]()           # dequantize X (lane 0)
            j1.record(l1)
            j2.record(l2)
            main.wait_event(j1)
            main.wait_event(j2)
        for i, c in enumerate(calls):
            if i not in in_layer:
                c()

    def run_step(events=None, main=None):
        if events is None and dag:
            run_step_dag(main or torch.cuda.current_stream())
        elif events is None:
            for c in calls:
                c()
        else:
            for i, c in enumerate(calls):
                c()
                events[i].record()

    if dag:
        set_lanes(torch.cuda.current_stream())

    for _ in range(a.warmup):
        run_step()
    torch.cuda.synchronize()

    # ---- timed region: K steps, an event after every call
    ev = [[torch.cuda.Event(enable_timing=True) for _ in calls] for _ in range(a.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    graph = None
    if not a.eager:
        # every C-ABI call takes the stream as its last argument
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        if dag:
            set_lanes(s)
        else:
            set_stream(s.cuda_stream)
        with torch.cuda.stream(s):
            run_step(main=s)    # eager pass on the capture stream first
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=s):
                run_step(main=s)
        torch.cuda.current_stream().wait_stream(s)
        if dag:
            set_lanes(torch.cuda.current_stream())
        else:
            set_stream(stream)
        graph = g
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for k in range(a.steps):
        if graph is not None:
            graph.replay()
        elif dag:
            run_step()
        else:
            run_step(ev[k])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / a.steps

    # per-call durations from an eager pass with events, one call at a time on
    # one stream (outside the timed region when the step is a graph or a DAG)
    pstart = None
    if graph is not None or dag:
        set_stream(stream)
        pstart = torch.cuda.Event(enable_timing=True)
        pstart.record()
        for k in range(a.steps):
            run_step(ev[k])
        torch.cuda.synchronize()
    # per-call durations: gap between consecutive events (first call of a step
    # measured from the previous step's last event, or from `start`)
    per_call = [[0.0] * len(calls) for _ in range(a.steps)]
    for k in range(a.steps):
        for i in range(len(calls)):
            if i == 0:
                prev_ev = ev[k - 1][-1] if k > 0 else None
                if prev_ev is None:
                    per_call[k][i] = (pstart or start).elapsed_time(ev[k][0])
                else:
                    per_call[k][i] = prev_ev.elapsed_time(ev[k][0])
            else:
                per_call[k][i] = ev[k][i - 1].elapsed_time(ev[k][i])
    # average over steps (NaN-safe)
    avg_ms = []
    for i in range(len(calls)):
        vals = [per_call[k][i] for k in range(a.steps) if per_call[k][i] == per_call[k][i]]
        avg_ms.append(sum(vals) / len(vals) if vals else float("nan"))

    groups = {}
    for i, c in enumerate(calls):
        gi = groups.setdefault(c.group, {"ms": 0.0, "n": 0, "flops": c.flops, "bytes": c.bytes, "op": c.op})
        gi["ms"] += avg_ms[i]
        gi["n"] += 1
    by_op = {}
    for i, c in enumerate(calls):
        o = by_op.setdefault(c.op, {"ms": 0.0, "flops": 0, "bytes": 0})
        o["ms"] += avg_ms[i]
        o["flops"] += c.flops
        o["bytes"] += c.bytes

    def peak_of(fname):
        return PEAK_MFMA[mfma_dtype(a.block, fmts_by_name.get(fname, mx.MX_E2M1), mx)]

    dom_key, dom = max(groups.items(), key=lambda kv: kv[1]["ms"])
    launch_s = dom["ms"] / dom["n"] / 1e3
    ai = dom["flops"] / dom["bytes"] if dom["bytes"] else 0.0
    dom_peak = peak_of(dom_key[2])
    if dom["flops"] and ai >= dom_peak / PEAK_HBM:
        achieved = dom["flops"] / launch_s
        roof = {"bound": "mfma", "achieved": achieved / 1e12, "peak": dom_peak / 1e12,
                "unit": "TFLOP/s", "mfma_dtype": mfma_dtype(a.block, fmts_by_name.get(dom_key[2]), mx)}
    else:
        achieved = dom["bytes"] / launch_s
        roof = {"bound": "hbm", "achieved": achieved / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel"] = f"{dom_key[0]} [{dom_key[1]}] {dom_key[2]}"
    roof["launch_us"] = launch_s * 1e6
    roof["algorithmic_per_launch"] = {"flops": dom["flops"], "bytes": dom["bytes"]}
    roof["traffic"] = None
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tfile):
        try:
            tr = json.load(open(tfile))
            ent = tr.get("kernels", {}).get(f"{a.workload}:{dom_key[2]}:{dom_key[0]}:{dom_key[1]}")
            if ent and tr.get("source_hash") == kernel_source_hash():
                roof["traffic"] = ent["hbm_bytes_per_launch"]
        except (ValueError, KeyError):
            pass
    roof["ai_flop_per_byte"] = ai

    # every call group (one call of one layer shape in one format), slowest
    # first: GEMMs against the dense MFMA peak and against what the roofline
    # allows at their arithmetic intensity (algorithmic bytes: quantized
    # operands read once, fp32 output written once); codec calls against 8 TB/s
    per_layer = []
    for (gop, tag, fname), g in sorted(groups.items(), key=lambda kv: -kv[1]["ms"]):
        ls = g["ms"] / g["n"] / 1e3
        ent = {"call": gop, "shape": tag, "fmt": fname, "launches": g["n"], "launch_us": round(ls * 1e6, 2)}
        if g["flops"]:
            pk = peak_of(fname)
            att = min(pk, g["flops"] / g["bytes"] * PEAK_HBM) if g["bytes"] else pk
            ach = g["flops"] / ls
            ent.update({"tflops": round(ach / 1e12, 2), "frac_of_peak": round(ach / pk, 4),
                        "attainable_frac_of_peak": round(att / pk, 4), "frac_of_attainable": round(ach / att, 4)})
        else:
            ach = g["bytes"] / ls
            ent.update({"gbps": round(ach / 1e9, 1), "frac_of_hbm": round(ach / PEAK_HBM, 4)})
        per_layer.append(ent)

    # per element format: its GEMM and codec rates and its share of the step
    per_fmt = {}
    for i, c in enumerate(calls):
        pf = per_fmt.setdefault(c.group[2], {"ms": 0.0, "gemm_ms": 0.0, "gemm_flops": 0, "q_ms": 0.0,
                                             "q_bytes": 0.0, "calls_ms": {}})
        pf["ms"] += avg_ms[i]
        pf["calls_ms"][c.group[0]] = pf["calls_ms"].get(c.group[0], 0.0) + avg_ms[i]
        if c.flops:
            pf["gemm_ms"] += avg_ms[i]
            pf["gemm_flops"] += c.flops
        elif c.op == "quantize":
            pf["q_ms"] += avg_ms[i]
            pf["q_bytes"] += c.bytes
    formats = {}
    for fname, pf in per_fmt.items():
        e = {"calls_ms_per_step": {k: round(v, 4) for k, v in pf["calls_ms"].items()},
             "ms_per_step_calls_alone": round(pf["ms"], 4)}
        if pf["gemm_flops"]:
            e["gemm_tflops"] = round(pf["gemm_flops"] / (pf["gemm_ms"] / 1e3) / 1e12, 2)
            e["gemm_frac_of_peak"] = round(pf["gemm_flops"] / (pf["gemm_ms"] / 1e3) / peak_of(fname), 4)
            e["step_tflops_calls_alone"] = round(pf["gemm_flops"] / (pf["ms"] / 1e3) / 1e12, 2)
        if pf["q_ms"]:
            e["quantize_gbps"] = round(pf["q_bytes"] / (pf["q_ms"] / 1e3) / 1e9, 1)
        formats[fname] = e

    conv_ms = sum(by_op.get(o, {"ms": 0.0})["ms"] for o in ("fwd", "dgrad", "wgrad"))
    q_ms = by_op.get("quantize", {"ms": 0.0})["ms"]
    q_bytes = by_op.get("quantize", {"bytes": 0})["bytes"]
    fnames = [WL.FMT_NAMES[f] for f in fmts]
    dtypes = sorted({mfma_dtype(a.block, f, mx) for f in fmts})
    lay0 = wl.layers[0]
    wdesc = f"{a.workload}: {wl.name}"
    if len(fmts) > 1:
        wdesc += ", run in " + " + ".join(n.upper() for n in fnames)
    if wl.lr_buffer is not None and not a.flow:
        wdesc += ", + latent-replay buffer %dx%d@%dx%d codec" % wl.lr_buffer

    result = {
        "metric": "effective TFLOP/s of MX conv fwd+dgrad+wgrad (implicit im2col); quantize GB/s",
        "value": total_flops / (ms_step / 1e3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "+".join(dtypes),
        "data": "synthetic",
        "config": {"workload": wdesc, "layers": len(wl.layers),
                   "batch": lay0.n, "elem_fmts": fnames,
                   **({"act_fmt": a.act_fmt, "variant": "MicroQonv+ (FP6 activations)"} if afmt else {}),
                   "block": "8x8 E4M3 scale + fp32 tensor scale" if a.block == 8
                            else "32x32 E8M0 scale, no tensor scale (scaled FP4 MFMA)",
                   "step": ("per format and layer: quantize X,W,dY; fwd; dgrad; wgrad; dequantize Xq"
                            + ("; then the replay buffer quantize+dequantize" if wl.lr_buffer else "")),
                   "step_flops": total_flops,
                   "graph": bool(graph is not None),
                   "streams": "layer DAG on 3 streams" if dag else "1 (serial)",
                   "producer_amax": {"chained_layers": n_chained} if a.producer_amax else False,
                   **({"replay_buffer_fmt": "ue2m1" if a.replay_compact else "e2m1"} if wl.lr_buffer else {})},
        "conv_tflops": total_flops / (conv_ms / 1e3) / 1e12 if conv_ms > 0 else None,
        "quantize_gbps": q_bytes / (q_ms / 1e3) / 1e9 if q_ms > 0 else None,
        "step_breakdown_ms": {k: v["ms"] for k, v in by_op.items()},
        "formats": formats,
        **({"flow": {"name": a.flow,
                     "quantizations_per_activation_element": flow_stats["quantized_elements"]
                     / max(flow_stats["activation_elements"], 1),
                     "stored_activation_bytes_for_backward": flow_stats["stored_activation_bytes"],
                     "note": "value and conv_tflops count fwd + wgrad only (the activation path)"}}
           if a.flow else {}),
        "roofline": roof,
        "per_layer": per_layer,
        "wall_s_timed": wall,
        "kernel_source": kernel_source_hash(),
    }
    if a.verbose:
        result["groups"] = {f"{k[0]} [{k[1]}] {k[2]}": {"ms_total": v["ms"], "launches": v["n"],
                                                        "flops": v["flops"], "bytes": v["bytes"]}
                            for k, v in sorted(groups.items(), key=lambda kv: -kv[1]["ms"])}

    if not a.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, fmts, afmt, a.cpu_seconds, a.flow is None)
    print(json.dumps(result), flush=True)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, fmts, afmt, budget_s, with_replay=True):
    """The CPU oracle, as it stands, on a bounded sample of the workload,
    reported in the metric's unit (input generation is outside the timed
    region, as it is for the GPU).

    Stacks whose layers the oracle can compute in full within the budget:
    the full quantize X/W/dY + fp64 fwd/dgrad/wgrad of the stack's layers,
    taken in stack order (wrapping round) until the budget is spent.

    A layer too large for that (the 256-channel stress layer: 2.8 TFLOP per
    format): per format, the full quantize of X, W and dY, the fp32
    dequantize of Xq, the fp64 operands of the GEMMs, and each GEMM on a
    seeded sample of outputs, evaluated one by one; the step time is the
    measured time of the full parts plus the sampled GEMM time scaled to all
    outputs (every output of one GEMM costs the same: one dot product over
    its K).  The replay buffer is quantized and dequantized in full."""
    import numpy as np

    import oracle as O
    from microscaling_quantized_convolution_mx_amd import workloads as WL

    O.lib()
    import microscaling_quantized_convolution_mx_amd as mx
    ofmt = {mx.MX_E2M1: O.E2M1, mx.MX_E2M3: O.E2M3, mx.MX_E4M3: O.E4M3, mx.MX_E3M2: O.E3M2}
    threads = O.threads()
    nl = len(wl.layers)
    if max(3 * l.flops() for l in wl.layers) <= 200e9:
        fmt_w = ofmt[fmts[0]]
        fmt_x = ofmt[afmt or fmts[0]]
        flops = 0
        spent = 0.0
        done = 0
        li = 0
        while spent < budget_s and done < 4 * nl:
            lay = wl.layers[li % nl]
            x = WL.gen_x(lay, wl.x_dist, WL.seed_for(wl.cfg_index, li % nl, 1)).numpy()
            w = WL.gen_w(lay, WL.seed_for(wl.cfg_index, li % nl, 2)).numpy()
            dy = WL.gen_dy(lay, wl.dy_sigma, WL.seed_for(wl.cfg_index, li % nl, 3)).numpy()
            cv = O.conv(lay.n, lay.c_in, lay.c_out, lay.h, lay.w, lay.k_h, lay.k_w,
                        lay.stride_h, lay.stride_w, lay.pad_h, lay.pad_w)
            t0 = time.perf_counter()
            qx = O.quantize(O.ACT, fmt_x, x)
            qw = O.quantize(O.WEIGHT, fmt_w, w)
            qdy = O.quantize(O.GRAD, fmt_w, dy, O.SR, WL.seed_for(wl.cfg_index, li % nl, 4))
            xe, we, dye = qx.exact(), qw.exact(), qdy.exact()
            O.conv_fwd(cv, we, xe)
            O.conv_dgrad(cv, we, dye)
            O.conv_wgrad(cv, dye, xe)
            spent += time.perf_counter() - t0
            flops += 3 * lay.flops()
            done += 1
            li += 1
        out = {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
               "cpu_model": cpu_model(), "nproc": os.cpu_count(),
               "sample": f"full quantize X/W/dY + fp64 fwd/dgrad/wgrad of {done} layer(s) of the "
                         f"{nl}-layer stack ({WL.FMT_NAMES[fmts[0]]}) taken in order from the first, "
                         f"{flops / 1e9:.2f} GFLOP in {spent:.1f} s",
               "seconds": spent}
        if nl == 1:
            # the single conv is also timed on one thread (same passes, same inputs)
            try:
                O.set_threads(1)
                t1 = 0.0
                reps = 0
                while t1 < min(budget_s, 5.0) and reps < done:
                    t0 = time.perf_counter()
                    qx = O.quantize(O.ACT, fmt_x, x)
                    qw = O.quantize(O.WEIGHT, fmt_w, w)
                    qdy = O.quantize(O.GRAD, fmt_w, dy, O.SR, WL.seed_for(wl.cfg_index, 0, 4))
                    xe, we, dye = qx.exact(), qw.exact(), qdy.exact()
                    O.conv_fwd(cv, we, xe)
                    O.conv_dgrad(cv, we, dye)
                    O.conv_wgrad(cv, dye, xe)
                    t1 += time.perf_counter() - t0
                    reps += 1
            finally:
                O.set_threads(threads)
            out["single_thread"] = {"value": reps * 3 * wl.layers[0].flops() / t1 / 1e12, "unit": "TFLOP/s",
                                    "cores": 1, "passes": reps, "seconds": t1}
        return out

    # sampled stress layer
    npts = {"fwd": 65536, "dgrad": 65536, "wgrad": 4096}
    measured = 0.0      # seconds actually spent in the oracle
    step_s = 0.0        # the same plus the sampled GEMMs scaled to all outputs
    flops = 0
    q_bytes = 0.0
    q_s = 0.0
    gemm_pts_flops = 0.0
    gemm_pts_s = 0.0
    detail = {}
    rng = np.random.default_rng(12345)
    for fmt in fmts:
        fw, fx = ofmt[fmt], ofmt[afmt or fmt]
        for li, lay in enumerate(wl.layers):
            x = WL.gen_x(lay, wl.x_dist, WL.seed_for(wl.cfg_index, li, 1)).numpy()
            w = WL.gen_w(lay, WL.seed_for(wl.cfg_index, li, 2)).numpy()
            dy = WL.gen_dy(lay, wl.dy_sigma, WL.seed_for(wl.cfg_index, li, 3)).numpy()
            cv = O.conv(lay.n, lay.c_in, lay.c_out, lay.h, lay.w, lay.k_h, lay.k_w,
                        lay.stride_h, lay.stride_w, lay.pad_h, lay.pad_w)
            t = {}
            t0 = time.perf_counter()
            qx = O.quantize(O.ACT, fx, x)
            qw = O.quantize(O.WEIGHT, fw, w)
            qdy = O.quantize(O.GRAD, fw, dy, O.SR, WL.seed_for(wl.cfg_index, li, 4))
            t["quantize"] = time.perf_counter() - t0
            t0 = time.perf_counter()
            O.dequantize(qx)
            t["dequantize"] = time.perf_counter() - t0
            t0 = time.perf_counter()
            xe, we, dye = qx.exact(), qw.exact(), qdy.exact()
            t["gemm_operands"] = time.perf_counter() - t0
            del qx, qw, qdy
            full = {}
            for op, n_out, fn, args in (("fwd", lay.numel_dy(), O.conv_fwd_points, (we, xe)),
                                        ("dgrad", lay.numel_x(), O.conv_dgrad_points, (we, dye)),
                                        ("wgrad", lay.numel_w(), O.conv_wgrad_points, (dye, xe))):
                k = min(npts[op], n_out)
                idx = np.sort(rng.choice(n_out, size=k, replace=False)).astype(np.int64)
                t0 = time.perf_counter()
                fn(cv, *args, idx)
                dt = time.perf_counter() - t0
                t[op + "_points"] = dt
                full[op] = dt * n_out / k
                gemm_pts_flops += lay.flops() * k / n_out
                gemm_pts_s += dt
            del xe, we, dye
            meas = sum(t.values())
            measured += meas
            step_s += t["quantize"] + t["dequantize"] + t["gemm_operands"] + sum(full.values())
            flops += 3 * lay.flops()
            nq = lay.numel_x() + lay.numel_w() + lay.numel_dy()
            q_bytes += nq * (8 + WL.FMT_BITS[fmt] / 8 + 1 / 64)
            q_s += t["quantize"]
            detail[f"{WL.FMT_NAMES[fmt]} L{li}"] = {k: round(v, 3) for k, v in t.items()}
    if wl.lr_buffer is not None and with_replay:
        nmaps, c, h, w_ = wl.lr_buffer
        maps = WL.gen_lr_maps(nmaps, c, h, w_, WL.seed_for(wl.cfg_index, 0, 5)).numpy()
        t0 = time.perf_counter()
        q = O.quantize(O.ACT, O.E2M1, maps)
        tq = time.perf_counter() - t0
        t0 = time.perf_counter()
        O.dequantize(q)
        tdq = time.perf_counter() - t0
        measured += tq + tdq
        step_s += tq + tdq
        q_bytes += maps.size * (8 + 4 / 8 + 1 / 64)
        q_s += tq
        detail["replay buffer"] = {"quantize": round(tq, 3), "dequantize": round(tdq, 3)}
    return {"value": flops / step_s / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "sample": (f"per format ({', '.join(WL.FMT_NAMES[f] for f in fmts)}) and layer: full quantize X/W/dY, "
                       f"fp32 dequantize Xq and fp64 GEMM operands; fwd, dgrad and wgrad on "
                       f"{npts['fwd']}, {npts['dgrad']} and {npts['wgrad']} seeded sampled outputs, their time "
                       f"scaled to all outputs; replay buffer quantize + dequantize in full"
                       if wl.lr_buffer else ""),
            "seconds": measured,
            "extrapolated_step_seconds": step_s,
            "oracle_gemm_gflops_on_sample": gemm_pts_flops / gemm_pts_s / 1e9 if gemm_pts_s else None,
            "oracle_quantize_gbps": q_bytes / q_s / 1e9 if q_s else None,
            "detail_seconds": detail}


if __name__ == "__main__":
    main()
