"""C ABI checks that need no GPU: the library loads, exports every entry point
the header declares, sizes buffers as documented, and rejects bad arguments
on the host before anything is enqueued."""
import ctypes
import os
import re

import pytest

import microscaling_quantized_convolution_mx_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxconv.h")

# fake device addresses: validation must reject the call before any use
A16 = 0x10000
MIS = 0x10001


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mx_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function():
    L = mx.lib()
    names = header_functions()
    assert set(names) == set(mx.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


@pytest.mark.parametrize("fmt,bits", [(mx.MX_E2M1, 4), (mx.MX_E2M3, 6), (mx.MX_E4M3, 8)])
def test_buffer_sizes(fmt, bits):
    d = mx.desc(16, 24, 40, 9, 7, 3, 3, 2, 2, 1, 1, elem_fmt=fmt)
    ho, wo = d.h_out, d.w_out
    assert (ho, wo) == (5, 4)
    assert mx.mx_code_bytes(d, mx.MX_ROLE_ACT) == 9 * 7 * 24 * 16 * bits // 8
    assert mx.mx_code_bytes(d, mx.MX_ROLE_GRAD) == ho * wo * 40 * 16 * bits // 8
    assert mx.mx_code_bytes(d, mx.MX_ROLE_WEIGHT) == 40 * 24 * 9 * bits // 8
    # one byte per block, padded to 16, then 2 KiB of amax-reduction scratch
    pad16 = lambda v: (v + 15) // 16 * 16
    assert mx.mx_scale_bytes(d, mx.MX_ROLE_ACT) == pad16(9 * 7 * 24 * 16 // 64) + 2048
    assert mx.mx_scale_bytes(d, mx.MX_ROLE_WEIGHT) == pad16(40 * 24 * 9 // 64) + 2048
    assert mx.mx_scale_bytes(mx.desc(0, 16, 16, 3, 3, 1, 1), mx.MX_ROLE_ACT) == 0
    ws = mx.mx_wgrad_workspace_bytes(d)
    assert ws > 0 and ws % (40 * 9 * 24 * 4) == 0


def test_invalid_descriptor_sizes_are_zero():
    assert mx.mx_code_bytes(mx.desc(8, 12, 16, 8, 8, 3, 3), mx.MX_ROLE_ACT) == 0
    assert mx.mx_scale_bytes(mx.desc(8, 16, 16, 8, 8, 3, 3), 9) == 0
    assert mx.mx_wgrad_workspace_bytes(mx.desc(8, 16, 16, 8, 8, 3, 3, block=4)) == 0


def test_status_strings():
    for code in range(-9, 1):
        assert len(mx.status_str(code)) > 0
    assert mx.status_str(-100) == "unknown status"


def q(codes=A16, scales=A16, t=A16, amax=A16):
    return mx.mx_qtensor(codes, scales, t, amax)


def quant(d, role=mx.MX_ROLE_ACT, src=A16, dst="ok", rounding=mx.MX_RNE):
    L = mx.lib()
    dptr = None if d is None else ctypes.byref(d)
    qp = None if dst is None else ctypes.byref(q() if dst == "ok" else dst)
    return L.mx_quantize_cbf(dptr, role, src, qp, rounding, 0, 0, None)


GOOD = dict(n=8, c_in=16, c_out=16, h=8, w=8, k_h=3, k_w=3)


@pytest.mark.parametrize("change,status", [
    (dict(block=4), -4), (dict(block=16), -4), (dict(block=32), -2),
    (dict(elem_fmt=0), -3), (dict(elem_fmt=6), -3), (dict(act_fmt=6), -3), (dict(act_fmt=-1), -3),
    (dict(c_in=12), -2), (dict(c_out=20), -2), (dict(n=12), -2), (dict(n=-8), -2),
    (dict(stride_h=0), -2), (dict(stride_w=-1), -2), (dict(pad_h=-1), -2),
    (dict(k_h=11), -2), (dict(h=0), -2), (dict(k_w=0), -2), (dict(c_in=0), -2),
    (dict(n=2 ** 30, h=64, w=64), -2),          # more elements than the kernels index
])
def test_descriptor_validation(change, status):
    kw = dict(GOOD)
    kw.update(change)
    d = mx.desc(**{k: kw[k] for k in GOOD}, **{k: v for k, v in kw.items() if k not in GOOD})
    assert quant(d) == status


def test_null_and_role_and_rounding():
    d = mx.desc(**GOOD)
    assert quant(None) == -1
    assert quant(d, role=3) == -7
    assert quant(d, rounding=2) == -9
    assert quant(d, dst=None) == -1
    assert quant(d, dst=q(codes=None)) == -1
    assert quant(d, dst=q(scales=None)) == -1
    assert quant(d, dst=q(t=None)) == -1
    assert quant(d, dst=q(amax=None)) == -1
    assert quant(d, src=None) == -1


def test_alignment():
    d = mx.desc(**GOOD)
    assert quant(d, dst=q(codes=MIS)) == -5
    assert quant(d, dst=q(scales=A16 + 4)) == -5   # the amax scratch tail needs 16-byte alignment
    assert quant(d, dst=q(t=A16 + 2)) == -5
    assert quant(d, src=A16 + 4) == -5


def test_conv_argument_checks():
    L = mx.lib()
    d = mx.desc(**GOOD)
    good = q()
    assert L.mx_conv_fwd(ctypes.byref(d), None, ctypes.byref(good), A16, None) == -1
    assert L.mx_conv_fwd(ctypes.byref(d), ctypes.byref(good), ctypes.byref(good), None, None) == -1
    assert L.mx_conv_fwd(ctypes.byref(d), ctypes.byref(good), ctypes.byref(good), MIS, None) == -5
    assert L.mx_conv_dgrad(ctypes.byref(d), ctypes.byref(good), ctypes.byref(q(codes=MIS)), A16, None) == -5
    assert L.mx_conv_dgrad(ctypes.byref(d), ctypes.byref(good), ctypes.byref(good), None, None) == -1
    need = mx.mx_wgrad_workspace_bytes(d)
    assert L.mx_conv_wgrad(ctypes.byref(d), ctypes.byref(good), ctypes.byref(good), A16, None, need, None) == -6
    assert L.mx_conv_wgrad(ctypes.byref(d), ctypes.byref(good), ctypes.byref(good), A16, A16, need - 4, None) == -6
    assert L.mx_conv_wgrad(ctypes.byref(d), ctypes.byref(good), ctypes.byref(good), None, A16, need, None) == -1
    assert L.mx_dequantize(ctypes.byref(d), 5, ctypes.byref(good), A16, None) == -7
    assert L.mx_dequantize(ctypes.byref(d), 0, ctypes.byref(good), MIS, None) == -5
    bad = mx.desc(**dict(GOOD, n=4))
    assert L.mx_conv_fwd(ctypes.byref(bad), ctypes.byref(good), ctypes.byref(good), A16, None) == -2
    # explicit im2col of the baseline flow
    assert L.mx_im2col_cbf(ctypes.byref(d), None, A16, None) == -1
    assert L.mx_im2col_cbf(ctypes.byref(d), A16, MIS, None) == -5
    assert L.mx_im2col_cbf(ctypes.byref(bad), A16, A16, None) == -2
    # fwd with the producer-fused amax: one word plus one per GEMM wave
    assert mx.mx_fwd_amax_bytes(d) >= 8 and mx.mx_fwd_amax_bytes(d) % 4 == 0
    assert mx.mx_fwd_amax_bytes(bad) == 0
    # fwd with the producer-fused amax: the amax word is checked too
    assert L.mx_conv_fwd_amax(ctypes.byref(d), ctypes.byref(good), ctypes.byref(good), A16, None, None) == -1
    assert L.mx_conv_fwd_amax(ctypes.byref(d), ctypes.byref(good), ctypes.byref(good), A16, A16 + 2, None) == -5
    assert L.mx_conv_fwd_amax(ctypes.byref(d), ctypes.byref(good), ctypes.byref(good), MIS, A16, None) == -5
    assert L.mx_conv_fwd_amax(ctypes.byref(bad), ctypes.byref(good), ctypes.byref(good), A16, A16, None) == -2


def test_binding_raises_on_error():
    with pytest.raises(mx.MxError) as e:
        mx.mx_conv_fwd(mx.desc(**dict(GOOD, block=2)), q(), q(), A16, stream=0)
    assert e.value.status == -4


def test_product_path_does_not_use_the_oracle():
    # the package must not import, link or call the oracle
    pkg = os.path.join(ROOT, "microscaling_quantized_convolution_mx_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "liboracle" not in text and "mxconv_oracle" not in text, f


def test_compact_activation_format_is_storage_only():
    # 3-bit codes: 3/8 byte per element, activations only, no GEMM
    d = mx.desc(16, 24, 40, 9, 7, 3, 3, 2, 2, 1, 1, elem_fmt=mx.MX_UE2M1)
    assert mx.mx_code_bytes(d, mx.MX_ROLE_ACT) == 9 * 7 * 24 * 16 * 3 // 8
    assert mx.mx_wgrad_workspace_bytes(d) == 0
    assert mx.mx_fwd_amax_bytes(d) == 0
    L = mx.lib()
    good = q()
    assert quant(d, role=mx.MX_ROLE_WEIGHT) == -3
    assert quant(d, role=mx.MX_ROLE_GRAD) == -3
    assert L.mx_dequantize(ctypes.byref(d), mx.MX_ROLE_GRAD, ctypes.byref(good), A16, None) == -3
    assert L.mx_conv_fwd(ctypes.byref(d), ctypes.byref(good), ctypes.byref(good), A16, None) == -3
    assert L.mx_conv_dgrad(ctypes.byref(d), ctypes.byref(good), ctypes.byref(good), A16, None) == -3
    assert L.mx_conv_wgrad(ctypes.byref(d), ctypes.byref(good), ctypes.byref(good), A16, A16, 1 << 20, None) == -3
    assert L.mx_conv_fwd_amax(ctypes.byref(d), ctypes.byref(good), ctypes.byref(good), A16, A16, None) == -3


def test_activation_format_pairs():
    # MicroQonv+ keeps X in FP6 while W and dY stay E2M1: each role is sized
    # in its own format, and the GEMMs take E2M1 with an FP6 activation
    L = mx.lib()
    good = q()
    for act, bits in ((mx.MX_E3M2, 6), (mx.MX_E2M3, 6)):
        d = mx.desc(16, 24, 40, 9, 7, 3, 3, 2, 2, 1, 1, elem_fmt=mx.MX_E2M1, act_fmt=act)
        assert mx.mx_code_bytes(d, mx.MX_ROLE_ACT) == 9 * 7 * 24 * 16 * bits // 8
        assert mx.mx_code_bytes(d, mx.MX_ROLE_WEIGHT) == 40 * 24 * 9 * 4 // 8
        assert mx.mx_code_bytes(d, mx.MX_ROLE_GRAD) == 5 * 4 * 40 * 16 * 4 // 8
        assert mx.mx_wgrad_workspace_bytes(d) > 0 and mx.mx_fwd_amax_bytes(d) > 0
        # past the format check: the misaligned output is what is rejected
        assert L.mx_conv_fwd(ctypes.byref(d), ctypes.byref(good), ctypes.byref(good), MIS, None) == -5
        assert L.mx_conv_wgrad(ctypes.byref(d), ctypes.byref(good), ctypes.byref(good), MIS, A16, 1 << 30, None) == -5
    # E3M2 throughout is a GEMM format too
    d = mx.desc(16, 24, 40, 9, 7, 3, 3, elem_fmt=mx.MX_E3M2)
    assert mx.mx_code_bytes(d, mx.MX_ROLE_WEIGHT) == 40 * 24 * 9 * 6 // 8
    assert L.mx_conv_dgrad(ctypes.byref(d), ctypes.byref(good), ctypes.byref(good), MIS, None) == -5
    # pairs without kernels: FP8 or FP6 weights with another activation format
    for fmt, act in ((mx.MX_E4M3, mx.MX_E3M2), (mx.MX_E2M3, mx.MX_E2M1), (mx.MX_E3M2, mx.MX_E2M3),
                     (mx.MX_E2M1, mx.MX_E4M3)):
        d = mx.desc(16, 24, 40, 9, 7, 3, 3, elem_fmt=fmt, act_fmt=act)
        assert L.mx_conv_fwd(ctypes.byref(d), ctypes.byref(good), ctypes.byref(good), A16, None) == -3
        assert L.mx_conv_wgrad(ctypes.byref(d), ctypes.byref(good), ctypes.byref(good), A16, A16, 1 << 30, None) == -3
        assert mx.mx_wgrad_workspace_bytes(d) == 0 and mx.mx_fwd_amax_bytes(d) == 0
        # the data gradient reads W and dY only
        assert L.mx_conv_dgrad(ctypes.byref(d), ctypes.byref(good), ctypes.byref(good), MIS, None) == -5
    # the compact codes as the activation format: storage only
    d = mx.desc(16, 24, 40, 9, 7, 3, 3, elem_fmt=mx.MX_E2M1, act_fmt=mx.MX_UE2M1)
    assert mx.mx_code_bytes(d, mx.MX_ROLE_ACT) == 9 * 7 * 24 * 16 * 3 // 8
    assert quant(d, role=mx.MX_ROLE_WEIGHT, dst=q(codes=MIS)) == -5   # W stays E2M1
    assert L.mx_conv_fwd(ctypes.byref(d), ctypes.byref(good), ctypes.byref(good), A16, None) == -3
    assert L.mx_conv_dgrad(ctypes.byref(d), ctypes.byref(good), ctypes.byref(good), MIS, None) == -5


def test_e8m0_block32_format():
    # E8M0 scale per 32x32 block: C_in, C_out and N multiples of 32, E2M1
    # elements throughout, one scale byte per block and no quantizer scratch
    L = mx.lib()
    good = q()
    d = mx.desc(64, 32, 96, 9, 7, 3, 3, 2, 2, 1, 1, block=32)
    assert mx.mx_code_bytes(d, mx.MX_ROLE_ACT) == 9 * 7 * 32 * 64 // 2
    assert mx.mx_code_bytes(d, mx.MX_ROLE_WEIGHT) == 96 * 32 * 9 // 2
    pad16 = lambda v: (v + 15) // 16 * 16
    assert mx.mx_scale_bytes(d, mx.MX_ROLE_ACT) == pad16(9 * 7 * 1 * 2)
    assert mx.mx_scale_bytes(d, mx.MX_ROLE_GRAD) == pad16(5 * 4 * 3 * 2)
    assert mx.mx_scale_bytes(d, mx.MX_ROLE_WEIGHT) == pad16(9 * 3 * 1)
    ws = mx.mx_wgrad_workspace_bytes(d)
    assert ws > 0 and ws % (96 * 9 * 32 * 4) == 0
    # the producer-fused amax feeds the two-level format only
    assert mx.mx_fwd_amax_bytes(d) == 0
    assert L.mx_conv_fwd_amax(ctypes.byref(d), ctypes.byref(good), ctypes.byref(good), A16, A16, None) == -4
    assert L.mx_conv_fwd(ctypes.byref(d), ctypes.byref(good), ctypes.byref(good), MIS, None) == -5
    for bad, status in ((dict(n=48), -2), (dict(c_in=16), -2), (dict(c_out=40), -2),
                        (dict(elem_fmt=mx.MX_E2M3), -3), (dict(act_fmt=mx.MX_E3M2), -3),
                        (dict(elem_fmt=mx.MX_E4M3), -3)):
        kw = dict(n=64, c_in=32, c_out=96, h=9, w=7, k_h=3, k_w=3, block=32)
        kw.update(bad)
        bd = mx.desc(kw.pop("n"), kw.pop("c_in"), kw.pop("c_out"), kw.pop("h"), kw.pop("w"), kw.pop("k_h"),
                     kw.pop("k_w"), **kw)
        assert quant(bd) == status, bad


def test_binding_rejects_unusable_tensors():
    # Every tensor argument is checked before anything touches the GPU: a
    # mistyped, strided, short or host tensor raises ValueError.  Host
    # tensors stand in here, so no GPU call is made.
    import torch
    d = mx.desc(**GOOD)
    nx = 8 * 8 * 16 * 8
    good_x = torch.zeros(8, 8, 16, 8)
    with pytest.raises(ValueError, match="float32"):
        mx.mx_quantize_cbf(d, mx.MX_ROLE_ACT, good_x.double(), None)
    with pytest.raises(ValueError, match="contiguous"):
        mx.mx_quantize_cbf(d, mx.MX_ROLE_ACT, good_x.transpose(0, 3), None)
    with pytest.raises(ValueError, match="needs %d" % (4 * nx)):
        mx.mx_quantize_cbf(d, mx.MX_ROLE_ACT, good_x[:4], None)
    with pytest.raises(ValueError, match="device memory"):
        mx.mx_quantize_cbf(d, mx.MX_ROLE_ACT, good_x, None)
    with pytest.raises(TypeError):
        mx.mx_quantize_cbf(d, mx.MX_ROLE_ACT, good_x.numpy(), None)
    # a quantized tensor's buffers: sized for the role under the descriptor
    qcpu = mx.QTensor(d, mx.MX_ROLE_ACT, device="cpu")
    with pytest.raises(ValueError, match="dst.codes: .*device memory"):
        mx.mx_quantize_cbf(d, mx.MX_ROLE_ACT, None, qcpu)
    small = mx.QTensor(mx.desc(**dict(GOOD, h=4, w=4)), mx.MX_ROLE_ACT, device="cpu")
    with pytest.raises(ValueError, match="dst.codes: .*needs %d" % mx.mx_code_bytes(d, mx.MX_ROLE_ACT)):
        mx.mx_quantize_cbf(d, mx.MX_ROLE_ACT, None, small)
    # GEMM outputs and the weight-gradient workspace
    ny = d.h_out * d.w_out * 16 * 8
    with pytest.raises(ValueError, match="y: .*needs %d" % (4 * ny)):
        mx.mx_conv_fwd(d, q(), q(), torch.zeros(ny - 1))
    with pytest.raises(ValueError, match="dx: .*float32"):
        mx.mx_conv_dgrad(d, q(), q(), torch.zeros(nx, dtype=torch.float16))
    with pytest.raises(ValueError, match="dw: .*needs"):
        mx.mx_conv_wgrad(d, q(), q(), torch.zeros(16 * 16 * 9 - 4), A16)
    need = mx.mx_wgrad_workspace_bytes(d)
    with pytest.raises(ValueError, match="workspace: .*needs %d" % (need + 4)):
        mx.mx_conv_wgrad(d, q(), q(), A16, torch.zeros(need // 4), ws_bytes=need + 4)
    with pytest.raises(ValueError, match="workspace: .*device memory"):
        mx.mx_conv_wgrad(d, q(), q(), A16, torch.zeros(need // 4))
    with pytest.raises(ValueError, match="y_amax: .*needs %d" % mx.mx_fwd_amax_bytes(d)):
        mx.mx_conv_fwd_amax(d, q(), q(), A16, torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError, match="xcol: .*needs"):
        mx.mx_im2col_cbf(d, A16, torch.zeros(nx))
    with pytest.raises(ValueError, match="dst: .*needs"):
        mx.mx_dequantize(d, mx.MX_ROLE_WEIGHT, q(), torch.zeros(16 * 16 * 9 - 1))
