"""MicroQonv microscaling convolution hot path for AMD MI355X (gfx950).

Thin ctypes binding of ``libmxconv.so`` (C ABI in ``include/mxconv.h``): the
functions below have the same names as the C entry points and only marshal
arguments -- every step of the computation runs in the HIP kernels.  PyTorch
is used for device memory and streams.  There is no CPU fallback: if the
library is missing, or a call fails, an exception is raised.

Method: "MicroQonv: Reshaping Convolution Tensors for Efficient Microscaling in
Training and Inference" (arXiv 2609.28358): quantize each convolution tensor
once in 8x8 microscaling blocks in a channel-batch-first layout (§IV-A,
§IV-B) and run the forward, data-gradient and weight-gradient GEMMs on the
quantized tensors through an implicit im2col.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmxconv.so")

MX_E2M1, MX_E2M3, MX_E4M3 = 1, 2, 3
MX_UE2M1 = 4  # compact 3-bit post-ReLU activation codes (quantize / dequantize only)
MX_E3M2 = 5   # FP6 with the wider range: MicroQonv+ activations (act_fmt)
CODE_BITS = {MX_E2M1: 4, MX_E2M3: 6, MX_E4M3: 8, MX_UE2M1: 3, MX_E3M2: 6}
MX_ROLE_ACT, MX_ROLE_WEIGHT, MX_ROLE_GRAD = 0, 1, 2
MX_RNE, MX_SR = 0, 1

STATUS = {0: "MX_OK", -1: "MX_ERR_NULL", -2: "MX_ERR_SHAPE", -3: "MX_ERR_FORMAT",
          -4: "MX_ERR_BLOCK", -5: "MX_ERR_ALIGN", -6: "MX_ERR_WORKSPACE", -7: "MX_ERR_ROLE",
          -8: "MX_ERR_LAUNCH", -9: "MX_ERR_ROUND"}

EXPORTS = ("mx_code_bytes", "mx_scale_bytes", "mx_wgrad_workspace_bytes", "mx_fwd_amax_bytes", "mx_quantize_cbf",
           "mx_conv_fwd", "mx_conv_fwd_amax", "mx_conv_dgrad", "mx_conv_wgrad", "mx_conv_wgrad_noalloc",
           "mx_dequantize", "mx_im2col_cbf", "mx_status_str")
# bytes of the static workspace of mx_conv_wgrad_noalloc (MX_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20


class MxError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_str(status)})")


class mx_conv_desc(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int32) for f in
                ("n", "c_in", "c_out", "h", "w", "k_h", "k_w", "stride_h", "stride_w",
                 "pad_h", "pad_w", "elem_fmt", "block", "act_fmt")]

    @property
    def h_out(self) -> int:
        return (self.h + 2 * self.pad_h - self.k_h) // self.stride_h + 1

    @property
    def w_out(self) -> int:
        return (self.w + 2 * self.pad_w - self.k_w) // self.stride_w + 1


class mx_qtensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("tensor_scale", ctypes.c_void_p), ("amax", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmxconv.so (built by build.py); raises if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build() "
                           "(or python -m microscaling_quantized_convolution_mx_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    D = ctypes.POINTER(mx_conv_desc)
    Q = ctypes.POINTER(mx_qtensor)
    P = ctypes.c_void_p
    for f in ("mx_code_bytes", "mx_scale_bytes"):
        getattr(L, f).restype = ctypes.c_size_t
        getattr(L, f).argtypes = [D, ctypes.c_int]
    L.mx_wgrad_workspace_bytes.restype = ctypes.c_size_t
    L.mx_wgrad_workspace_bytes.argtypes = [D]
    L.mx_quantize_cbf.restype = ctypes.c_int
    L.mx_quantize_cbf.argtypes = [D, ctypes.c_int, P, Q, ctypes.c_int, ctypes.c_uint64, ctypes.c_int, P]
    for f in ("mx_conv_fwd", "mx_conv_dgrad"):
        getattr(L, f).restype = ctypes.c_int
        getattr(L, f).argtypes = [D, Q, Q, P, P]
    L.mx_fwd_amax_bytes.restype = ctypes.c_size_t
    L.mx_fwd_amax_bytes.argtypes = [D]
    L.mx_conv_fwd_amax.restype = ctypes.c_int
    L.mx_conv_fwd_amax.argtypes = [D, Q, Q, P, P, P]
    L.mx_conv_wgrad.restype = ctypes.c_int
    L.mx_conv_wgrad.argtypes = [D, Q, Q, P, P, ctypes.c_size_t, P]
    L.mx_conv_wgrad_noalloc.restype = ctypes.c_int
    L.mx_conv_wgrad_noalloc.argtypes = [D, Q, Q, P, P]
    L.mx_dequantize.restype = ctypes.c_int
    L.mx_dequantize.argtypes = [D, ctypes.c_int, Q, P, P]
    L.mx_im2col_cbf.restype = ctypes.c_int
    L.mx_im2col_cbf.argtypes = [D, P, P, P]
    L.mx_status_str.restype = ctypes.c_char_p
    L.mx_status_str.argtypes = [ctypes.c_int]
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().mx_status_str(status).decode()


def desc(n, c_in, c_out, h, w, k_h, k_w, stride_h=1, stride_w=1, pad_h=0, pad_w=0,
         elem_fmt=MX_E2M1, block=8, act_fmt=0) -> mx_conv_desc:
    """act_fmt: format of the activation X (0: elem_fmt, the format of W and dY).
    block: 8 (E4M3 block scale and fp32 tensor scale) or 32 (E8M0 scale per
    32x32 block, E2M1 elements)."""
    return mx_conv_desc(n, c_in, c_out, h, w, k_h, k_w, stride_h, stride_w, pad_h, pad_w,
                        elem_fmt, block, act_fmt)


def desc_from_layer(layer, elem_fmt: int, act_fmt: int = 0, block: int = 8) -> mx_conv_desc:
    return desc(layer.n, layer.c_in, layer.c_out, layer.h, layer.w, layer.k_h, layer.k_w,
                layer.stride_h, layer.stride_w, layer.pad_h, layer.pad_w, elem_fmt, block=block, act_fmt=act_fmt)


def role_fmt(d: mx_conv_desc, role: int) -> int:
    """Element format of the tensor of `role` under descriptor d."""
    return d.act_fmt if (role == MX_ROLE_ACT and d.act_fmt != 0) else d.elem_fmt


def role_numel(d: mx_conv_desc, role: int) -> int:
    """fp32 elements of the tensor of `role` under d (0 for a bad role)."""
    if role == MX_ROLE_ACT:
        return d.h * d.w * d.c_in * d.n
    if role == MX_ROLE_GRAD:
        return max(d.h_out, 0) * max(d.w_out, 0) * d.c_out * d.n
    if role == MX_ROLE_WEIGHT:
        return d.c_out * d.c_in * d.k_h * d.k_w
    return 0


def _buf(t, need: int, what: str, fp32: bool = True) -> int | None:
    """Device address of a caller buffer after checking that it can take the
    call: a float32 tensor (fp32 data; any dtype for workspace and scratch
    words), contiguous, at least `need` bytes, in device memory.  The checks
    run before anything touches the GPU, so a host, strided, mistyped or
    short tensor raises ValueError instead of reaching a kernel.  An int is
    taken as a raw device address that the caller vouches for, as at the C
    ABI; None passes through (the library reports MX_ERR_NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch tensor or a device address, got {type(t).__name__}")
    if fp32 and t.dtype != torch.float32:
        raise ValueError(f"{what}: must be float32, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")
    nbytes = t.numel() * t.element_size()
    if nbytes < need:
        raise ValueError(f"{what}: {nbytes} bytes, the call needs {need}")
    if t.device.type != "cuda":
        raise ValueError(f"{what}: must be in device memory, got a {t.device.type} tensor")
    return t.data_ptr() if t.numel() > 0 else None


def _stream(stream) -> int | None:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, where: str) -> None:
    if status != 0:
        raise MxError(status, where)


def mx_code_bytes(d: mx_conv_desc, role: int) -> int:
    return lib().mx_code_bytes(ctypes.byref(d), role)


def mx_scale_bytes(d: mx_conv_desc, role: int) -> int:
    return lib().mx_scale_bytes(ctypes.byref(d), role)


def mx_wgrad_workspace_bytes(d: mx_conv_desc) -> int:
    return lib().mx_wgrad_workspace_bytes(ctypes.byref(d))


class QTensor:
    """Device buffers of one quantized tensor (owned by torch)."""

    def __init__(self, d: mx_conv_desc, role: int, device="cuda"):
        import torch
        self.role = role
        self.fmt = role_fmt(d, role)
        nc = mx_code_bytes(d, role)
        ns = mx_scale_bytes(d, role)
        # at least 16 bytes, so that an empty tensor still has valid pointers
        self.codes = torch.empty(max(nc, 16), dtype=torch.uint8, device=device)
        self.scales = torch.empty(max(ns, 16), dtype=torch.uint8, device=device)
        self.tensor_scale = torch.zeros(1, dtype=torch.float32, device=device)
        self.amax = torch.zeros(1, dtype=torch.float32, device=device)
        self.code_bytes, self.scale_bytes = nc, ns
        # stored block scales: one byte per block (8x8 E4M3 or 32x32 E8M0;
        # the rest of the scales buffer is the quantizer's scratch)
        self.block = d.block
        self.nblocks = nc * 8 // (d.block * d.block * CODE_BITS[self.fmt])

    def c(self) -> mx_qtensor:
        return mx_qtensor(self.codes.data_ptr(), self.scales.data_ptr(),
                          self.tensor_scale.data_ptr(), self.amax.data_ptr())


def _q(q, d: mx_conv_desc | None = None, role: int | None = None, what: str = "q"):
    """Pointer to the mx_qtensor of q.  A QTensor is checked against the
    buffers the call needs for `role` under d (as _buf does for plain
    tensors); an mx_qtensor struct holds raw device addresses and passes
    through unchecked."""
    if q is None:
        return None
    if isinstance(q, QTensor):
        if d is not None and role is not None:
            _buf(q.codes, mx_code_bytes(d, role), f"{what}.codes", fp32=False)
            _buf(q.scales, mx_scale_bytes(d, role), f"{what}.scales", fp32=False)
        _buf(q.tensor_scale, 4, f"{what}.tensor_scale")
        _buf(q.amax, 4, f"{what}.amax")
        return ctypes.byref(q.c())
    if isinstance(q, mx_qtensor):
        return ctypes.byref(q)
    raise TypeError(f"{what}: expected a QTensor or an mx_qtensor, got {type(q).__name__}")


def mx_quantize_cbf(d: mx_conv_desc, role: int, src, dst, rounding: int = MX_RNE, seed: int = 0,
                    amax_given: bool = False, stream=None) -> None:
    args = (ctypes.byref(d), role, _buf(src, 4 * role_numel(d, role), "src"), _q(dst, d, role, "dst"), rounding,
            seed & (2 ** 64 - 1), int(bool(amax_given)))
    _check(lib().mx_quantize_cbf(*args, _stream(stream)), "mx_quantize_cbf")


def mx_conv_fwd(d: mx_conv_desc, wq, xq, y, stream=None) -> None:
    args = (ctypes.byref(d), _q(wq, d, MX_ROLE_WEIGHT, "wq"), _q(xq, d, MX_ROLE_ACT, "xq"),
            _buf(y, 4 * role_numel(d, MX_ROLE_GRAD), "y"))
    _check(lib().mx_conv_fwd(*args, _stream(stream)), "mx_conv_fwd")


def mx_fwd_amax_bytes(d: mx_conv_desc) -> int:
    return lib().mx_fwd_amax_bytes(ctypes.byref(d))


def mx_conv_fwd_amax(d: mx_conv_desc, wq, xq, y, y_amax, stream=None) -> None:
    args = (ctypes.byref(d), _q(wq, d, MX_ROLE_WEIGHT, "wq"), _q(xq, d, MX_ROLE_ACT, "xq"),
            _buf(y, 4 * role_numel(d, MX_ROLE_GRAD), "y"), _buf(y_amax, mx_fwd_amax_bytes(d), "y_amax", fp32=False))
    _check(lib().mx_conv_fwd_amax(*args, _stream(stream)), "mx_conv_fwd_amax")


def mx_conv_dgrad(d: mx_conv_desc, wq, dyq, dx, stream=None) -> None:
    args = (ctypes.byref(d), _q(wq, d, MX_ROLE_WEIGHT, "wq"), _q(dyq, d, MX_ROLE_GRAD, "dyq"),
            _buf(dx, 4 * role_numel(d, MX_ROLE_ACT), "dx"))
    _check(lib().mx_conv_dgrad(*args, _stream(stream)), "mx_conv_dgrad")


def mx_conv_wgrad(d: mx_conv_desc, dyq, xq, dw, workspace, ws_bytes: int | None = None,
                  stream=None) -> None:
    """ws_bytes: bytes of workspace the library may use (default: all of it)."""
    if ws_bytes is None:
        ws_bytes = 0 if workspace is None or isinstance(workspace, int) else workspace.numel() * workspace.element_size()
    args = (ctypes.byref(d), _q(dyq, d, MX_ROLE_GRAD, "dyq"), _q(xq, d, MX_ROLE_ACT, "xq"),
            _buf(dw, 4 * role_numel(d, MX_ROLE_WEIGHT), "dw"), _buf(workspace, ws_bytes, "workspace", fp32=False),
            ws_bytes)
    _check(lib().mx_conv_wgrad(*args, _stream(stream)), "mx_conv_wgrad")


def mx_conv_wgrad_noalloc(d: mx_conv_desc, dyq, xq, dw, stream=None) -> None:
    """mx_conv_wgrad with the library's static per-GPU workspace (for callers
    that cannot allocate); calls that overlap in time on one GPU race."""
    args = (ctypes.byref(d), _q(dyq, d, MX_ROLE_GRAD, "dyq"), _q(xq, d, MX_ROLE_ACT, "xq"),
            _buf(dw, 4 * role_numel(d, MX_ROLE_WEIGHT), "dw"))
    _check(lib().mx_conv_wgrad_noalloc(*args, _stream(stream)), "mx_conv_wgrad_noalloc")


def mx_im2col_cbf(d: mx_conv_desc, x, xcol, stream=None) -> None:
    ncol = max(d.h_out, 0) * max(d.w_out, 0) * d.k_h * d.k_w * d.c_in * d.n
    args = (ctypes.byref(d), _buf(x, 4 * role_numel(d, MX_ROLE_ACT), "x"), _buf(xcol, 4 * ncol, "xcol"))
    _check(lib().mx_im2col_cbf(*args, _stream(stream)), "mx_im2col_cbf")


def mx_dequantize(d: mx_conv_desc, role: int, q, dst, stream=None) -> None:
    args = (ctypes.byref(d), role, _q(q, d, role, "q"), _buf(dst, 4 * role_numel(d, role), "dst"))
    _check(lib().mx_dequantize(*args, _stream(stream)), "mx_dequantize")
