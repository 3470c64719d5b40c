"""CPU oracle for the MicroQonv hot path -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never links, loads
or calls it, and it shares no code with the HIP implementation.

The arithmetic lives in ``mxconv_oracle.c`` (plain nested loops, fp32 steps as
single IEEE operations, fp64 GEMMs on exact dequantized values).  This module
builds it with gcc and wraps it with ctypes + numpy.  Everything it computes
follows "MicroQonv: Reshaping Convolution Tensors for Efficient Microscaling in
Training and Inference" (arXiv 2609.28358):

* quantizer (two-level NVFP4-style scaling, 8x8 square blocks) -- §III-A, §IV-B
* channel-batch-first layouts -- §IV-A, Fig. 3
* explicit im2col and the three GEMMs -- §II-C, §IV-B
* quantization-event counts of the three flows -- §IV-C, Table I
* the original microscaling format (E8M0 power-of-two scale per square block,
  no tensor scale) on 32x32 blocks -- §II-D, §IV-B
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mxconv_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

E2M1, E2M3, E4M3, E3M2 = 1, 2, 3, 4
UE2M1 = 5  # E2M1 magnitude without sign: 3-bit post-ReLU activation codes
ACT, WEIGHT, GRAD = 0, 1, 2
RNE, SR = 0, 1


def build() -> str:
    """Compile the oracle with gcc (no fast-math, no fp contraction)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-std=c11", "-Wall", "-o", LIB + ".tmp", SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


class OrcConv(ctypes.Structure):
    """Convolution geometry (the oracle's own definition)."""
    _fields_ = [(name, ctypes.c_int32) for name in
                ("n", "c_in", "c_out", "h", "w", "k_h", "k_w",
                 "stride_h", "stride_w", "pad_h", "pad_w")]

    @property
    def h_out(self) -> int:
        return (self.h + 2 * self.pad_h - self.k_h) // self.stride_h + 1

    @property
    def w_out(self) -> int:
        return (self.w + 2 * self.pad_w - self.k_w) // self.stride_w + 1


def conv(n, c_in, c_out, h, w, k_h, k_w, stride_h=1, stride_w=1, pad_h=0, pad_w=0) -> OrcConv:
    return OrcConv(n, c_in, c_out, h, w, k_h, k_w, stride_h, stride_w, pad_h, pad_w)


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    L = ctypes.CDLL(LIB)
    L.orc_fmt_value.restype = ctypes.c_double
    L.orc_fmt_value.argtypes = [ctypes.c_int, ctypes.c_int]
    L.orc_fmt_max.restype = ctypes.c_double
    L.orc_fmt_max.argtypes = [ctypes.c_int]
    for f in ("orc_fmt_nmag", "orc_fmt_sign_shift", "orc_fmt_bits"):
        getattr(L, f).restype = ctypes.c_int
        getattr(L, f).argtypes = [ctypes.c_int]
    L.orc_round_rne.restype = ctypes.c_int
    L.orc_round_rne.argtypes = [ctypes.c_int, ctypes.c_float]
    L.orc_round_sr.restype = ctypes.c_int
    L.orc_round_sr.argtypes = [ctypes.c_int, ctypes.c_float, ctypes.c_float]
    L.orc_e4m3_code.restype = ctypes.c_int
    L.orc_e4m3_code.argtypes = [ctypes.c_float]
    L.orc_splitmix64.restype = ctypes.c_uint64
    L.orc_splitmix64.argtypes = [ctypes.c_uint64]
    L.orc_sr_uniform.restype = ctypes.c_float
    L.orc_sr_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
    L.orc_role_nblocks.restype = _I64
    L.orc_role_nblocks.argtypes = [ctypes.c_int, _I64, _I64, _I64, _I64]
    L.orc_role_src_index.restype = _I64
    L.orc_role_src_index.argtypes = [ctypes.c_int, _I64, _I64, _I64, _I64, _I64,
                                     ctypes.c_int, ctypes.c_int]
    L.orc_quantize.restype = ctypes.c_int
    L.orc_quantize.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint64, _P,
                               _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P]
    L.orc_quantize_blocks.restype = ctypes.c_int
    L.orc_quantize_blocks.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                                      _P, _I64, _I64, _I64, _I64, ctypes.c_float, _P, _I64,
                                      _P, _P, _P]
    for f in ("orc_dequantize", "orc_dequantize64"):
        getattr(L, f).restype = ctypes.c_int
        getattr(L, f).argtypes = [ctypes.c_int, ctypes.c_int, _I64, _I64, _I64, _I64, _P, _P,
                                  ctypes.c_float, _P]
    L.orc_e8m0_code.restype = ctypes.c_int
    L.orc_e8m0_code.argtypes = [ctypes.c_int, ctypes.c_float, ctypes.c_int]
    L.orc_mx_nblocks.restype = _I64
    L.orc_mx_nblocks.argtypes = [ctypes.c_int, ctypes.c_int, _I64, _I64, _I64, _I64]
    L.orc_mx_src_index.restype = _I64
    L.orc_mx_src_index.argtypes = [ctypes.c_int, ctypes.c_int, _I64, _I64, _I64, _I64, _I64,
                                   ctypes.c_int, ctypes.c_int]
    L.orc_quantize_mx.restype = ctypes.c_int
    L.orc_quantize_mx.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint64, ctypes.c_int, _P,
                                  _I64, _I64, _I64, _I64, _P, _P]
    L.orc_dequantize_mx.restype = ctypes.c_int
    L.orc_dequantize_mx.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _I64, _I64, _I64, _I64, _P, _P,
                                    _P, _P]
    L.orc_pack.restype = ctypes.c_int
    L.orc_pack.argtypes = [ctypes.c_int, _P, _I64, _P]
    L.orc_im2col_src.restype = _I64
    L.orc_im2col_src.argtypes = [ctypes.POINTER(OrcConv), _I64, _I64]
    for f in ("orc_conv_fwd", "orc_conv_dgrad", "orc_conv_wgrad"):
        getattr(L, f).restype = ctypes.c_int
        getattr(L, f).argtypes = [ctypes.POINTER(OrcConv), _P, _P, _P, _P]
    for f in ("orc_conv_fwd_points", "orc_conv_dgrad_points", "orc_conv_wgrad_points"):
        getattr(L, f).restype = ctypes.c_int
        getattr(L, f).argtypes = [ctypes.POINTER(OrcConv), _P, _P, _P, _I64, _P, _P]
    L.orc_conv_direct.restype = ctypes.c_int
    L.orc_conv_direct.argtypes = [ctypes.POINTER(OrcConv), _P, _P, _P]
    L.orc_count_act_quant.restype = _I64
    L.orc_count_act_quant.argtypes = [ctypes.POINTER(OrcConv), ctypes.c_int, _P]
    L.orc_count_operand_quant.restype = _I64
    L.orc_count_operand_quant.argtypes = [ctypes.POINTER(OrcConv), ctypes.c_int, ctypes.c_int, _P]
    L.orc_quantize_after_im2col.restype = ctypes.c_int
    L.orc_threads.restype = ctypes.c_int
    L.orc_threads.argtypes = []
    L.orc_set_threads.restype = None
    L.orc_set_threads.argtypes = [ctypes.c_int]
    L.orc_quantize_after_im2col.argtypes = [ctypes.POINTER(OrcConv), ctypes.c_int, _P, _P, _P, _P, _P]
    _lib = L
    return L


def threads() -> int:
    """Threads the oracle's OpenMP loops run on."""
    return lib().orc_threads()


def set_threads(n: int) -> None:
    """Threads for the oracle's OpenMP loops (for timing; results do not depend on it)."""
    lib().orc_set_threads(int(n))


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------
# formats
# --------------------------------------------------------------------------

def fmt_value(fmt: int, mag: int) -> float:
    return lib().orc_fmt_value(fmt, mag)


def fmt_grid(fmt: int) -> np.ndarray:
    return np.array([fmt_value(fmt, m) for m in range(lib().orc_fmt_nmag(fmt))])


def fmt_max(fmt: int) -> float:
    return lib().orc_fmt_max(fmt)


def fmt_bits(fmt: int) -> int:
    return lib().orc_fmt_bits(fmt)


def sign_shift(fmt: int) -> int:
    return lib().orc_fmt_sign_shift(fmt)


def round_rne(fmt: int, v: float) -> int:
    return lib().orc_round_rne(fmt, v)


def round_sr(fmt: int, v: float, u: float) -> int:
    return lib().orc_round_sr(fmt, v, u)


def e4m3_code(v: float) -> int:
    return lib().orc_e4m3_code(v)


def sr_uniform(seed: int, idx: int) -> float:
    return lib().orc_sr_uniform(seed, idx)


def splitmix64(z: int) -> int:
    return lib().orc_splitmix64(z)


# --------------------------------------------------------------------------
# quantizer
# --------------------------------------------------------------------------

def role_dims(role: int, shape) -> tuple:
    """(d0, d1, d2, d3) for the oracle: (H, W, C, N) or (Co, Ci, Kh, Kw)."""
    assert len(shape) == 4
    return tuple(int(s) for s in shape)


def nblocks(role: int, dims) -> int:
    return lib().orc_role_nblocks(role, *dims)


def block_src_index(role: int, dims, b: int, r: int, c: int) -> int:
    return lib().orc_role_src_index(role, *dims, b, r, c)


class QTensor:
    """Oracle-side quantized tensor: unpacked codes (one byte per element in
    block order), E4M3 block scales, fp32 tensor scale and amax."""

    def __init__(self, role, fmt, dims, codes, scales, t, amax):
        self.role, self.fmt, self.dims = role, fmt, dims
        self.codes, self.scales = codes, scales
        self.t, self.amax = t, amax

    def packed(self) -> np.ndarray:
        return pack(self.fmt, self.codes)

    def dequantize(self) -> np.ndarray:
        return dequantize(self)

    def exact(self) -> np.ndarray:
        return dequantize64(self)


def quantize(role: int, fmt: int, src: np.ndarray, rounding: int = RNE, seed: int = 0,
             amax: float | None = None) -> QTensor:
    src = np.ascontiguousarray(src, dtype=np.float32)
    dims = role_dims(role, src.shape)
    nb = nblocks(role, dims)
    codes = np.zeros(nb * 64, dtype=np.uint8)
    scales = np.zeros(nb, dtype=np.uint8)
    t = np.zeros(1, dtype=np.float32)
    am = np.zeros(1, dtype=np.float32)
    amax_in = None
    if amax is not None:
        amax_in = np.array([amax], dtype=np.float32)
    rc = lib().orc_quantize(role, fmt, rounding, seed, _ptr(src), *dims,
                            _ptr(amax_in) if amax_in is not None else None,
                            _ptr(codes), _ptr(scales), _ptr(t), _ptr(am))
    if rc != 0:
        raise ValueError("oracle quantize rejected its arguments")
    return QTensor(role, fmt, dims, codes, scales, float(t[0]), float(am[0]))


def quantize_blocks(role: int, fmt: int, src: np.ndarray, blocks: np.ndarray, amax: float,
                    rounding: int = RNE, seed: int = 0):
    """Quantize only the listed blocks given the tensor amax.
    Returns (codes [nsel, 64], scales [nsel], T)."""
    src = np.ascontiguousarray(src, dtype=np.float32)
    dims = role_dims(role, src.shape)
    blocks = np.ascontiguousarray(blocks, dtype=np.int64)
    codes = np.zeros(blocks.size * 64, dtype=np.uint8)
    scales = np.zeros(blocks.size, dtype=np.uint8)
    t = np.zeros(1, dtype=np.float32)
    rc = lib().orc_quantize_blocks(role, fmt, rounding, seed, _ptr(src), *dims, amax,
                                   _ptr(blocks), blocks.size, _ptr(codes), _ptr(scales), _ptr(t))
    if rc != 0:
        raise ValueError("oracle quantize_blocks rejected its arguments")
    return codes.reshape(-1, 64), scales, float(t[0])


def dequantize(q: QTensor) -> np.ndarray:
    out = np.zeros(q.dims, dtype=np.float32)
    lib().orc_dequantize(q.role, q.fmt, *q.dims, _ptr(q.codes), _ptr(q.scales), q.t, _ptr(out))
    return out


def dequantize64(q: QTensor) -> np.ndarray:
    out = np.zeros(q.dims, dtype=np.float64)
    lib().orc_dequantize64(q.role, q.fmt, *q.dims, _ptr(q.codes), _ptr(q.scales), q.t, _ptr(out))
    return out


# --------------------------------------------------------------------------
# the original microscaling format on square blocks (E8M0 scale per block)
# --------------------------------------------------------------------------

MX_BLOCK = 32


def e8m0_code(fmt: int, amax: float, nonfinite: bool = False) -> int:
    return lib().orc_e8m0_code(fmt, amax, int(bool(nonfinite)))


def mx_nblocks(role: int, dims, block: int = MX_BLOCK) -> int:
    return lib().orc_mx_nblocks(role, block, *dims)


def mx_src_index(role: int, dims, b: int, r: int, c: int, block: int = MX_BLOCK) -> int:
    return lib().orc_mx_src_index(role, block, *dims, b, r, c)


class MxTensor:
    """Oracle-side MX tensor: unpacked codes (one byte per element in block
    order), one E8M0 scale per S x S block, no tensor scale."""

    def __init__(self, role, fmt, dims, block, codes, scales):
        self.role, self.fmt, self.dims, self.block = role, fmt, dims, block
        self.codes, self.scales = codes, scales

    def packed(self) -> np.ndarray:
        return pack(self.fmt, self.codes)

    def _deq(self, want64: bool):
        out = np.zeros(self.dims, dtype=np.float64 if want64 else np.float32)
        args = (_ptr(out), None) if want64 else (None, _ptr(out))
        if lib().orc_dequantize_mx(self.role, self.fmt, self.block, *self.dims, _ptr(self.codes),
                                   _ptr(self.scales), *args) != 0:
            raise ValueError("bad format")
        return out

    def dequantize(self) -> np.ndarray:
        return self._deq(False)

    def exact(self) -> np.ndarray:
        return self._deq(True)


def quantize_mx(role: int, fmt: int, src: np.ndarray, rounding: int = RNE, seed: int = 0,
                block: int = MX_BLOCK) -> MxTensor:
    src = np.ascontiguousarray(src, dtype=np.float32)
    dims = role_dims(role, src.shape)
    nb = mx_nblocks(role, dims, block)
    codes = np.zeros(nb * block * block, dtype=np.uint8)
    scales = np.zeros(nb, dtype=np.uint8)
    rc = lib().orc_quantize_mx(role, fmt, rounding, seed, block, _ptr(src), *dims, _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError("oracle quantize_mx rejected its arguments")
    return MxTensor(role, fmt, dims, block, codes, scales)


def pack(fmt: int, codes: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    nbytes = codes.size * fmt_bits(fmt) // 8
    out = np.zeros(nbytes, dtype=np.uint8)
    if lib().orc_pack(fmt, _ptr(codes), codes.size, _ptr(out)) != 0:
        raise ValueError("bad format")
    return out


# --------------------------------------------------------------------------
# convolution
# --------------------------------------------------------------------------

def im2col_src(cv: OrcConv, k: int, j: int) -> int:
    return lib().orc_im2col_src(ctypes.byref(cv), k, j)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def conv_fwd(cv: OrcConv, w: np.ndarray, x: np.ndarray):
    """Y = W_f X' (fp64); w OIHW, x [H][W][Ci][N] -> (y, S) in [Ho][Wo][Co][N]."""
    w, x = _f64(w), _f64(x)
    y = np.zeros((cv.h_out, cv.w_out, cv.c_out, cv.n))
    s = np.zeros_like(y)
    if lib().orc_conv_fwd(ctypes.byref(cv), _ptr(w), _ptr(x), _ptr(y), _ptr(s)) != 0:
        raise MemoryError("oracle conv_fwd")
    return y, s


def conv_dgrad(cv: OrcConv, w: np.ndarray, dy: np.ndarray):
    """dX = col2im(W_f^T G_Y) -> (dx, S) in [H][W][Ci][N]."""
    w, dy = _f64(w), _f64(dy)
    dx = np.zeros((cv.h, cv.w, cv.c_in, cv.n))
    s = np.zeros_like(dx)
    if lib().orc_conv_dgrad(ctypes.byref(cv), _ptr(w), _ptr(dy), _ptr(dx), _ptr(s)) != 0:
        raise MemoryError("oracle conv_dgrad")
    return dx, s


def conv_wgrad(cv: OrcConv, dy: np.ndarray, x: np.ndarray):
    """dW = G_Y X'^T -> (dw, S) in OIHW."""
    dy, x = _f64(dy), _f64(x)
    dw = np.zeros((cv.c_out, cv.c_in, cv.k_h, cv.k_w))
    s = np.zeros_like(dw)
    if lib().orc_conv_wgrad(ctypes.byref(cv), _ptr(dy), _ptr(x), _ptr(dw), _ptr(s)) != 0:
        raise MemoryError("oracle conv_wgrad")
    return dw, s


def _points(fn, cv, a, b, idx):
    a, b = _f64(a), _f64(b)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    val = np.zeros(idx.size)
    s = np.zeros(idx.size)
    fn(ctypes.byref(cv), _ptr(a), _ptr(b), _ptr(idx), idx.size, _ptr(val), _ptr(s))
    return val, s


def conv_fwd_points(cv, w, x, idx):
    return _points(lib().orc_conv_fwd_points, cv, w, x, idx)


def conv_dgrad_points(cv, w, dy, idx):
    return _points(lib().orc_conv_dgrad_points, cv, w, dy, idx)


def conv_wgrad_points(cv, dy, x, idx):
    return _points(lib().orc_conv_wgrad_points, cv, dy, x, idx)


def conv_direct(cv: OrcConv, w: np.ndarray, x: np.ndarray) -> np.ndarray:
    w, x = _f64(w), _f64(x)
    y = np.zeros((cv.h_out, cv.w_out, cv.c_out, cv.n))
    lib().orc_conv_direct(ctypes.byref(cv), _ptr(w), _ptr(x), _ptr(y))
    return y


FLOW_MICROQONV, FLOW_IM2COL_SQUARE, FLOW_DACAPO = 0, 1, 2


def count_act_quant(cv: OrcConv, flow: int):
    """Per-activation quantization counts and total events of one flow."""
    counts = np.zeros((cv.h, cv.w, cv.c_in, cv.n), dtype=np.int32)
    events = lib().orc_count_act_quant(ctypes.byref(cv), flow, _ptr(counts))
    return counts, int(events)


TENSOR_W, TENSOR_DY = 1, 2


def count_operand_quant(cv: OrcConv, flow: int, tensor: int):
    """Per-element quantization counts and total events of the weight
    (TENSOR_W, counts [Kh*Kw][C_out][C_in]) or the output gradient
    (TENSOR_DY, counts [C_out][Ho*Wo*N]) under one flow."""
    if tensor == TENSOR_W:
        shape = (cv.k_h * cv.k_w, cv.c_out, cv.c_in)
    else:
        shape = (cv.c_out, cv.h_out * cv.w_out * cv.n)
    counts = np.zeros(shape, dtype=np.int32)
    events = lib().orc_count_operand_quant(ctypes.byref(cv), flow, tensor, _ptr(counts))
    if events < 0:
        raise ValueError("bad flow or tensor")
    return counts, int(events)


def quantize_after_im2col(cv: OrcConv, fmt: int, x: np.ndarray):
    """Square-block quantization of the conventional explicit im2col matrix
    (K x J, channel-major rows, batch-major columns).  Returns per-entry
    codes, scales and referenced activation index (-1 = padding) as [K][J]
    arrays, and the tensor scale."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    K = cv.k_h * cv.k_w * cv.c_in
    J = cv.h_out * cv.w_out * cv.n
    codes = np.zeros((K, J), dtype=np.uint8)
    scales = np.zeros((K, J), dtype=np.uint8)
    src = np.zeros((K, J), dtype=np.int64)
    t = np.zeros(1, dtype=np.float32)
    rc = lib().orc_quantize_after_im2col(ctypes.byref(cv), fmt, _ptr(x), _ptr(codes),
                                         _ptr(scales), _ptr(src), _ptr(t))
    if rc != 0:
        raise ValueError("quantize_after_im2col needs K and J multiples of 8")
    return codes, scales, src, float(t[0])
