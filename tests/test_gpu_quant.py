"""GPU parity of the quantizer and the dequantizer against the CPU oracle:
codes, block scales, tensor scale and amax bit-exact (MicroQonv, arXiv
2609.28358, §III-A, §IV-B)."""
import numpy as np
import pytest
import torch

import microscaling_quantized_convolution_mx_amd as mx
import oracle as O
from microscaling_quantized_convolution_mx_amd import workloads as WL
from gpu_util import DEV, assert_quant_equal, gpu_quantize, ofmt, oracle_quantize, say

pytestmark = pytest.mark.gpu

FMTS = [mx.MX_E2M1, mx.MX_E2M3, mx.MX_E4M3, mx.MX_E3M2]

# (n, c_in, c_out, h, w, k, stride, pad): ragged block rows (N/8 not a multiple
# of the 32 blocks a wavefront covers), several workgroups, stride 2
SHAPES = [
    (40, 24, 16, 5, 3, 3, 1, 1),
    (8, 16, 32, 9, 7, 3, 2, 1),
    (264, 8, 8, 4, 4, 1, 1, 0),
    (16, 64, 136, 6, 5, 3, 1, 0),
    (72, 16, 24, 9, 8, 3, 1, 1),    # X 1296 and dY 1944 blocks: the bulk path
]


# Tensors above the quantizer's one-workgroup limit (256 blocks) take the
# bulk path (an amax pass, then two lanes per block); the edge cases below
# run at both sizes.  BULK: H, W, C, N with 1296 blocks, N/8 = 9 blocks per
# channel row, so the 32-block groups of a wave straddle positions.
BULK_BLOCKS = 1100
BULK = (9, 8, 16, 72)


def bulk_desc(fmt):
    h, w, c, n = BULK
    return mx.desc(n, c, c, h, w, 1, 1, elem_fmt=fmt)


def src_for(d, role, seed, dist="normal", sigma=1.0):
    lay = WL.ConvLayer(d.n, d.c_in, d.c_out, d.h, d.w, d.k_h, d.k_w, d.stride_h, d.stride_w,
                       d.pad_h, d.pad_w)
    if role == mx.MX_ROLE_ACT:
        return WL.gen_x(lay, dist, seed)
    if role == mx.MX_ROLE_WEIGHT:
        return WL.gen_w(lay, seed)
    return WL.gen_dy(lay, sigma, seed)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("role,rounding", [(mx.MX_ROLE_ACT, mx.MX_RNE), (mx.MX_ROLE_WEIGHT, mx.MX_RNE),
                                           (mx.MX_ROLE_GRAD, mx.MX_SR), (mx.MX_ROLE_GRAD, mx.MX_RNE),
                                           (mx.MX_ROLE_WEIGHT, mx.MX_SR)])
def test_quantize_bit_exact(fmt, shape, role, rounding):
    n, ci, co, h, w, k, s, p = shape
    d = mx.desc(n, ci, co, h, w, k, k, s, s, p, p, elem_fmt=fmt)
    say("quantize", fmt, shape, role, rounding)
    src = src_for(d, role, seed=hash((fmt, shape, role)) % 1000)
    gq = gpu_quantize(d, role, src, rounding, seed=123)
    oq = oracle_quantize(d, role, src, rounding, seed=123)
    assert_quant_equal(gq, oq, f"fmt {fmt} role {role}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dist", ["halfnormal", "silu", "uniform"])
def test_quantize_distributions(fmt, dist):
    d = mx.desc(64, 32, 32, 7, 7, 3, 3, 1, 1, 1, 1, elem_fmt=fmt)
    say("quantize dist", fmt, dist)
    src = WL.gen_tensor((7, 7, 32, 64), dist, 77)
    assert_quant_equal(gpu_quantize(d, mx.MX_ROLE_ACT, src), oracle_quantize(d, mx.MX_ROLE_ACT, src))


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_extreme_magnitudes(fmt):
    # tiny (subnormal fp32), huge, ties on the grid, signed zeros
    d = mx.desc(16, 16, 16, 2, 2, 1, 1, elem_fmt=fmt)
    say("quantize extremes", fmt)
    g = torch.Generator().manual_seed(5)
    x = torch.randn(2, 2, 16, 16, generator=g)
    x[0, 0] *= 1e-38           # a block of fp32 subnormals next to normal blocks
    x[0, 1] *= 1e-30
    x[1, 0] *= 3e30
    x[1, 1, 0, :4] = torch.tensor([0.0, -0.0, 1e-45, -1e-45])
    for role, rnd in ((mx.MX_ROLE_ACT, mx.MX_RNE), (mx.MX_ROLE_GRAD, mx.MX_SR)):
        assert_quant_equal(gpu_quantize(d, role, x, rnd, seed=9), oracle_quantize(d, role, x, rnd, seed=9))
    # only tiny values: T itself subnormal
    xs = x * 1e-8
    assert_quant_equal(gpu_quantize(d, mx.MX_ROLE_ACT, xs), oracle_quantize(d, mx.MX_ROLE_ACT, xs))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("min_blocks", [0, BULK_BLOCKS])
def test_quantize_grid_ties(fmt, min_blocks):
    # T = 1 (amax = 448 * max) and every other block holds the element
    # maximum, so its scale is exactly 1 and the grid midpoints placed in it
    # are exact ties after scaling: both sides must pick the even code
    grid = O.fmt_grid(ofmt(fmt))
    mids = (grid[1:] + grid[:-1]) / 2
    vals = np.concatenate([mids, -mids, grid[:-1]]).astype(np.float32)
    nchunks = -(-vals.size // 63)
    npos = max(nchunks + 1, min_blocks)
    d = mx.desc(8, 8, 8, 1, npos, 1, 1, elem_fmt=fmt)
    x = np.zeros((1, npos, 8, 8), dtype=np.float32)
    for p in range(npos - 1):
        blk = x[0, p].reshape(-1)
        c = p % nchunks
        chunk = vals[c * 63:(c + 1) * 63]
        blk[0] = grid[-1]
        blk[1:1 + chunk.size] = chunk
    x[0, npos - 1, 7, 7] = 448.0 * grid[-1]
    say("quantize ties", fmt)
    xt = torch.from_numpy(x)
    oq = oracle_quantize(d, mx.MX_ROLE_ACT, xt)
    assert oq.t == 1.0 and np.all(oq.scales[:-1] == 0x38)
    assert_quant_equal(gpu_quantize(d, mx.MX_ROLE_ACT, xt), oq)
    for rnd in (mx.MX_SR,):
        assert_quant_equal(gpu_quantize(d, mx.MX_ROLE_GRAD, xt, rnd, 11),
                           oracle_quantize(d, mx.MX_ROLE_GRAD, xt, rnd, 11))


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_extreme_magnitudes_bulk(fmt):
    d = bulk_desc(fmt)
    say("quantize extremes bulk", fmt)
    g = torch.Generator().manual_seed(6)
    x = torch.randn(*BULK, generator=g)
    x[0, 0] *= 1e-38           # whole positions of fp32 subnormals, tiny and huge values
    x[3, 5] *= 1e-30
    x[8, 7, :8] *= 3e30        # the last position: its first channel block only
    x[4, 4, 0, :4] = torch.tensor([0.0, -0.0, 1e-45, -1e-45])
    for role, rnd in ((mx.MX_ROLE_ACT, mx.MX_RNE), (mx.MX_ROLE_GRAD, mx.MX_SR), (mx.MX_ROLE_GRAD, mx.MX_RNE)):
        assert_quant_equal(gpu_quantize(d, role, x, rnd, seed=9), oracle_quantize(d, role, x, rnd, seed=9))
    # without the huge values: blocks of tiny elements next to normal ones
    xm = x.clone()
    xm[8, 7] = torch.randn(16, 72, generator=g)
    for role, rnd in ((mx.MX_ROLE_ACT, mx.MX_RNE), (mx.MX_ROLE_GRAD, mx.MX_SR)):
        assert_quant_equal(gpu_quantize(d, role, xm, rnd, seed=4), oracle_quantize(d, role, xm, rnd, seed=4))
    xs = xm * 1e-8             # T itself subnormal
    assert_quant_equal(gpu_quantize(d, mx.MX_ROLE_ACT, xs), oracle_quantize(d, mx.MX_ROLE_ACT, xs))


@pytest.mark.parametrize("size", ["small", "bulk"])
def test_quantize_sr_thresholds(size):
    # T = 1 (amax 448 * 6) and a 6 in every other block (scale exactly 1), so
    # that v = |x| exactly; every other element sits on, one representable
    # step below or one step above its own stochastic-rounding threshold u
    # (the oracle's uniform for that element), in each part of the E2M1 grid
    # (below 0.5, [0.5, 1), [1, 1.5), [2, 3), [4, 6)).  Round up iff frac > u
    # (MicroQonv, arXiv 2609.28358, §III-A; the rule of the oracle): both
    # sides must take the same decision at the threshold itself.
    shape = (2, 2, 16, 16) if size == "small" else BULK
    h, w, c, n = shape
    d = mx.desc(n, c, c, h, w, 1, 1, elem_fmt=mx.MX_E2M1)
    seed = 77
    u = np.array([O.sr_uniform(seed, i) for i in range(h * w * c * n)], np.float64).reshape(shape)
    rng = np.random.default_rng(5 if size == "small" else 6)
    region = rng.integers(0, 5, shape)
    lo = np.array([0.0, 0.5, 1.0, 2.0, 4.0])[region]
    step = np.array([0.5, 0.5, 0.5, 1.0, 2.0])[region]
    res = np.array([2.0 ** -24, 2.0 ** -23, 2.0 ** -22, 2.0 ** -22, 2.0 ** -22])[region]  # finest frac there
    frac = np.clip(np.floor(u / res) * res + rng.integers(-1, 2, shape) * res, 0.0, 1.0 - res)
    v = lo + frac * step
    assert np.array_equal(v.astype(np.float32).astype(np.float64), v)  # every value exact in fp32
    x = (v * np.where(rng.random(shape) < 0.5, -1.0, 1.0)).astype(np.float32)
    x[:, :, ::8, ::8] = 6.0
    x[0, 0, 0, 0] = 448.0 * 6.0
    ties = np.sum((frac == u) & (u > 0))
    assert ties > (5 if size == "small" else 500), ties   # elements exactly on their threshold
    say("quantize SR thresholds", size)
    xt = torch.from_numpy(x)
    oq = oracle_quantize(d, mx.MX_ROLE_GRAD, xt, mx.MX_SR, seed)
    assert oq.t == 1.0 and np.sum(oq.scales != 0x38) == 1
    assert_quant_equal(gpu_quantize(d, mx.MX_ROLE_GRAD, xt, mx.MX_SR, seed), oq)


@pytest.mark.parametrize("bad", [float("nan"), float("inf"), float("-inf")])
def test_quantize_nonfinite_bulk(bad):
    d = bulk_desc(mx.MX_E2M1)
    x = WL.gen_tensor(BULK, "normal", 13)
    x[6, 2, 11, 70] = bad
    say("quantize nonfinite bulk", bad)
    for role, rnd in ((mx.MX_ROLE_ACT, mx.MX_RNE), (mx.MX_ROLE_GRAD, mx.MX_SR)):
        gq = gpu_quantize(d, role, x, rnd, 2)
        assert_quant_equal(gq, oracle_quantize(d, role, x, rnd, 2))
        assert np.isnan(gq.tensor_scale.item())
        assert (gq.scales[:gq.nblocks] == 0x7F).all()


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_zero_and_given_amax_bulk(fmt):
    d = bulk_desc(fmt)
    say("quantize zero / given amax bulk", fmt)
    z = torch.zeros(*BULK)
    gq = gpu_quantize(d, mx.MX_ROLE_GRAD, z, mx.MX_SR, 1)
    assert_quant_equal(gq, oracle_quantize(d, mx.MX_ROLE_GRAD, z, mx.MX_SR, 1))
    assert gq.tensor_scale.item() == 0.0
    x = WL.gen_tensor(BULK, "normal", 21)
    true_amax = float(x.abs().max())
    for a in (true_amax * 3.0, true_amax * 0.25):
        assert_quant_equal(gpu_quantize(d, mx.MX_ROLE_ACT, x, amax=a),
                           oracle_quantize(d, mx.MX_ROLE_ACT, x, amax=np.float32(a)), f"amax {a}")
    assert np.isnan(gpu_quantize(d, mx.MX_ROLE_ACT, x, amax=float("nan")).tensor_scale.item())


@pytest.mark.parametrize("bad", [float("nan"), float("inf"), float("-inf")])
def test_quantize_nonfinite(bad):
    d = mx.desc(16, 16, 16, 3, 3, 1, 1, elem_fmt=mx.MX_E2M1)
    x = WL.gen_tensor((3, 3, 16, 16), "normal", 3)
    x[2, 1, 5, 9] = bad
    say("quantize nonfinite", bad)
    gq = gpu_quantize(d, mx.MX_ROLE_ACT, x)
    assert_quant_equal(gq, oracle_quantize(d, mx.MX_ROLE_ACT, x))
    assert np.isnan(gq.tensor_scale.item())
    assert (gq.scales[:gq.nblocks] == 0x7F).all()


def test_quantize_all_zero_and_empty():
    d = mx.desc(16, 16, 16, 3, 3, 1, 1, elem_fmt=mx.MX_E2M3)
    x = torch.zeros(3, 3, 16, 16)
    say("quantize zero")
    gq = gpu_quantize(d, mx.MX_ROLE_GRAD, x, mx.MX_SR, 1)
    assert_quant_equal(gq, oracle_quantize(d, mx.MX_ROLE_GRAD, x, mx.MX_SR, 1))
    assert gq.tensor_scale.item() == 0.0
    # empty batch: nothing to quantize, T and amax still published as 0
    de = mx.desc(0, 16, 16, 3, 3, 1, 1, elem_fmt=mx.MX_E2M1)
    q = mx.QTensor(de, mx.MX_ROLE_ACT, DEV)
    q.tensor_scale.fill_(5.0)
    q.amax.fill_(5.0)
    mx.mx_quantize_cbf(de, mx.MX_ROLE_ACT, torch.empty(0, device=DEV), q)
    torch.cuda.synchronize()
    assert q.tensor_scale.item() == 0.0 and q.amax.item() == 0.0


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_given_amax(fmt):
    d = mx.desc(24, 16, 16, 4, 4, 3, 3, 1, 1, 1, 1, elem_fmt=fmt)
    x = WL.gen_tensor((4, 4, 16, 24), "normal", 8)
    true_amax = float(x.abs().max())
    say("quantize given amax", fmt)
    for a in (true_amax * 3.0, true_amax * 0.25):  # larger: coarser scales; smaller: saturation
        gq = gpu_quantize(d, mx.MX_ROLE_ACT, x, amax=a)
        oq = oracle_quantize(d, mx.MX_ROLE_ACT, x, amax=np.float32(a))
        assert_quant_equal(gq, oq, f"amax {a}")
    gq = gpu_quantize(d, mx.MX_ROLE_ACT, x, amax=float("nan"))
    assert np.isnan(gq.tensor_scale.item())


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("role", [mx.MX_ROLE_ACT, mx.MX_ROLE_WEIGHT, mx.MX_ROLE_GRAD])
def test_dequantize_bit_exact(fmt, role):
    d = mx.desc(40, 24, 16, 5, 3, 3, 3, 1, 1, 1, 1, elem_fmt=fmt)
    say("dequantize", fmt, role)
    src = src_for(d, role, 31)
    rnd = mx.MX_SR if role == mx.MX_ROLE_GRAD else mx.MX_RNE
    gq = gpu_quantize(d, role, src, rnd, 3)
    out = torch.empty(src.shape, device=DEV)
    mx.mx_dequantize(d, role, gq, out)
    torch.cuda.synchronize()
    ref = O.dequantize(oracle_quantize(d, role, src, rnd, 3))
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_dequantize_nonfinite_tensor():
    d = mx.desc(8, 8, 8, 2, 2, 1, 1, elem_fmt=mx.MX_E2M1)
    x = WL.gen_tensor((2, 2, 8, 8), "normal", 2)
    x[0, 0, 0, 0] = float("nan")
    gq = gpu_quantize(d, mx.MX_ROLE_ACT, x)
    out = torch.empty(x.shape, device=DEV)
    mx.mx_dequantize(d, mx.MX_ROLE_ACT, gq, out)
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
