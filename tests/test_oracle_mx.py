"""Pins of the oracle's original-microscaling quantizer: one E8M0 power-of-two
scale per 32x32 square block and no tensor scale (MicroQonv, arXiv
2609.28358, §II-D: the original format's block scale is a power of two in
E8M0; §IV-B: the method holds for any block scale).  The shared exponent
follows the OCP MX rule: floor(log2 amax_block) minus the exponent of the
element format's largest value, clamped to E8M0's [-127, 127].

Each check reaches the expected value by another route than the oracle's
bit-level code: hand-worked values, a brute-force search over powers of two
and over the element grid, closed-form invariances, and the exact Eq. 7
factorisation of a blocked dot product."""
import math

import numpy as np
import pytest

import oracle as O

FMTS = [O.E2M1, O.E2M3, O.E3M2, O.E4M3]
EMAX = {O.E2M1: 2, O.E2M3: 2, O.E3M2: 4, O.E4M3: 8}   # 6 = 1.5*2^2, 7.5, 28 = 1.75*2^4, 448 = 1.75*2^8


@pytest.fixture(scope="module")
def orc():
    O.lib()


def test_hand_worked_block(orc):
    # amax 7.9: floor(log2 7.9) = 2 = emax(E2M1), so the scale is 2^0
    # (E8M0 code 127) and the elements are rounded as they are:
    #   5.0 is the midpoint of 4 (code 6) and 6 (code 7): even code 6
    #   2.6 -> 3 (code 5); 0.3 -> 0.5 (code 1, above the midpoint 0.25)
    #  -0.75 is the midpoint of 0.5 and 1: even code 2, sign bit 8 -> 0xA
    #   7.9 saturates to 6 (code 7)
    x = np.zeros((1, 1, 32, 32), np.float32)
    x[0, 0, 0, :5] = [5.0, 2.6, 0.3, -0.75, 7.9]
    q = O.quantize_mx(O.ACT, O.E2M1, x)
    assert list(q.scales) == [127]
    assert list(q.codes[:5]) == [6, 5, 1, 0xA, 7]
    assert not q.codes[5:].any()
    assert list(q.exact()[0, 0, 0, :5]) == [4.0, 3.0, 0.5, -1.0, 6.0]
    # amax 0.01 = 1.28 * 2^-7: scale 2^(-7-2) = 2^-9 (code 118); 0.01 * 2^9 =
    # 5.12 lies nearer 6 than 4, so it dequantizes to 6 * 2^-9
    x[0, 0, 0, :5] = [0.01, 0, 0, 0, 0]
    q = O.quantize_mx(O.ACT, O.E2M1, x)
    assert list(q.scales) == [118] and q.codes[0] == 7
    assert q.exact()[0, 0, 0, 0] == 6 * 2.0 ** -9


def brute_force_e8m0(fmt, amax):
    # the largest k with 2^k <= amax, by search over every fp32 exponent
    if amax == 0.0:
        return 0
    k = max(k for k in range(-149, 128) if math.ldexp(1.0, k) <= amax)
    return min(max(k - EMAX[fmt], -127), 127) + 127


@pytest.mark.parametrize("fmt", FMTS)
def test_scale_exponent_matches_search(orc, fmt):
    rng = np.random.default_rng(fmt)
    vals = [0.0, 1e-45, 2.0 ** -126, 2.0 ** -127, 1.0, 2.0, 4.0, 448.0, 3.4e38]
    for k in (-140, -100, -3, 0, 1, 7, 60, 127):
        p = math.ldexp(1.0, k)
        vals += [p, float(np.nextafter(np.float32(p), np.float32(0))), float(np.nextafter(np.float32(p), np.float32(np.inf)))]
    vals += list(np.exp2(rng.uniform(-148, 127, 200)))
    for a in vals:
        a32 = float(np.float32(a))
        assert O.e8m0_code(fmt, a32) == brute_force_e8m0(fmt, a32), a32
    assert O.e8m0_code(fmt, float("inf"), True) == 0xFF


def grid_argmin(grid, v):
    # nearest grid value, ties to the even code; beyond the top: saturate
    if v >= grid[-1]:
        return len(grid) - 1
    d = np.abs(grid - v)
    best = np.flatnonzero(d == d.min())
    return int(best[0]) if best.size == 1 else int(best[best % 2 == 0][0])


@pytest.mark.parametrize("fmt", FMTS)
def test_elements_are_nearest_grid_points(orc, fmt):
    rng = np.random.default_rng(10 + fmt)
    x = (rng.standard_normal((2, 1, 32, 64)) * np.exp2(rng.integers(-6, 6, (2, 1, 32, 64)))).astype(np.float32)
    q = O.quantize_mx(O.ACT, fmt, x)
    grid = O.fmt_grid(fmt)
    sh = O.sign_shift(fmt)
    dims = q.dims
    for b in range(O.mx_nblocks(O.ACT, dims)):
        e = int(q.scales[b]) - 127
        for r in range(0, 32, 3):
            for c in range(0, 32, 5):
                si = O.mx_src_index(O.ACT, dims, b, r, c)
                xv = float(x.flat[si])
                v = abs(xv) / 2.0 ** e          # exact in fp64
                code = int(q.codes[b * 1024 + r * 32 + c])
                assert code & ((1 << sh) - 1) == grid_argmin(grid, v), (b, r, c, xv)
                assert (code >> sh) == (1 if np.signbit(xv) else 0)


@pytest.mark.parametrize("fmt", FMTS)
def test_power_of_two_equivariance(orc, fmt):
    rng = np.random.default_rng(20 + fmt)
    x = rng.standard_normal((1, 2, 32, 32)).astype(np.float32)
    q = O.quantize_mx(O.ACT, fmt, x)
    for k in (5, -9):
        qk = O.quantize_mx(O.ACT, fmt, (x * np.float32(2.0 ** k)).astype(np.float32))
        assert np.array_equal(qk.scales.astype(int), q.scales.astype(int) + k)
        assert np.array_equal(qk.codes, q.codes)


def test_zero_and_nonfinite_blocks(orc):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 3, 32, 32)).astype(np.float32)
    x[0, 0] = 0.0
    x[0, 1, 7, 9] = np.nan
    q = O.quantize_mx(O.ACT, O.E2M1, x)
    assert q.scales[0] == 0 and not q.codes[:1024].any()
    assert q.scales[1] == 0xFF and not q.codes[1024:2048].any()
    ref = O.quantize_mx(O.ACT, O.E2M1, x[:, 2:3].copy())
    assert q.scales[2] == ref.scales[0] and np.array_equal(q.codes[2048:], ref.codes)
    d = q.exact()
    assert (d[0, 0] == 0).all() and np.isnan(d[0, 1]).all() and np.isfinite(d[0, 2]).all()


def test_block_order(orc):
    # activations: blocks [H][W][C/32][N/32], element (r, c) = (channel, sample);
    # weights: blocks [Kh][Kw][Co/32][Ci/32], element (r, c) = (co, ci) of OIHW
    H, W, C, N = 2, 3, 64, 96
    dims = (H, W, C, N)
    seen = np.zeros(H * W * C * N, bool)
    for b in range(O.mx_nblocks(O.ACT, dims)):
        pos, rem = divmod(b, (C // 32) * (N // 32))
        cb, nb = divmod(rem, N // 32)
        for r in (0, 13, 31):
            for c in (0, 7, 31):
                si = O.mx_src_index(O.ACT, dims, b, r, c)
                assert si == (pos * C + cb * 32 + r) * N + nb * 32 + c
        for r in range(32):
            for c in range(32):
                seen[O.mx_src_index(O.ACT, dims, b, r, c)] = True
    assert seen.all()
    Co, Ci, Kh, Kw = 64, 32, 3, 2
    wd = (Co, Ci, Kh, Kw)
    for b in range(O.mx_nblocks(O.WEIGHT, wd)):
        tap, cob = divmod(b, Co // 32)   # Ci // 32 == 1
        kh, kw = divmod(tap, Kw)
        assert O.mx_src_index(O.WEIGHT, wd, b, 5, 17) == ((cob * 32 + 5) * Ci + 17) * Kh * Kw + kh * Kw + kw


def test_stochastic_rounding(orc):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, 1, 32, 32)).astype(np.float32)
    grid = O.fmt_grid(O.E2M1)
    qr = O.quantize_mx(O.GRAD, O.E2M1, x)
    e = int(qr.scales[0]) - 127
    v = np.abs(x[0, 0].astype(np.float64)) / 2.0 ** e
    seeds = range(400)
    vals = np.zeros((len(seeds), 32, 32))
    for i, s in enumerate(seeds):
        q = O.quantize_mx(O.GRAD, O.E2M1, x, O.SR, s)
        assert q.scales[0] == qr.scales[0]
        mag = (q.codes & 7).reshape(32, 32)
        vals[i] = grid[mag]
        # only the two neighbours of v
        lo = np.array([grid[grid <= t].max() if t < grid[-1] else grid[-1] for t in v.ravel()]).reshape(32, 32)
        hi = np.array([grid[grid >= t].min() if t < grid[-1] else grid[-1] for t in v.ravel()]).reshape(32, 32)
        assert np.all((vals[i] == lo) | (vals[i] == hi))
    inside = v < grid[-1]
    lo = np.array([grid[grid <= t].max() if t < grid[-1] else 0 for t in v.ravel()]).reshape(32, 32)
    hi = np.array([grid[grid >= t].min() if t < grid[-1] else 0 for t in v.ravel()]).reshape(32, 32)
    var = (v - lo) * (hi - v)
    err = np.abs(vals.mean(0) - v)
    assert np.all(err[inside] <= 4 * np.sqrt(var[inside] / len(seeds)) + 1e-12)


def test_blocked_dot_product_factorisation(orc):
    # Eq. 7 with E8M0 scales and T = 1: along K, a dot product of two MX
    # tensors is sum_j 2^(e_a,j + e_b,j) sum_{i in block j} q_a,i q_b,i
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((32, 64, 1, 1)) * np.array([1.0, 50.0])[None, :, None, None].repeat(32, 1)).astype(np.float32)
    x = rng.standard_normal((1, 1, 64, 32)).astype(np.float32)
    qw = O.quantize_mx(O.WEIGHT, O.E2M1, w)
    qx = O.quantize_mx(O.ACT, O.E2M1, x)
    grid = O.fmt_grid(O.E2M1)

    def val(q, b, r, c):
        code = int(q.codes[b * 1024 + r * 32 + c])
        return -grid[code & 7] if code & 8 else grid[code & 7]

    wf = qw.exact()[:, :, 0, 0]
    xf = qx.exact()[0, 0]
    for co in (0, 17, 31):
        for n in (0, 9, 31):
            total = 0.0
            for kb in range(2):
                ew, ex = int(qw.scales[kb]) - 127, int(qx.scales[kb]) - 127
                inner = sum(val(qw, kb, co, k) * val(qx, kb, k, n) for k in range(32))
                total += 2.0 ** (ew + ex) * inner
            assert total == float(wf[co] @ xf[:, n])


def test_fp32_dequantization_is_exact(orc):
    rng = np.random.default_rng(6)
    for fmt in FMTS:
        x = rng.standard_normal((2, 1, 32, 32))
        x[0] *= 1e-30            # scales near the bottom of E8M0: fp32 subnormal results
        x[1] *= 1e30
        x = x.astype(np.float32)
        q = O.quantize_mx(O.ACT, fmt, x)
        assert np.array_equal(q.dequantize().astype(np.float64), q.exact())
