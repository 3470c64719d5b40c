"""The compact 3-bit activation codes of the latent-replay buffer.

After a ReLU every activation is non-negative, so the E2M1 sign bit carries
nothing and can be dropped, leaving 3-bit codes: 3 + 8/64 = 3.125 bits per
element with the block scale (MicroQonv, arXiv 2609.28358, §VI-A;
§VII stores the replay buffer that way).  The oracle's UE2M1 format is that
reading: E2M1 quantization with the sign dropped, packed as a 3-bit stream."""
import numpy as np
import pytest

import oracle as O


@pytest.fixture(scope="module")
def orc():
    O.build()
    return O


def act(shape, seed, relu=True):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    return np.maximum(x, 0.0).astype(np.float32) if relu else x


def test_codes_are_the_e2m1_magnitudes(orc):
    # any sign: same T, same block scales, codes = E2M1 codes without the sign bit
    x = act((3, 5, 16, 24), 1, relu=False)
    q4 = O.quantize(O.ACT, O.E2M1, x)
    q3 = O.quantize(O.ACT, O.UE2M1, x)
    assert O.fmt_bits(O.UE2M1) == 3
    assert q3.t == q4.t and np.array_equal(q3.scales, q4.scales)
    assert np.array_equal(q3.codes, q4.codes & 7)
    assert int(q3.codes.max()) <= 7


def test_post_relu_dequantizes_exactly_like_e2m1(orc):
    x = act((4, 4, 32, 16), 2)
    x[0, 0, :8, :8] = 0.0  # an all-zero block
    q4 = O.quantize(O.ACT, O.E2M1, x)
    q3 = O.quantize(O.ACT, O.UE2M1, x)
    assert np.array_equal(O.dequantize(q3).view(np.uint32), O.dequantize(q4).view(np.uint32))


def test_three_bit_stream_packing(orc):
    # element e of a block at bits 3e .. 3e+2, little-endian: codes 0..7 form
    # the 24-bit value 0xFAC688 (worked by hand: sum of c << 3c)
    codes = np.tile(np.arange(8, dtype=np.uint8), 8)
    p = O.pack(O.UE2M1, codes)
    assert p.size == 24
    assert list(p[:3]) == [0x88, 0xC6, 0xFA]
    assert list(p[3:6]) == [0x88, 0xC6, 0xFA]


def test_three_point_one_two_five_bits_per_element(orc):
    # §VI-A: 3 bits per activation pixel + 8/64 for the E4M3 block scale
    x = act((8, 8, 64, 16), 3)
    q = O.quantize(O.ACT, O.UE2M1, x)
    bits = (q.packed().size + q.scales.size) * 8 / x.size
    assert bits == 3.125
