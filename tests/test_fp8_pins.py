"""Pins of the E4M3 oracle (oracle/wsp_fp8.py) against the format's own
definition (OCP 8-bit floating point, E4M3: bias 7, 3 mantissa bits, no
infinities, S.1111.111 = NaN, largest finite 448) -- closed forms, round
trips, tie cases and error bounds -- independent of the encoder's search."""
import numpy as np

import oracle as O


def test_decode_closed_forms():
    cases = {0x00: 0.0, 0x38: 1.0, 0xB8: -1.0, 0x7E: 448.0, 0xFE: -448.0, 0x01: 2.0 ** -9,
             0x07: 7 / 8 * 2.0 ** -6, 0x08: 2.0 ** -6, 0x40: 2.0, 0x3C: 1.5, 0x77: 240.0, 0x30: 0.5}
    for c, v in cases.items():
        assert O.e4m3_decode(np.uint8(c)) == v, hex(c)
    assert np.isnan(O.e4m3_decode(np.uint8(0x7F))) and np.isnan(O.e4m3_decode(np.uint8(0xFF)))


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(O.e4m3_encode(O.e4m3_decode(codes)), codes)   # 0x80 is -0.0


def test_signed_zero():
    assert O.e4m3_encode(-0.0) == 0x80 and O.e4m3_encode(0.0) == 0x00
    assert O.e4m3_encode(-1e-12) == 0x80 and O.e4m3_encode(1e-12) == 0x00
    assert O.e4m3_decode(np.uint8(0x80)) == 0.0 and np.signbit(O.e4m3_decode(np.uint8(0x80)))


def test_ties_go_to_even_and_saturate():
    assert O.e4m3_encode(1.0625) == 0x38          # between 1.0 (0x38) and 1.125 (0x39)
    assert O.e4m3_encode(1.1875) == 0x3A          # between 1.125 (0x39) and 1.25 (0x3A)
    assert O.e4m3_encode(-1.0625) == 0xB8
    mid_sub = (7 / 8 * 2.0 ** -6 + 2.0 ** -6) / 2  # subnormal 0x07 / normal 0x08
    assert O.e4m3_encode(mid_sub) == 0x08
    assert O.e4m3_encode(2.0 ** -10) == 0x00      # half of the smallest subnormal: tie to 0
    assert O.e4m3_encode(1.5 * 2.0 ** -10) == 0x01
    for big in (448.0, 460.0, 1000.0, 1e30):
        assert O.e4m3_encode(big) == 0x7E and O.e4m3_encode(-big) == 0xFE


def test_relative_error_bound_and_monotone():
    x = np.geomspace(2.0 ** -6, 448.0, 20001)
    y = O.e4m3_decode(O.e4m3_encode(x))
    assert np.all(np.abs(y - x) <= 2.0 ** -4 * x * (1 + 1e-12))   # half a unit in the last place
    assert np.all(np.diff(O.e4m3_encode(x).astype(int)) >= 0)
    sub = np.linspace(0, 2.0 ** -6, 4001)
    assert np.all(np.abs(O.e4m3_decode(O.e4m3_encode(sub)) - sub) <= 2.0 ** -10 * (1 + 1e-12))


def test_quantize_per_head_scale():
    rng = np.random.default_rng([88, 1])
    x = (rng.standard_normal((50, 3, 128)) * np.array([1.0, 0.01, 30.0])[None, :, None]).astype(np.float32)
    amax = O.fp8_amax(x)
    assert np.allclose(amax, np.abs(x).max(axis=(0, 2)))
    code = O.fp8_quantize(x, amax)
    # the largest element of each head lands on +-448
    for h in range(3):
        i = np.unravel_index(np.argmax(np.abs(x[:, h])), x[:, h].shape)
        assert O.e4m3_decode(code[:, h][i]) == np.sign(x[:, h][i]) * 448.0
    back = O.fp8_dequantize(code, amax)
    assert np.all(np.abs(back - x) <= 2.0 ** -4 * np.abs(x) + amax[None, :, None] / 448 * 2.0 ** -9 * 1.01)
    # an all-zero head quantises to zero codes and dequantises to zero
    z = np.zeros((4, 1, 128), np.float32)
    assert np.all(O.fp8_quantize(z, O.fp8_amax(z)) == 0) and np.all(O.fp8_dequantize(O.fp8_quantize(z, [0.0]), [0.0]) == 0)
