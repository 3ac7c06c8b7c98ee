"""Pins of the MXFP4 oracle (oracle/mxfp4.py) against values the format fixes.  CPU only."""

import numpy as np
import pytest

from oracle import mxfp4


def test_e2m1_values_round_trip():
    """Every representable magnitude (and its negative) quantises to itself at scale 1."""
    vals = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -1.5, -2, -3, -4, -6, 0])
    x = np.zeros(32)
    x[:16] = vals
    x[16] = 6.0                         # block max 6 -> floor(log2 6) = 2 -> scale 2^0
    codes, sb = mxfp4.quantize(x)
    assert sb[0] == 127
    np.testing.assert_array_equal(mxfp4.dequantize(codes, sb), x)
    np.testing.assert_array_equal(codes[:8], np.arange(8))
    np.testing.assert_array_equal(codes[8:15], 8 + np.array([1, 2, 3, 4, 5, 6, 7]))


@pytest.mark.parametrize("mid,expect", [(0.25, 0.0), (0.75, 1.0), (1.25, 1.0), (1.75, 2.0),
                                        (2.5, 2.0), (3.5, 4.0), (5.0, 4.0)])
def test_ties_go_to_the_even_code(mid, expect):
    x = np.zeros(32)
    x[0] = 4.0                          # scale 2^0 (floor(log2 4) - 2 = 0)
    x[1] = mid
    x[2] = -mid
    codes, sb = mxfp4.quantize(x)
    assert sb[0] == 127
    deq = mxfp4.dequantize(codes, sb)
    assert deq[1] == expect and deq[2] == -expect


def test_scale_is_floor_log2_max_minus_two_and_saturates():
    rng = np.random.default_rng(0)
    for k in range(-20, 20):
        x = rng.standard_normal(32) * 2.0 ** k
        codes, sb = mxfp4.quantize(x)
        amax = np.abs(x).max()
        assert sb[0] == int(np.floor(np.log2(amax))) - 2 + 127
        deq = mxfp4.dequantize(codes, sb)
        scale = 2.0 ** (int(sb[0]) - 127)
        # the largest element maps into [4, 8) * scale and saturates at 6 * scale
        assert np.abs(deq).max() <= 6 * scale
        # every element is within half a grid step of the nearest value (step <= 2 * scale)
        assert np.all(np.abs(deq - np.clip(x, -6 * scale, 6 * scale)) <= 1.0 * scale + 1e-300)
    x = np.zeros(32)
    x[0] = 7.9                         # 7.9 / 2^0 saturates to 6
    codes, sb = mxfp4.quantize(x)
    assert sb[0] == 127 and mxfp4.dequantize(codes, sb)[0] == 6.0


def test_zero_block_and_negative_zero_rounding():
    codes, sb = mxfp4.quantize(np.zeros(64))
    assert np.all(codes == 0) and np.all(sb == 0)
    assert np.all(mxfp4.dequantize(codes, sb) == 0)
    x = np.zeros(32)
    x[0] = 4.0
    x[1] = -0.1                        # rounds to magnitude 0, keeps the sign bit
    codes, _ = mxfp4.quantize(x)
    assert codes[1] == 8


def test_worked_block_and_packing():
    """A block with max 12 has scale 2^1: 12 -> 6, 5 -> 2.5 -> tie -> 2 (value 4), -0.7 ->
    -0.35 -> 0.5 (value -1), 1 -> 0.5 (value 1)."""
    x = np.zeros(32)
    x[:4] = [12.0, 5.0, -0.7, 1.0]
    codes, sb = mxfp4.quantize(x)
    assert sb[0] == 128
    np.testing.assert_array_equal(codes[:4], [7, 4, 9, 1])
    np.testing.assert_array_equal(mxfp4.dequantize(codes, sb)[:4], [12.0, 4.0, -1.0, 1.0])
    p = mxfp4.pack(codes)
    assert p.shape == (16,) and p[0] == 7 | (4 << 4) and p[1] == 9 | (1 << 4)
    np.testing.assert_array_equal(mxfp4.unpack(p), codes)
