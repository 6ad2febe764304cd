"""Pins for the oracle's integer-only requantization (get_mn, requant_int).

"Quantization" blog, 量化模式: integer quantization (power of two) replaces float
arithmetic by integer operations; FQ-ViT article, LayerNorm code: get_MN writes a
positive real as an 8-bit mantissa M and a shift N.  The pins are closed forms of
get_MN, its defining inequality in exact rationals, an exact-rational brute force
of the rounding (Python's round() on Fraction rounds half to even), hand-built
ties, and the agreement with the binary32 requant where both are exact.  CPU only.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle as O


@pytest.mark.parametrize("k", range(0, 25))
def test_get_mn_of_powers_of_two(k):
    # x = 2^-k: mantissa 2^7 at shift 7 + k until the shift saturates at 31
    m, n = O.get_mn(2.0 ** -k)
    assert (m, n) == ((128, 7 + k) if 7 + k <= 31 else (128 >> (7 + k - 31), 31))


def test_get_mn_closed_forms():
    assert O.get_mn(1.0) == (128, 7)
    assert O.get_mn(3.0) == (192, 6)          # 3 = 192 * 2^-6
    assert O.get_mn(0.3) == (153, 9)          # floor(0.3 * 512) = 153
    assert O.get_mn(200.0) == (200, 0)        # shift clamps at 0
    assert O.get_mn(300.0) == (255, 0)        # mantissa clamps at 2^bit - 1
    assert O.get_mn(2.0 ** -40) == (0, 31)    # shift clamps at 31: floor(2^-9) = 0


def test_get_mn_brackets_x_exactly():
    rng = np.random.default_rng(1)
    for x in np.exp(rng.uniform(np.log(2.0 ** -20), np.log(100.0), 500)).astype(np.float32):
        m, n = O.get_mn(x)
        assert 128 <= m <= 255 and 0 <= n <= 31
        fx = Fraction(float(x))
        assert Fraction(m, 2 ** n) <= fx < Fraction(m + 1, 2 ** n)


def _brute(acc, m, n, relu, z, lo, hi):
    out = np.empty(acc.shape, np.int64)
    for idx in np.ndindex(acc.shape):
        c = idx[-1]
        q = round(Fraction(int(acc[idx]) * int(m[c]), 2 ** int(n[c])))   # half to even
        if relu:
            q = max(q, 0)
        out[idx] = min(max(q + z, lo), hi)
    return out


@pytest.mark.parametrize("relu,qtype,z", [(False, O.INT8, 0), (True, O.UINT8, 7), (False, O.UINT8, 128),
                                          (True, O.UINT4, 3), (False, O.INT4, -2)])
def test_requant_int_matches_exact_rationals(relu, qtype, z):
    rng = np.random.default_rng(2 + z)
    ch = 6
    m = rng.integers(128, 256, ch)
    n = np.array([0, 1, 5, 12, 20, 31])
    acc = rng.integers(-(1 << 31), 1 << 31, size=(40, ch), dtype=np.int64)
    acc[:20] = rng.integers(-5000, 5000, size=(20, ch))   # values that land inside the code range
    lo, hi = O.qrange(qtype)
    got = O.requant_int(acc, m, n, O.EPI_RELU if relu else O.EPI_NONE, z, qtype)
    assert np.array_equal(got, _brute(acc, m, n, relu, z, lo, hi))


def test_requant_int_ties_go_to_even():
    # acc * M / 2^N = k + 1/2 exactly: the result is the even one of k, k + 1
    m = np.array([128])
    n = np.array([8])                          # acc * 128 / 256 = acc / 2
    acc = np.array([[1], [3], [5], [-1], [-3], [7]], np.int64)
    got = O.requant_int(acc, m, n, O.EPI_NONE, 0, O.INT8)
    assert got[:, 0].tolist() == [0, 2, 2, 0, -2, 4]


def test_requant_int_equals_float_path_where_both_are_exact():
    # x = M * 2^-N with an 8-bit M is exact in binary32, and for |acc| < 2^16 so is
    # float(acc) * x: both paths round the same rational to even
    rng = np.random.default_rng(3)
    ch = 16
    m = rng.integers(128, 256, ch)
    n = rng.integers(8, 20, ch)
    x = np.array([math.ldexp(int(a), -int(b)) for a, b in zip(m, n)], np.float32)
    acc = rng.integers(-(1 << 16), 1 << 16, size=(300, ch), dtype=np.int64)
    for epi, qtype, z in [(O.EPI_NONE, O.INT8, 0), (O.EPI_RELU, O.UINT8, 9)]:
        a = O.requant_int(acc, m, n, epi, z, qtype)
        b = O.requant(acc, x, epi, z, qtype)
        assert np.array_equal(a, b)
