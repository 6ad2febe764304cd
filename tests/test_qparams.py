"""Quantization parameters from a real range (iqnn_choose_qparams): the oracle's
choose_qparams pinned to closed forms and to the properties the pages' MinMax
scheme implies (FQ-ViT article, §3.1; Horizon QAT talk, section 三), and the C
entry point (host code, no GPU) equal to the oracle bit for bit."""
import os

import numpy as np
import pytest

import oracle as O
from integer_quantized_nn_amd import binding as B

U8, I8, U4, I4 = O.UINT8, O.INT8, O.UINT4, O.INT4
LIB_TYPE = {U8: B.UINT8, I8: B.INT8, U4: B.UINT4, I4: B.INT4}
f32 = np.float32


@pytest.mark.parametrize("vmin,vmax,qt,sym,scale,zp", [
    (0.0, 255.0, U8, False, 1.0, 0),          # codes equal the reals
    (-128.0, 127.0, U8, False, 1.0, 128),
    (0.0, 255.0, I8, False, 1.0, -128),
    (2.0, 10.0, U8, False, f32(10.0) / f32(255), 0),      # positive range widened to hold 0
    (-10.0, -2.0, U8, False, f32(10.0) / f32(255), 255),  # negative range: 0 at the top code
    (-0.5, 7.0, U4, False, 0.5, 1),
    (-1.25, 6.25, U4, False, 0.5, 2),          # min / S = -2.5 exactly: ties to even (not 3)
    (-1.75, 5.75, U4, False, 0.5, 4),          # min / S = -3.5: ties to even (4)
    (-1.0, 3.0, U4, False, f32(4.0) / f32(15), 4),       # -min / S = 3.75 -> 4
    (-1.0, 1.0, I8, True, f32(1.0) / f32(127), 0),
    (-2.0, 0.5, I8, True, f32(2.0) / f32(127), 0),
    (0.25, 3.5, I4, True, 0.5, 0),
    (0.0, 0.0, U8, False, 1.0, 0),            # zero range: every value is the code Z
    (0.0, 0.0, I8, False, 1.0, -128),
    (0.0, 0.0, I4, True, 1.0, 0),
])
def test_oracle_closed_forms(vmin, vmax, qt, sym, scale, zp):
    s, z = O.choose_qparams(vmin, vmax, qt, sym)
    assert s.dtype == np.float32 and s == f32(scale) and z == zp


@pytest.mark.parametrize("qt", [U8, I8, U4, I4])
def test_oracle_range_maps_onto_the_codes(qt):
    """The real 0 is exactly the code Z, the range's ends land on the end codes up to
    the one code that rounding Z can move them, and every real in the range comes back
    within one scale step (the oracle's quantize / dequantize, pinned elsewhere)."""
    rng = np.random.default_rng(qt)
    lo, hi = O.qrange(qt)
    for _ in range(300):
        a, b = np.sort(rng.normal(0, 10.0 ** rng.uniform(-6, 6), 2)).astype(np.float32)
        if rng.random() < 0.2:
            a = f32(abs(a))   # all-positive ranges
        a, b = min(a, b), max(a, b)
        for sym in ([False, True] if lo < 0 else [False]):
            s, z = O.choose_qparams(a, b, qt, sym)
            assert lo <= z <= hi
            assert O.dequantize(np.array([z], np.int32), s, z)[0] == 0.0
            mn, mx = min(a, f32(0)), max(b, f32(0))
            qmn = int(O.quantize(np.array([mn], np.float32), s, z, qt)[0])
            qmx = int(O.quantize(np.array([mx], np.float32), s, z, qt)[0])
            if sym:
                assert max(abs(qmn), abs(qmx)) == hi
            else:
                assert qmn - lo <= 1 and hi - qmx <= 1
            x = rng.uniform(mn, mx, 64).astype(np.float32)
            back = O.dequantize(O.quantize(x, s, z, qt), s, z)
            assert np.all(np.abs(back.astype(np.float64) - x) <= 1.0001 * float(s))


def test_oracle_catches_a_planted_mistake():
    """A half-away-from-zero Z (a plausible slip) would change the tie case above."""
    s, z = O.choose_qparams(-1.25, 6.25, U4)
    assert z == 2 and int(np.floor(2.5 + 0.5)) == 3


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libiqnn.so is not built (run __graft_entry__.build())")
    return B.lib()


def test_library_equals_oracle(lib):
    rng = np.random.default_rng(7)
    n = 0
    for qt in (U8, I8, U4, I4):
        lo, _ = O.qrange(qt)
        for _ in range(1500):
            a, b = np.sort(rng.normal(0, 10.0 ** rng.uniform(-30, 30), 2)).astype(np.float32)
            if rng.random() < 0.1:
                a = f32(0)
            if rng.random() < 0.1:
                b = a
            a, b = min(a, b), max(a, b)
            for sym in ([False, True] if lo < 0 else [False]):
                want = O.choose_qparams(a, b, qt, sym)
                got = B.iqnn_choose_qparams(a, b, LIB_TYPE[qt], sym)
                assert got[1] == want[1] and got[0].view(np.uint32) == want[0].view(np.uint32), (a, b, qt, sym)
                n += 1
    assert n > 8000


def test_library_rejects_bad_ranges(lib):
    for args in [(np.nan, 1.0, B.UINT8, False), (0.0, np.inf, B.UINT8, False), (2.0, 1.0, B.INT8, False),
                 (-1.0, 1.0, B.UINT8, True), (-1.0, 1.0, B.INT32, False)]:
        with pytest.raises(B.IqnnError) as ei:
            B.iqnn_choose_qparams(*args)
        assert ei.value.status == 1
    with pytest.raises(B.IqnnError) as ei:
        B.iqnn_choose_qparams(-3e38, 3e38, B.UINT8, False)
    assert ei.value.status == 4
