"""Pins for the oracle's quantize / dequantize / packing / qparams / epilogue.

Each test ties the oracle to something other than itself: values printed on
the pages (tests/golden/*, each with its citation), closed forms, library
routines (torch's quantize_per_tensor / quantize_per_channel / dequantize) and
invariants (quantize(dequantize(q)) == q, monotonicity).  CPU only.
"""
import numpy as np
import pytest
import torch

import oracle as O
from conftest import read_golden

QT = {"INT8": O.INT8, "UINT8": O.UINT8, "INT4": O.INT4, "UINT4": O.UINT4}


def test_worked_example_from_page():
    for kind, value, scale, zp, qtype, expected in read_golden("quantize_worked_example.txt"):
        if kind == "quant":
            q = O.quantize(np.array([float(value)], np.float32), np.float32(scale), int(zp), QT[qtype])
            assert q[0] == int(expected)
        else:
            x = O.dequantize(np.array([int(value)], np.int32), np.float32(scale), int(zp))
            assert x[0] == np.float32(expected)


def test_round_half_to_even_ties():
    for xs, scale, zp, qtype, expected in read_golden("rne_ties.txt"):
        s = np.float32(scale)
        x = np.float32(float(xs) * float(s))  # exact: power-of-two scale
        assert float(x) / float(s) == float(xs)
        q = O.quantize(np.array([x]), s, int(zp), QT[qtype])
        assert q[0] == int(expected), (xs, qtype)


def test_saturation_boundaries():
    for x, scale, zp, qtype, expected in read_golden("saturation.txt"):
        q = O.quantize(np.array([float(x)], np.float32), np.float32(scale), int(zp), QT[qtype])
        assert q[0] == int(expected), (x, qtype)


def test_infinities_saturate_and_nan_is_rejected():
    q = O.quantize(np.array([np.inf, -np.inf], np.float32), 0.5, 0, O.INT8)
    assert list(q) == [127, -128]
    with pytest.raises(O.OracleError):
        O.quantize(np.array([np.nan], np.float32), 0.5, 0, O.INT8)


def test_code_ranges_are_reached():
    # Every code of each type is produced by some input, and nothing outside.
    for qt, (lo, hi) in [(O.INT8, (-128, 127)), (O.UINT8, (0, 255)), (O.INT4, (-8, 7)), (O.UINT4, (0, 15))]:
        x = np.linspace(-300, 300, 60001, dtype=np.float32)
        q = O.quantize(x, 1.0, 0, qt)
        assert q.min() == lo and q.max() == hi
        assert set(np.unique(q)) == set(range(lo, hi + 1))


def test_nibble_and_byte_packing_golden():
    for qtype, codes, packed in read_golden("nibble_packing.txt"):
        q = np.array([int(c) for c in codes.split(",")], np.int32)
        b = np.array([int(h, 16) for h in packed.split(",")], np.uint8)
        assert np.array_equal(O.pack(q, QT[qtype]), b), qtype
        assert np.array_equal(O.unpack(b, QT[qtype]), q), qtype


def test_pack_roundtrip_all_codes():
    rng = np.random.default_rng(5)
    for qt in (O.INT8, O.UINT8, O.INT4, O.UINT4):
        lo, hi = O.qrange(qt)
        q = rng.integers(lo, hi + 1, size=(7, 64), dtype=np.int32)
        assert np.array_equal(O.unpack(O.pack(q, qt), qt), q)
        with pytest.raises(O.OracleError):
            O.pack(np.array([hi + 1, lo], np.int32), qt)


def _not_near_tie(x, s, z=0):
    v = x.astype(np.float64) / np.float64(s)
    frac = np.abs(v - np.floor(v) - 0.5)
    return frac > 1e-3


def test_quantize_matches_torch_per_tensor():
    rng = np.random.default_rng(0)
    for dtype, qt, zp in [(torch.qint8, O.INT8, 0), (torch.quint8, O.UINT8, 37), (torch.qint8, O.INT8, -5)]:
        s = np.float32(rng.uniform(0.003, 0.2))
        x = (rng.standard_normal(20000) * 40 * s).astype(np.float32)
        x = x[_not_near_tie(x, s)]
        ref = torch.quantize_per_tensor(torch.from_numpy(x), float(s), zp, dtype).int_repr().numpy()
        assert np.array_equal(O.quantize(x, s, zp, qt), ref.astype(np.int32))


def test_quantize_matches_torch_per_channel():
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((16, 3, 3, 8)) * 0.05).astype(np.float32)
    s = (np.abs(w).reshape(16, -1).max(1) / 127).astype(np.float32)
    keep = np.ones(w.shape, bool)
    for c in range(16):
        keep[c] = _not_near_tie(w[c], s[c])
    ref = torch.quantize_per_channel(torch.from_numpy(w), torch.from_numpy(s.astype(np.float64)),
                                     torch.zeros(16, dtype=torch.int64), 0, torch.qint8).int_repr().numpy()
    got = O.quantize(w, s, np.zeros(16, np.int32), O.INT8, axis=0)
    assert np.array_equal(got[keep], ref[keep].astype(np.int32))
    assert np.abs(got).reshape(16, -1).max(1).tolist() == [127] * 16  # amax maps to the end code
    # last-axis (activation) per-channel too
    x = (np.abs(rng.standard_normal((5, 7, 6))) * 3).astype(np.float32)
    sx = np.linspace(0.01, 0.05, 6).astype(np.float32)
    zx = np.arange(6, dtype=np.int32)
    ref = torch.quantize_per_channel(torch.from_numpy(x), torch.from_numpy(sx.astype(np.float64)),
                                     torch.from_numpy(zx.astype(np.int64)), 2, torch.quint8).int_repr().numpy()
    keep = np.stack([_not_near_tie(x[..., c], sx[c]) for c in range(6)], -1)
    assert np.array_equal(O.quantize(x, sx, zx, O.UINT8)[keep], ref[keep].astype(np.int32))


def test_dequantize_matches_torch():
    rng = np.random.default_rng(2)
    q = rng.integers(0, 256, size=5000).astype(np.uint8)
    s, z = 0.0173, 91
    tq = torch._make_per_tensor_quantized_tensor(torch.from_numpy(q), s, z)
    ref = tq.dequantize().numpy()
    assert np.array_equal(O.dequantize(q.astype(np.int32), np.float32(s), z), ref)


def test_quantize_dequantize_roundtrip_every_code():
    rng = np.random.default_rng(3)
    for qt in (O.INT8, O.UINT8, O.INT4, O.UINT4):
        lo, hi = O.qrange(qt)
        codes = np.arange(lo, hi + 1, dtype=np.int32)
        for _ in range(300):
            s = np.float32(10 ** rng.uniform(-6, 3))
            z = int(rng.integers(lo, hi + 1)) if qt in (O.UINT8, O.UINT4) else 0
            x = O.dequantize(codes, s, z)
            assert np.array_equal(O.quantize(x, s, z, qt), codes), (qt, s, z)


def test_quantize_is_monotone():
    rng = np.random.default_rng(4)
    x = np.sort(rng.standard_normal(100000).astype(np.float32) * 3)
    q = O.quantize(x, np.float32(0.021), 100, O.UINT8)
    assert np.all(np.diff(q) >= 0)


def test_requant_multiplier_and_bias_closed_forms():
    # Power-of-two scales make every step exact: M = S_in*S_w/S_out.
    assert O.requant_multiplier(0.5, 0.25, 2.0)[0] == np.float32(0.0625)
    assert O.requant_multiplier(0.5, 0.25, 0.0625)[0] == np.float32(2.0)
    assert O.requant_multiplier(1.0, 0.125, 0.5)[0] == np.float32(0.25)
    assert O.residual_multiplier(0.25, 2.0) == np.float32(0.125)
    # bias / (S_in*S_w) at exact ties rounds half to even
    s_in, s_w = np.float32(0.5), np.float32(0.25)
    b = np.array([2.5, 3.5, -2.5, 1.0, 0.4], np.float32) * np.float32(0.125)
    assert O.quantize_bias(b, s_in, s_w).tolist() == [2, 4, -2, 1, 0]
    with pytest.raises(O.OracleError):
        O.quantize_bias(np.array([1e10], np.float32), 1e-3, 1e-3)
    # non-power-of-two: within half an ulp-level of the real quotient
    rng = np.random.default_rng(9)
    for _ in range(200):
        a, bb, c = (np.float32(10 ** rng.uniform(-3, 0)) for _ in range(3))
        m = O.requant_multiplier(a, bb, c)[0]
        assert abs(float(m) - float(a) * float(bb) / float(c)) <= 2 * np.spacing(m)


def test_requant_ties_golden():
    for acc, m, z, expected in read_golden("requant_ties.txt"):
        qt = O.UINT8 if int(z) != 0 else O.INT8
        out = O.requant(np.array([[int(acc)]], np.int64), np.float32(m), O.EPI_NONE, int(z), qt)
        assert out[0, 0] == int(expected), acc


def test_passive_relu_is_clamp_at_zero_point():
    # "Quantization" blog, section 量化激活函数: relu keeps the scale, so the
    # quantized ReLU is max(code, Z_out) of the un-activated result.
    rng = np.random.default_rng(6)
    acc = rng.integers(-20000, 20000, size=(300, 16)).astype(np.int64)
    m = (rng.uniform(0.001, 0.02, 16)).astype(np.float32)
    for z in (0, 7, 200):
        none = O.requant(acc, m, O.EPI_NONE, z, O.UINT8)
        relu = O.requant(acc, m, O.EPI_RELU, z, O.UINT8)
        assert np.array_equal(relu, np.maximum(none, z))


def test_add_with_equal_scales_is_integer_add():
    # "Quantization" blog, section 量化加法: with equal scales the add needs no rescale.
    # A zero accumulator plus a residual with S_res == S_out gives r - Z_res + Z_out.
    rng = np.random.default_rng(7)
    r = rng.integers(0, 256, size=(100, 8)).astype(np.int32)
    acc = np.zeros((100, 8), np.int64)
    out = O.requant(acc, np.float32(0.37), O.EPI_ADD, 5, O.UINT8, res=r, z_res=12, m_res=1.0)
    assert np.array_equal(out, np.clip(r - 12 + 5, 0, 255))
    out = O.requant(acc, np.float32(0.37), O.EPI_ADD_RELU, 5, O.UINT8, res=r, z_res=12, m_res=1.0)
    assert np.array_equal(out, np.clip(r - 12 + 5, 5, 255))


def test_requant_raw_passthrough_and_overflow():
    acc = np.array([[-(2 ** 31), 2 ** 31 - 1, 0]], np.int64)
    assert O.requant(acc, 1.0, O.EPI_RAW, 0, O.INT32).tolist() == [[-(2 ** 31), 2 ** 31 - 1, 0]]
    with pytest.raises(O.OracleError):
        O.requant(np.array([[2 ** 31]], np.int64), 1.0, O.EPI_NONE, 0, O.INT8)


def test_requant_is_unfused():
    # Inputs where a fused multiply-add (a*M + u rounded once) differs from the two
    # rounded products plus a rounded sum.  The oracle must give the unfused result.
    acc, r = np.meshgrid(np.arange(-15000, 15000, dtype=np.int64), np.arange(256, dtype=np.int32))
    acc, r = acc.ravel(), r.ravel()
    m = np.float32(0.00731)
    m_res = np.float32(0.0413)
    a = acc.astype(np.float32)
    t_unfused = (a * m) + ((r - 9).astype(np.float32) * m_res)
    t_fused = (a.astype(np.float64) * np.float64(m) + (r - 9).astype(np.float64) * np.float64(m_res)).astype(np.float32)
    diff = (np.rint(t_unfused) != np.rint(t_fused)) & (np.abs(t_unfused) < 120)
    assert diff.sum() >= 5, "too few canaries"
    idx = np.nonzero(diff)[0]
    out = O.requant(acc[idx, None], m, O.EPI_ADD, 0, O.INT8, res=r[idx, None], z_res=9, m_res=m_res)[:, 0]
    assert np.array_equal(out, np.rint(t_unfused[idx]).astype(np.int32))


def test_quantize_divides_rather_than_multiplying_by_reciprocal():
    # READING of the "Quantization" blog's value / scale: one correctly rounded
    # binary32 division.  numpy's float32 divide is IEEE-exact; on inputs where
    # x * (1/S) rounds to a different code than x / S, the oracle follows the division.
    rng = np.random.default_rng(10)
    s = np.float32(0.0371)
    x = (rng.integers(-127, 128, 400000) + rng.choice([-0.5, 0.5], 400000)).astype(np.float32) * s
    by_div = np.rint(x / s)
    by_rcp = np.rint(x * (np.float32(1) / s))
    idx = np.nonzero(by_div != by_rcp)[0]
    assert idx.size >= 5, "too few canaries"
    assert np.array_equal(O.quantize(x[idx], s, 0, O.INT8), np.clip(by_div[idx], -128, 127).astype(np.int32))
