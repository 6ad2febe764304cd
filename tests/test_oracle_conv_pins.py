"""Pins for the oracle's direct convolution, GEMM, im2col and max pooling.

The accumulators are integers, so library routines pin them exactly:
torch.nn.functional.conv2d in float64 on (x - Z) (every partial sum is an
integer far below 2^53), numpy int64 matmul, torch max_pool2d.  Closed forms
(identity / centre-tap / corner-tap kernels, all-ones window sums) and the
identities the pages state (im2col == direct conv, Linear == 1x1 conv, a
column permutation of B permutes the columns of C, zero-point folding) pin the
index arithmetic and the padding reading.  A real-valued float64 evaluation of
the whole quantized operator bounds the oracle's requantized output to one code.
CPU only.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O


def _rand_codes(rng, shape, lo, hi):
    return rng.integers(lo, hi + 1, size=shape, dtype=np.int64).astype(np.int32)


def _torch_conv_acc(x, z_in, w, stride, pad, bias_q=None):
    xt = torch.from_numpy((x.astype(np.float64) - z_in)).permute(0, 3, 1, 2)
    wt = torch.from_numpy(w.astype(np.float64)).permute(0, 3, 1, 2)
    y = F.conv2d(xt, wt, stride=stride, padding=pad).permute(0, 2, 3, 1).numpy()
    y = np.rint(y).astype(np.int64)
    if bias_q is not None:
        y = y + bias_q.astype(np.int64)
    return y


CONV_CASES = [
    # n, h, w, ci, co, kh, kw, stride, pad
    (1, 5, 5, 1, 1, 3, 3, (1, 1), (1, 1)),
    (2, 5, 4, 3, 4, 3, 3, (1, 1), (0, 0)),
    (2, 7, 6, 4, 5, 3, 3, (2, 2), (1, 1)),
    (1, 9, 9, 3, 2, 7, 7, (2, 2), (3, 3)),
    (2, 6, 5, 5, 3, 1, 1, (2, 2), (0, 0)),
    (1, 6, 7, 2, 3, 3, 1, (2, 1), (1, 0)),
    (1, 4, 4, 2, 2, 3, 3, (1, 1), (2, 2)),
    (1, 8, 8, 16, 8, 3, 3, (1, 1), (1, 1)),
]


@pytest.mark.parametrize("case", CONV_CASES)
def test_conv_acc_matches_torch_conv2d_exactly(case):
    n, h, w, ci, co, kh, kw, stride, pad = case
    rng = np.random.default_rng(hash(case) % 2 ** 32)
    for (lo, hi, z) in [(0, 255, 37), (-128, 127, 0), (0, 15, 3), (-128, 127, -11)]:
        x = _rand_codes(rng, (n, h, w, ci), lo, hi)
        wt = _rand_codes(rng, (co, kh, kw, ci), -128, 127)
        bq = _rand_codes(rng, (co,), -5000, 5000)
        got = O.conv2d_acc(x, z, wt, 0, stride, pad, bq)
        assert np.array_equal(got, _torch_conv_acc(x, z, wt, stride, pad, bq))


def test_conv_acc_with_weight_zero_point_matches_torch():
    rng = np.random.default_rng(11)
    x = _rand_codes(rng, (2, 5, 5, 3), 0, 255)
    wt = _rand_codes(rng, (4, 3, 3, 3), 0, 15)
    got = O.conv2d_acc(x, 40, wt, 8, 1, 1)
    assert np.array_equal(got, _torch_conv_acc(x, 40, wt - 8, 1, 1))


@pytest.mark.parametrize("case", CONV_CASES[1:5])
def test_asymmetric_weights_match_torch_conv2d(case):
    # MegEngine 4-bit article, section 緩解精度下降: weights in UINT4 (or UINT8) carry a
    # zero point Z_W; the accumulator is sum (Q(I) - Z_I)(Q(W) - Z_W).  torch conv2d in
    # float64 on the centred operands is exact for these integer sums.
    n, h, w, ci, co, kh, kw, stride, pad = case
    rng = np.random.default_rng((hash(case) + 91) % 2 ** 32)
    for (wlo, whi, zw) in [(0, 255, 131), (0, 255, 0), (0, 15, 7), (-128, 127, -9), (-8, 7, 3)]:
        x = _rand_codes(rng, (n, h, w, ci), 0, 255)
        wt = _rand_codes(rng, (co, kh, kw, ci), wlo, whi)
        bq = _rand_codes(rng, (co,), -5000, 5000)
        got = O.conv2d_acc(x, 21, wt, zw, stride, pad, bq)
        assert np.array_equal(got, _torch_conv_acc(x, 21, wt - zw, stride, pad, bq))


def test_weight_zero_point_term_is_a_per_pixel_window_sum():
    # MegEngine 4-bit article, section 緩解精度下降: a nonzero Z_W adds the red term
    # -Z_W * sum Q(I), which depends on the input and so varies per output pixel:
    # acc(Z_W) == acc(0) - Z_W * (window sums of Q(I) - Z_I), the window sums taken by an
    # all-ones kernel (torch conv2d, float64, exact).
    rng = np.random.default_rng(12)
    x = _rand_codes(rng, (2, 7, 6, 5), 0, 255)
    wt = _rand_codes(rng, (3, 3, 3, 5), 0, 255)
    for zw, z_in, stride, pad in [(117, 30, 1, 1), (200, 0, 2, 1), (1, 255, 1, 2)]:
        a0 = O.conv2d_acc(x, z_in, wt, 0, stride, pad)
        az = O.conv2d_acc(x, z_in, wt, zw, stride, pad)
        ones = np.ones((1, 3, 3, 5), np.int32)
        win = _torch_conv_acc(x, z_in, ones, stride, pad)[..., 0]
        assert np.array_equal(az, a0 - zw * win[..., None])


def test_weights_equal_to_their_zero_point_give_the_bias():
    rng = np.random.default_rng(13)
    x = _rand_codes(rng, (1, 6, 6, 4), 0, 255)
    bq = _rand_codes(rng, (3,), -1000, 1000)
    for zw in (0, 9, 200):
        wt = np.full((3, 3, 3, 4), zw, np.int32)
        acc = O.conv2d_acc(x, 77, wt, zw, 2, 1, bq)
        assert np.array_equal(acc, np.broadcast_to(bq.astype(np.int64), acc.shape))


def test_gemm_with_weight_zero_point_matches_numpy():
    rng = np.random.default_rng(14)
    a = _rand_codes(rng, (29, 128), 0, 255)
    b = _rand_codes(rng, (13, 128), 0, 255)
    bq = _rand_codes(rng, (13,), -1000, 1000)
    want = (a.astype(np.int64) - 111) @ (b.astype(np.int64) - 140).T + bq
    assert np.array_equal(O.gemm_acc(a, 111, b, 140, bq), want)


def test_identity_1x1_gives_centred_input():
    rng = np.random.default_rng(12)
    x = _rand_codes(rng, (2, 5, 6, 4), 0, 255)
    wt = np.eye(4, dtype=np.int32).reshape(4, 1, 1, 4)
    acc = O.conv2d_acc(x, 20, wt)
    assert np.array_equal(acc, x.astype(np.int64) - 20)


def test_centre_tap_and_corner_tap_pin_padding():
    rng = np.random.default_rng(13)
    x = _rand_codes(rng, (1, 6, 5, 2), 0, 255)
    z = 77
    centre = np.zeros((2, 3, 3, 2), np.int32)
    centre[0, 1, 1, 0] = 1
    centre[1, 1, 1, 1] = 1
    assert np.array_equal(O.conv2d_acc(x, z, centre, 0, 1, 1), x.astype(np.int64) - z)
    # top-left tap: output (oy, ox) reads input (oy-1, ox-1); the first row and column
    # read the padding, which holds the real value 0 (code Z_in).
    corner = np.zeros((2, 3, 3, 2), np.int32)
    corner[0, 0, 0, 0] = 1
    corner[1, 0, 0, 1] = 1
    acc = O.conv2d_acc(x, z, corner, 0, 1, 1)
    want = np.zeros_like(acc)
    want[:, 1:, 1:, :] = x[:, :-1, :-1, :].astype(np.int64) - z
    assert np.array_equal(acc, want)


def test_all_ones_kernel_gives_window_sums():
    # Horizon J5 lecture: ReduceSum is a conv with an all-ones kernel.  Window sums are
    # computed here independently with a 2-D prefix sum over the zero-padded (x - Z).
    rng = np.random.default_rng(14)
    x = _rand_codes(rng, (2, 7, 6, 3), 0, 255)
    z, k, p, s = 100, 3, 1, 2
    wt = np.ones((1, k, k, 3), np.int32)
    acc = O.conv2d_acc(x, z, wt, 0, s, p)[..., 0]
    d = (x.astype(np.int64) - z).sum(-1)
    d = np.pad(d, ((0, 0), (p + 1, p), (p + 1, p)))
    ps = d.cumsum(1).cumsum(2)
    oh, ow = acc.shape[1:]
    want = np.empty_like(acc)
    for oy, ox in itertools.product(range(oh), range(ow)):
        y0, x0 = oy * s, ox * s
        y1, x1 = y0 + k, x0 + k
        want[:, oy, ox] = ps[:, y1, x1] - ps[:, y0, x1] - ps[:, y1, x0] + ps[:, y0, x0]
    assert np.array_equal(acc, want)


@pytest.mark.parametrize("case", CONV_CASES[:6])
def test_im2col_gemm_equals_direct_conv(case):
    # MegEngine 4-bit article, section conv 算子優化, Fig. 5: conv == im2col matrix product.
    n, h, w, ci, co, kh, kw, stride, pad = case
    rng = np.random.default_rng(15)
    x = _rand_codes(rng, (n, h, w, ci), 0, 255)
    wt = _rand_codes(rng, (co, kh, kw, ci), -128, 127)
    cols = O.im2col(x, 9, kh, kw, stride, pad)
    acc_mm = (cols.astype(np.int64) - 9) @ wt.reshape(co, -1).T.astype(np.int64)
    acc = O.conv2d_acc(x, 9, wt, 0, stride, pad)
    assert np.array_equal(acc.reshape(-1, co), acc_mm)
    # and through the oracle's own GEMM
    assert np.array_equal(O.gemm_acc(cols, 9, wt.reshape(co, -1), 0), acc_mm)


def test_zero_point_folding_identity():
    # MegEngine 4-bit article, section 緩解精度下降: with Z_W = 0 the Z_I term is
    # Z_I * sum Q(W), known before inference.  sum (q - Z) w == sum q w - Z sum w, where
    # pads hold the code Z so the fold uses the full weight sum at borders too.
    rng = np.random.default_rng(16)
    x = _rand_codes(rng, (2, 6, 6, 8), 0, 255)
    wt = _rand_codes(rng, (5, 3, 3, 8), -127, 127)
    z = 123
    acc = O.conv2d_acc(x, z, wt, 0, 1, 1)
    xp = np.pad(x.astype(np.int64), ((0, 0), (1, 1), (1, 1), (0, 0)), constant_values=z)
    win = np.lib.stride_tricks.sliding_window_view(xp, (3, 3), axis=(1, 2))  # n,oh,ow,c,kh,kw
    raw = np.einsum("nhwcij,oijc->nhwo", win, wt.astype(np.int64))
    folded = raw - z * wt.astype(np.int64).reshape(5, -1).sum(1)
    assert np.array_equal(acc, folded)


def test_output_channel_permutation():
    # MegEngine 4-bit article, section conv 算子優化, Fig. 8: swapping columns of B swaps
    # the same columns of C.  Permuting weight rows permutes output channels.
    rng = np.random.default_rng(17)
    x = _rand_codes(rng, (1, 5, 5, 4), 0, 255)
    wt = _rand_codes(rng, (8, 3, 3, 4), -128, 127)
    perm = rng.permutation(8)
    a = O.conv2d_acc(x, 3, wt, 0, 1, 1)
    b = O.conv2d_acc(x, 3, wt[perm], 0, 1, 1)
    assert np.array_equal(a[..., perm], b)


def test_gemm_matches_numpy_matmul():
    rng = np.random.default_rng(18)
    for (m, k, n, za, lo, hi) in [(37, 65, 19, 128, 0, 255), (16, 256, 32, 0, -128, 127), (5, 30, 7, 4, 0, 15)]:
        a = _rand_codes(rng, (m, k), lo, hi)
        b = _rand_codes(rng, (n, k), -128, 127)
        bq = _rand_codes(rng, (n,), -1000, 1000)
        want = (a.astype(np.int64) - za) @ b.astype(np.int64).T + bq
        assert np.array_equal(O.gemm_acc(a, za, b, 0, bq), want)


def test_linear_equals_1x1_conv():
    # Horizon J5 lecture: nn.Linear is a 1x1 conv after reshaping the weights.
    rng = np.random.default_rng(19)
    x = _rand_codes(rng, (2, 3, 4, 16), 0, 255)
    wt = _rand_codes(rng, (8, 16), -128, 127)
    conv = O.conv2d_acc(x, 50, wt.reshape(8, 1, 1, 16))
    gemm = O.gemm_acc(x.reshape(-1, 16), 50, wt)
    assert np.array_equal(conv.reshape(-1, 8), gemm)


def test_accumulator_overflow_is_reported():
    x = np.full((1, 1, 1, 70000), 255, np.int32)
    wt = np.full((1, 1, 1, 70000), 127, np.int32)
    with pytest.raises(O.OracleError):
        O.conv2d_acc(x, 0, wt)


def _torch_maxpool(x, k, s, p):
    # torch pads with -inf: a tap outside the image can never be the maximum
    ref = F.max_pool2d(torch.from_numpy(x.astype(np.float64)).permute(0, 3, 1, 2), k, s, p)
    return np.rint(ref.permute(0, 2, 3, 1).numpy()).astype(np.int32)


@pytest.mark.parametrize("lo,hi", [(0, 255), (-128, 127), (-8, 7), (-128, -1)],
                         ids=["uint8", "int8", "int4", "negative_only"])
def test_maxpool_matches_torch(lo, hi):
    """Max pooling of codes ("Quantization" blog, 量化激活函数: passive, the max of the
    codes) against torch max_pool2d.  Signed codes matter: with unsigned codes a tap
    outside the image read as code 0 could never change the max, with negative codes it
    would."""
    rng = np.random.default_rng(20 + abs(lo) + hi)
    for (n, h, w, c, k, s, p) in [(2, 9, 8, 5, 3, 2, 1), (1, 7, 7, 3, 3, 1, 1), (1, 6, 5, 2, 2, 2, 0),
                                   (1, 4, 4, 3, 3, 2, 1), (2, 1, 1, 4, 3, 2, 1)]:
        x = _rand_codes(rng, (n, h, w, c), lo, hi)
        assert np.array_equal(O.maxpool2d(x, k, s, p), _torch_maxpool(x, k, s, p))


def test_maxpool_border_windows_of_negative_codes():
    """All-negative windows at the borders: every output of a 3x3 / stride 2 / pad 1
    pooling of a constant -100 image is -100 (a border window holds only 4 or 6 image
    taps), and a single -1 surrounded by -128 is found from every window that holds it."""
    x = np.full((1, 5, 6, 2), -100, np.int32)
    assert np.all(O.maxpool2d(x, 3, 2, 1) == -100)
    x = np.full((1, 5, 5, 1), -128, np.int32)
    x[0, 0, 0, 0] = -1
    y = O.maxpool2d(x, 3, 2, 1)
    assert y[0, 0, 0, 0] == -1 and np.all(y.reshape(-1)[1:] == -128)
    assert np.array_equal(y, _torch_maxpool(x, 3, 2, 1))


def _exact_real_output(x, z_in, s_in, wt, s_w, bias, res, z_res, s_res, stride, pad):
    """Real value of the quantized operator in float64: dequantized operands, fp32 bias."""
    xt = torch.from_numpy((x.astype(np.float64) - z_in) * np.float64(s_in)).permute(0, 3, 1, 2)
    wt_r = wt.astype(np.float64) * s_w.astype(np.float64)[:, None, None, None]
    y = F.conv2d(xt, torch.from_numpy(wt_r).permute(0, 3, 1, 2), stride=stride, padding=pad)
    y = y.permute(0, 2, 3, 1).numpy() + bias.astype(np.float64)
    if res is not None:
        y = y + (res.astype(np.float64) - z_res) * np.float64(s_res)
    return y


@pytest.mark.parametrize("epi", [O.EPI_NONE, O.EPI_RELU, O.EPI_ADD_RELU])
def test_requantized_conv_within_one_code_of_real_value(epi):
    # The only differences from rounding the exact real output are the bias rounding and
    # binary32 rounding near ties; both stay below one output code.
    rng = np.random.default_rng(21 + epi)
    x = _rand_codes(rng, (2, 6, 6, 16), 0, 255)
    wt = _rand_codes(rng, (8, 3, 3, 16), -127, 127)
    s_in, z_in = np.float32(0.013), 17
    s_w = rng.uniform(0.001, 0.004, 8).astype(np.float32)
    bias = rng.normal(0, 0.5, 8).astype(np.float32)
    res, z_res, s_res = (None, 0, 1.0)
    if epi == O.EPI_ADD_RELU:
        res, z_res, s_res = _rand_codes(rng, (2, 6, 6, 8), 0, 255), 9, np.float32(0.021)
    s_out, z_out = np.float32(0.05), 40
    q = O.qconv(x, z_in, s_in, wt, s_w, bias, s_out, z_out, O.UINT8, epi, 1, 1, res, s_res, z_res)
    y = _exact_real_output(x, z_in, s_in, wt, s_w, bias, res, z_res, s_res, 1, 1)
    if epi != O.EPI_NONE:
        y = np.maximum(y, 0)
    want = np.clip(np.rint(y / np.float64(s_out)) + z_out, 0, 255)
    assert np.abs(q - want).max() <= 1
    assert (q != want).mean() < 0.01


def test_tiny_brute_force_in_exact_rationals():
    # A third evaluation with Python Fractions: real-valued conv of dequantized codes,
    # one code of slack for the binary32 steps, on every output of a tiny case.
    rng = np.random.default_rng(22)
    x = _rand_codes(rng, (1, 3, 3, 2), 0, 15)
    wt = _rand_codes(rng, (2, 3, 3, 2), -8, 7)
    s_in, z_in, s_w, s_out, z_out = np.float32(0.25), 3, np.float32(0.125), np.float32(0.5), 2
    q = O.qconv(x, z_in, s_in, wt, s_w, None, s_out, z_out, O.UINT4, O.EPI_RELU, 1, 1)
    for oy, ox, oc in itertools.product(range(3), range(3), range(2)):
        tot = Fraction(0)
        for ky, kx, ci in itertools.product(range(3), range(3), range(2)):
            iy, ix = oy - 1 + ky, ox - 1 + kx
            xv = int(x[0, iy, ix, ci]) if 0 <= iy < 3 and 0 <= ix < 3 else z_in
            tot += Fraction(xv - z_in) * Fraction(float(s_in)) * Fraction(int(wt[oc, ky, kx, ci])) * Fraction(float(s_w))
        t = max(tot / Fraction(float(s_out)), Fraction(0))
        fl = t.numerator // t.denominator
        rem = t - fl
        r = fl + (1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2) else 0)
        want = min(max(r + z_out, 0), 15)
        # every step is exact here (power-of-two scales, small sums), so no slack is needed
        assert q[0, oy, ox, oc] == want
