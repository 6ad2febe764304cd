"""GPU parity of the integer-only requantization (IQNN_EPI_INT_REQUANT): every output
byte equals the oracle's direct accumulator followed by get_mn / requant_int
("Quantization" blog, 量化模式: integer (power of two) quantization; FQ-ViT article,
LayerNorm code: get_MN).  The layers cover the streaming kernel (8-bit activations
with whole 64-channel stages, each of its integer-requantizing block configurations),
the direct 3x3 kernel, and the register-staged kernel's other gathers (the element
gather for C_in % 16 != 0, the 4-channel stem input, 4-bit activations), and a GEMM."""
import numpy as np
import pytest

import oracle as O
from integer_quantized_nn_amd import synth
from parity_util import assert_bytes_equal, conv_codes, otype, require_gpu, to_bytes

pytestmark = pytest.mark.gpu

U8, I8, U4, I4 = synth.UINT8, synth.INT8, synth.UINT4, synth.INT4
NONE, RELU = synth.EPI_NONE, synth.EPI_RELU
INT_RQ = 16


def oracle_int(case, x, w):
    co = w.shape[0]
    s_w = np.broadcast_to(np.atleast_1d(np.asarray(case.s_w, np.float32)), (co,))
    bias_q = O.quantize_bias(case.bias, case.s_in, s_w)
    acc = O.conv2d_acc(x, case.z_in, w, 0, case.stride, case.pad, bias_q)
    mn = [O.get_mn(m) for m in O.requant_multiplier(case.s_in, s_w, case.s_out)]
    m = np.array([a for a, _ in mn])
    n = np.array([b for _, b in mn])
    return O.requant_int(acc, m, n, case.epi, case.z_out, otype(case.y_type))


CASES = [
    # n, h, w, c_in, c_out, k, stride, pad, x_type, w_type, y_type, epi
    (2, 9, 11, 64, 64, 3, 1, 1, U8, I8, U8, RELU),
    (1, 13, 7, 128, 96, 1, 1, 0, U8, I8, I8, NONE),
    (2, 8, 8, 48, 80, 3, 2, 1, I8, I8, U8, RELU),
    (1, 10, 10, 24, 40, 3, 1, 1, U8, I8, U8, NONE),     # element gather, ragged channels
    (2, 15, 15, 4, 64, 7, 2, 3, U8, I8, U8, RELU),      # stem-like 4-channel input
    (2, 8, 8, 32, 64, 3, 1, 1, U4, I4, U4, RELU),       # 4-bit activations and output
    (1, 7, 9, 64, 128, 3, 1, 1, U4, I4, I8, NONE),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "n%dh%dw%dci%dco%dk%ds%dp%d_x%dw%dy%de%d" % c)
def test_conv_integer_requant(case):
    torch = require_gpu()
    from integer_quantized_nn_amd.layers import QConv
    n, h, w, ci, co, k, s, p, xt, wt, yt, epi = case
    c = synth.conv_case((hash(case) + 77) % 2 ** 31, n, h, w, ci, co, k, s, p, xt, wt, yt, epi)
    x, wq, _ = conv_codes(c)
    want = to_bytes(oracle_int(c, x, wq), yt)
    conv = QConv(n, h, w, ci, co, k, s, p, xt, wt, yt, epi | INT_RQ, c.z_in, c.z_out, to_bytes(wq, wt), c.bias,
                 c.s_in, c.s_w, c.s_out)
    y = conv(torch.from_numpy(to_bytes(x, xt)).cuda())
    torch.cuda.synchronize()
    assert_bytes_equal(y.cpu().numpy(), want, str(case))
    # discrimination: the 8-bit cases span many codes
    if yt in (U8, I8):
        assert len(np.unique(y.cpu().numpy())) >= 32


def test_gemm_integer_requant():
    torch = require_gpu()
    from integer_quantized_nn_amd.layers import QGemm
    rng = np.random.default_rng(8)
    m, n, k = 211, 72, 160
    a = rng.integers(0, 256, size=(m, k)).astype(np.int32)
    b = rng.integers(-128, 128, size=(n, k)).astype(np.int32)
    s_a, s_out = np.float32(0.02), np.float32(0.6)
    s_b = rng.uniform(0.002, 0.004, n).astype(np.float32)
    bias = rng.normal(0, 0.5, n).astype(np.float32)
    acc = O.gemm_acc(a, 119, b, 0, O.quantize_bias(bias, s_a, s_b))
    mn = [O.get_mn(v) for v in O.requant_multiplier(s_a, s_b, s_out)]
    want = O.requant_int(acc, np.array([v[0] for v in mn]), np.array([v[1] for v in mn]), O.EPI_NONE, 0, O.INT8)
    g = QGemm(m, n, k, U8, I8, I8, NONE | INT_RQ, 119, 0, to_bytes(b, I8), bias, s_a, s_b, s_out)
    c = g(torch.from_numpy(to_bytes(a, U8)).cuda())
    torch.cuda.synchronize()
    assert_bytes_equal(c.cpu().numpy(), to_bytes(want, I8), "gemm integer requant")
    assert len(np.unique(c.cpu().numpy())) >= 32


@pytest.mark.parametrize("h,co,xt,yt,epi", [(6, 64, U8, U8, RELU), (5, 128, I8, I8, NONE), (2, 64, U8, I8, RELU)])
def test_direct3x3_integer_requant(h, co, xt, yt, epi):
    """The direct 3x3 kernel with the integer-only epilogue (forced through tile 18):
    64-channel 3x3 convs on 56-pixel rows, odd and two-row heights, one and two
    64-channel output blocks, uint8 and int8 codes."""
    torch = require_gpu()
    from integer_quantized_nn_amd import binding as B
    from integer_quantized_nn_amd.layers import QConv
    c = synth.conv_case(h * 1000 + co + xt, 2, h, 56, 64, co, 3, 1, 1, xt, I8, yt, epi)
    x, wq, _ = conv_codes(c)
    want = to_bytes(oracle_int(c, x, wq), yt)
    conv = QConv(2, h, 56, 64, co, 3, 1, 1, xt, I8, yt, epi | INT_RQ, c.z_in, c.z_out, to_bytes(wq, I8), c.bias,
                 c.s_in, c.s_w, c.s_out)
    y = conv(torch.from_numpy(to_bytes(x, xt)).cuda(), cfg=(18, 0))
    torch.cuda.synchronize()
    assert_bytes_equal(y.cpu().numpy(), want, "direct 3x3 integer requant h=%d co=%d" % (h, co))


def test_integer_requant_3x3_workload_full_size():
    """The 3x3 workload (N=32, 56x56, 64 -> 64, Conv_Relu to uint8) with the integer-only
    epilogue, on the kernel the library picks for it (the direct 3x3 kernel): every
    output byte against the oracle."""
    torch = require_gpu()
    from integer_quantized_nn_amd.layers import QConv
    c = synth.conv3x3_int8()
    x, wq, _ = conv_codes(c)
    n, h, w, ci = x.shape
    conv = QConv(n, h, w, ci, c.c_out, 3, 1, 1, c.x_type, I8, c.y_type, c.epi | INT_RQ, c.z_in, c.z_out,
                 to_bytes(wq, I8), c.bias, c.s_in, c.s_w, c.s_out)
    y = conv(torch.from_numpy(to_bytes(x, c.x_type)).cuda())
    torch.cuda.synchronize()
    want = to_bytes(oracle_int(c, x, wq), c.y_type)
    assert_bytes_equal(y.cpu().numpy(), want, "3x3 workload, integer requant")
    assert len(np.unique(y.cpu().numpy())) >= 64


# the streaming kernel's integer-requantizing block configurations (tiles 8, 10, 11, 14,
# 16 and 22), 1x1 and 3x3, on 2 x 9 x 13 pixels: several pixel tiles and a ragged tail
STREAM_TILES = [(8, 1, 64, 64), (8, 3, 64, 64), (10, 1, 128, 128), (10, 3, 64, 192), (11, 1, 64, 64),
                (11, 3, 128, 64), (14, 1, 256, 128), (14, 3, 128, 128), (16, 1, 256, 256), (16, 3, 64, 256),
                (22, 1, 256, 512), (22, 3, 64, 512)]


@pytest.mark.parametrize("tile,k,ci,co", STREAM_TILES, ids=lambda v: str(v))
def test_streaming_integer_requant_tiles(tile, k, ci, co):
    """Every byte of the streaming kernel's integer-only epilogue against the oracle's
    requant_int, for each block configuration compiled with it."""
    torch = require_gpu()
    from integer_quantized_nn_amd.layers import QConv
    n, h, w = 2, 9, 13
    c = synth.conv_case(tile * 100 + k * 10 + co, n, h, w, ci, co, k, 1, k // 2, U8, I8, U8, RELU)
    x, wq, _ = conv_codes(c)
    want = to_bytes(oracle_int(c, x, wq), U8)
    conv = QConv(n, h, w, ci, co, k, 1, k // 2, U8, I8, U8, RELU | INT_RQ, c.z_in, c.z_out, to_bytes(wq, I8),
                 c.bias, c.s_in, c.s_w, c.s_out)
    y = conv(torch.from_numpy(to_bytes(x, U8)).cuda(), cfg=(tile, 0))
    torch.cuda.synchronize()
    assert_bytes_equal(y.cpu().numpy(), want, "integer requant tile %d k=%d co=%d" % (tile, k, co))
    assert len(np.unique(y.cpu().numpy())) >= 32


@pytest.mark.parametrize("mult,y_type,epi", [(0.5, I8, NONE), (0.5, U8, RELU), (3.0, I8, NONE), (2.0 ** -30, U8, RELU)])
@pytest.mark.parametrize("k", [1, 3])
def test_integer_requant_exact_rounding(mult, y_type, epi, k):
    """Scales chosen to fix the multiplier: 0.5 (power-of-two scales; get_MN gives
    M = 128, N = 8, and every odd accumulator is a tie, rounded half to even), about 3
    (N = 6 < 8: large products, most codes clipped) and 2^-30 (N clamped to 31,
    M = 2).  Every byte against the oracle's requant_int, on the streaming kernel."""
    torch = require_gpu()
    from integer_quantized_nn_amd.layers import QConv
    n, h, w, ci, co = 2, 7, 11, 64, 128
    c = synth.conv_case(int(mult * 1000) + k, n, h, w, ci, co, k, 1, k // 2, U8, I8, y_type, epi)
    c.s_in = np.float32(2.0 ** -4)
    c.s_w = np.full(co, 2.0 ** -9, np.float32)
    c.s_out = np.float32(2.0 ** -13 / mult)
    x, wq, _ = conv_codes(c)
    mm = O.requant_multiplier(c.s_in, c.s_w, c.s_out)
    if mult == 0.5:
        assert all(O.get_mn(v) == (128, 8) for v in mm)
    want = to_bytes(oracle_int(c, x, wq), y_type)
    conv = QConv(n, h, w, ci, co, k, 1, k // 2, U8, I8, y_type, epi | INT_RQ, c.z_in, c.z_out, to_bytes(wq, I8),
                 c.bias, c.s_in, c.s_w, c.s_out)
    y = conv(torch.from_numpy(to_bytes(x, U8)).cuda())
    torch.cuda.synchronize()
    assert_bytes_equal(y.cpu().numpy(), want, "integer requant mult=%g k=%d" % (mult, k))
