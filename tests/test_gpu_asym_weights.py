"""GPU parity of asymmetric weights (MegEngine 4-bit article, section 緩解精度下降: a
weight zero point Z_W != 0 adds the per-pixel term Z_W * sum Q(I)).  Weight codes
are the oracle's quantization of the synthetic float weights with per-tensor
min-max parameters (UINT8, UINT4), or symmetric INT8 codes moved by a constant
together with their zero point.  Every output byte must equal the oracle's
direct sum (q_I - Z_I)(q_W - Z_W) followed by the same requantization."""
import numpy as np
import pytest

import oracle as O
from integer_quantized_nn_amd import synth
from parity_util import (assert_bytes_equal, conv_codes, gpu_conv, gpu_gemm, oracle_conv, otype, require_gpu,
                         to_bytes)

pytestmark = pytest.mark.gpu

U8, I8, U4, I4, I32 = synth.UINT8, synth.INT8, synth.UINT4, synth.INT4, synth.INT32
NONE, RELU, ADD, ADD_RELU, RAW = synth.EPI_NONE, synth.EPI_RELU, synth.EPI_ADD, synth.EPI_ADD_RELU, synth.EPI_RAW


def asym_weights(case, w_type):
    """(codes, s_w, z_w) of case.w as w_type with a per-tensor zero point."""
    if w_type == I8:   # symmetric codes and their zero point moved by the same constant
        w = O.quantize(case.w, case.s_w, 0, O.INT8, axis=0)
        z_w = 5
        return np.clip(w + z_w, -128, 127), case.s_w, z_w
    s_w, z_w = synth.minmax_qparams(case.w.min(), case.w.max(), w_type)
    return O.quantize(case.w, s_w, z_w, otype(w_type)), s_w, z_w


CASES = [
    # n, h, w, c_in, c_out, k, stride, pad, x_type, w_type, y_type, epi, res_type
    (2, 9, 11, 64, 64, 3, 1, 1, U8, U8, U8, RELU, U8),        # 64-channel blocks
    (1, 13, 7, 128, 96, 3, 2, 1, U8, U8, U8, ADD_RELU, U8),   # 128-channel blocks, residual, ragged
    (2, 8, 9, 64, 256, 1, 1, 0, I8, U8, I8, NONE, U8),        # 1x1, signed activations
    (1, 7, 7, 192, 48, 1, 1, 0, U8, U4, U8, ADD, U8),         # UINT4 weights
    (3, 5, 5, 64, 40, 3, 1, 1, U8, I8, U8, RELU, U8),         # INT8 weights, Z_W != 0, C_out % 16 != 0
    (1, 6, 6, 64, 64, 3, 1, 1, U8, U8, I32, RAW, U8),         # raw accumulators
    (1, 4, 4, 128, 128, 3, 1, 2, U8, U8, U8, NONE, U8),       # padding dominates
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "n%dh%dw%dci%dco%dk%ds%dp%d_x%dw%dy%de%d" % c[:12])
def test_conv_asymmetric_weights(case):
    require_gpu()
    n, h, w, ci, co, k, s, p, xt, wt, yt, epi, rt = case
    c = synth.conv_case(hash(case) % 2 ** 31, n, h, w, ci, co, k, s, p, xt, I8, yt, epi, res_type=rt)
    x, _, res = conv_codes(c)
    wq, s_w, z_w = asym_weights(c, wt)
    want = to_bytes(oracle_conv(c, x, wq, res, z_w=z_w, s_w=s_w), yt)
    got = gpu_conv(c, x, wq, res, w_type=wt, z_w=z_w, s_w=s_w)
    assert_bytes_equal(got, want, str(case))


def test_conv3x3_asymmetric_weights_full_size():
    """The ResNet 3x3 workload (N=32 56x56 64->64, Conv_Relu) with UINT8 weights and a
    per-tensor weight zero point; every output byte against the oracle."""
    require_gpu()
    c = synth.conv3x3_int8(seed=0)
    x, _, _ = conv_codes(c)
    wq, s_w, z_w = asym_weights(c, U8)
    assert z_w not in (0, 128)
    got = gpu_conv(c, x, wq, None, w_type=U8, z_w=z_w, s_w=s_w)
    want = to_bytes(oracle_conv(c, x, wq, None, z_w=z_w, s_w=s_w), c.y_type)
    assert_bytes_equal(got, want, "conv3x3 uint8 weights")
    assert len(np.unique(got)) >= 64


def test_gemm_asymmetric_weights():
    require_gpu()
    import torch
    from integer_quantized_nn_amd.layers import QGemm
    rng = np.random.default_rng(5)
    m, n, k = 300, 96, 192
    a = rng.integers(0, 256, size=(m, k)).astype(np.int32)
    b = rng.integers(0, 256, size=(n, k)).astype(np.int32)
    z_a, z_b, z_out = 121, 77, 3
    s_a, s_out = np.float32(0.02), np.float32(0.25)
    s_b = rng.uniform(0.002, 0.004, n).astype(np.float32)
    bias = rng.normal(0, 0.5, n).astype(np.float32)
    want = O.qgemm(a, z_a, s_a, b, s_b, bias, s_out, z_out, O.UINT8, O.EPI_RELU, z_b=z_b)
    g = QGemm(m, n, k, U8, U8, U8, RELU, z_a, z_out, to_bytes(b, U8), bias, s_a, s_b, s_out, z_b=z_b)
    c = g(torch.from_numpy(to_bytes(a, U8)).cuda())
    torch.cuda.synchronize()
    assert_bytes_equal(c.cpu().numpy(), to_bytes(want, U8), "gemm uint8 weights")
    assert len(np.unique(c.cpu().numpy())) >= 64
