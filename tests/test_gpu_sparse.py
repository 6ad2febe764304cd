"""GPU parity of 2:4-sparse weights (IQNN_INT8_2OF4, the sparse int8 MFMA): the
oracle computes the plain convolution / GEMM of the same int8 codes, zeros
included, so every output byte must equal it.  The float weights are magnitude-
pruned to 2:4 along the input channels before quantization (a symmetric per-channel
quantization keeps the zeros and each channel's largest weight, so the scales are
those of the unpruned weights)."""
import numpy as np
import pytest

import oracle as O
from integer_quantized_nn_amd import binding as B
from integer_quantized_nn_amd import synth
from parity_util import (assert_bytes_equal, conv_codes, gpu_conv, oracle_conv, oracle_gemm, require_gpu,
                         to_bytes)

pytestmark = pytest.mark.gpu

U8, I8, I32 = synth.UINT8, synth.INT8, synth.INT32
NONE, RELU, ADD_RELU, RAW = synth.EPI_NONE, synth.EPI_RELU, synth.EPI_ADD_RELU, synth.EPI_RAW
SP = B.INT8_2OF4

CASES = [
    # n, h, w, c_in, c_out, k, stride, pad, x_type, y_type, epi
    (2, 9, 11, 64, 96, 3, 1, 1, U8, U8, RELU),         # 3x3, a partly empty channel block
    (2, 6, 9, 128, 256, 1, 2, 0, U8, U8, NONE),        # strided 1x1 (gather path), two channel blocks
    (3, 7, 7, 64, 128, 3, 2, 1, U8, U8, ADD_RELU),     # residual stage
    (1, 13, 5, 64, 80, 1, 1, 0, I8, I8, NONE),         # 1x1, int8 codes, ragged pixels
    (1, 10, 10, 128, 48, 3, 1, 1, U8, I32, RAW),       # raw int32 accumulators
    (1, 1, 1, 1024, 2048, 1, 1, 0, U8, U8, ADD_RELU),  # one pixel, K = 1024, 16 channel blocks
    (2, 14, 14, 256, 256, 3, 1, 1, U8, U8, RELU),      # K = 2304: 36 stages, several tiles per workgroup
    (1, 5, 5, 192, 64, 3, 1, 1, U8, U8, RELU),         # K = 1728: an odd stage count (27)
    (2, 8, 8, 64, 128, 1, 1, 0, U8, U8, RELU),         # K = 64: a single stage
]


def sparse_case(case):
    n, h, w, ci, co, k, s, p, xt, yt, epi = case
    c = synth.conv_case(hash(case) % 2 ** 31, n, h, w, ci, co, k, s, p, xt, I8, yt, epi, res_type=U8)
    c.w = synth.prune_2of4(c.w)
    return c


@pytest.mark.parametrize("case", CASES, ids=lambda c: "n%dh%dw%dci%dco%dk%ds%dp%d_x%dy%de%d" % c)
def test_conv_2of4_small_shapes(case):
    require_gpu()
    c = sparse_case(case)
    x, wc, res = conv_codes(c)
    assert np.all((wc.reshape(-1, 4) != 0).sum(axis=1) <= 2)
    want = to_bytes(oracle_conv(c, x, wc, res), c.y_type)
    got = gpu_conv(c, x, wc, res, w_type=SP)
    assert_bytes_equal(got, want, str(case))


@pytest.mark.parametrize("h,co,xt,yt,epi", [(6, 64, U8, U8, RELU), (5, 128, I8, I8, NONE), (2, 64, U8, I32, RAW)])
def test_conv_2of4_direct3x3(h, co, xt, yt, epi):
    """2:4 weights on the direct 3x3 kernel (forced through tile 18): 64-channel 3x3
    convs on 56-pixel rows, odd and two-row heights, one and two output blocks, uint8
    and int8 codes, raw int32."""
    require_gpu()
    from integer_quantized_nn_amd import binding as B
    c = synth.conv_case(h * 100 + co + xt, 2, h, 56, 64, co, 3, 1, 1, xt, I8, yt, epi)
    c.w = synth.prune_2of4(c.w)
    x, wc, res = conv_codes(c)
    want = to_bytes(oracle_conv(c, x, wc, res), yt)
    got = gpu_conv(c, x, wc, res, w_type=SP, cfg=(18, 0))
    assert_bytes_equal(got, want, "direct 2:4 h=%d co=%d" % (h, co))


def test_conv_2of4_equals_dense_kernel_on_the_3x3_workload():
    """The 3x3 workload (N=32, 56x56, 64 -> 64, Conv_Relu to uint8) with 2:4-pruned
    weights (the direct kernel's sparse variant): every output byte against the oracle
    and against the dense kernel."""
    require_gpu()
    c = synth.conv3x3_int8()
    c.w = synth.prune_2of4(c.w)
    x, wc, res = conv_codes(c)
    got = gpu_conv(c, x, wc, res, w_type=SP)
    dense = gpu_conv(c, x, wc, res, w_type=I8)
    assert_bytes_equal(got, dense, "sparse vs dense kernel")
    want = to_bytes(oracle_conv(c, x, wc, res), c.y_type)
    assert_bytes_equal(got, want, "sparse vs oracle")
    assert len(np.unique(got)) >= 64


def _gpu_gemm_2of4(case, a, b):
    import torch
    from integer_quantized_nn_amd.layers import QGemm
    m, k = a.shape
    g = QGemm(m, b.shape[0], k, case.a_type, SP, case.c_type, case.epi, case.z_a, case.z_out, to_bytes(b, I8),
              case.bias, case.s_a, case.s_b, case.s_out)
    c = g(torch.from_numpy(to_bytes(a, case.a_type)).cuda())
    torch.cuda.synchronize()
    return c.cpu().numpy()


def test_gemm_2of4_ragged():
    require_gpu()
    g = synth.vitl_fc1(seed=3, m=1000, k=256, n=384, sparse_2of4=True)
    a = O.quantize(g.a, g.s_a, g.z_a, O.UINT8)
    b = O.quantize(g.b, g.s_b, 0, O.INT8, axis=0)
    got = _gpu_gemm_2of4(g, a, b)
    assert_bytes_equal(got, to_bytes(oracle_gemm(g, a, b), g.c_type), "gemm 1000x256x384")


@pytest.mark.parametrize("m,k,n", [(1, 64, 128), (2, 128, 16), (129, 64, 300)])
def test_gemm_2of4_edges(m, k, n):
    """One row and one stage, a 16-channel output (a partly empty 128-channel block),
    ragged rows with channels spanning three blocks."""
    require_gpu()
    g = synth.vitl_fc1(seed=m + k + n, m=m, k=k, n=n, sparse_2of4=True)
    a = O.quantize(g.a, g.s_a, g.z_a, O.UINT8)
    b = O.quantize(g.b, g.s_b, 0, O.INT8, axis=0)
    got = _gpu_gemm_2of4(g, a, b)
    assert_bytes_equal(got, to_bytes(oracle_gemm(g, a, b), g.c_type), "gemm %dx%dx%d" % (m, k, n))


def test_gemm_2of4_vitl_fc1_full_size():
    """ViT-L fc1 (12608 x 1024 -> 4096) with 2:4-pruned weights: every output byte
    against the oracle's dense product of the same codes."""
    require_gpu()
    g = synth.vitl_fc1(sparse_2of4=True)
    a = O.quantize(g.a, g.s_a, g.z_a, O.UINT8)
    b = O.quantize(g.b, g.s_b, 0, O.INT8, axis=0)
    got = _gpu_gemm_2of4(g, a, b)
    assert_bytes_equal(got, to_bytes(oracle_gemm(g, a, b), g.c_type), "fc1 2:4")
    assert len(np.unique(got)) >= 64 and (np.abs(got.view(np.int8).astype(int)) == 127).mean() < 0.01
