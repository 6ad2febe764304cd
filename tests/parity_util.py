"""Shared helpers of the parity tests: run one seeded case through the CPU oracle
and through libiqnn, and compare the output bytes."""
import numpy as np
import pytest

import oracle as O

# library dtype / epilogue numbering as named in include/iqnn.h
LIB_T = {"INT8": 0, "UINT8": 1, "INT4": 2, "UINT4": 3, "INT32": 4}
# oracle numbering, matched by name (the two sides define their own constants)
ORC_T = {"INT8": O.INT8, "UINT8": O.UINT8, "INT4": O.INT4, "UINT4": O.UINT4, "INT32": O.INT32}
T_NAME = {0: "INT8", 1: "UINT8", 2: "INT4", 3: "UINT4", 4: "INT32",
          5: "INT8"}   # IQNN_INT8_2OF4: 2:4-sparse weights are dense INT8 codes to the oracle
EPI_NAME = {0: "NONE", 1: "RELU", 2: "ADD", 3: "ADD_RELU", 4: "RAW"}
ORC_EPI = {"NONE": O.EPI_NONE, "RELU": O.EPI_RELU, "ADD": O.EPI_ADD, "ADD_RELU": O.EPI_ADD_RELU, "RAW": O.EPI_RAW}


def otype(t):
    """Oracle type for a synth/library type number."""
    return ORC_T[T_NAME[t]]


def oepi(e):
    return ORC_EPI[EPI_NAME[e]]


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this process")
    # On a GPU machine the library must be there: no fallback exists.
    from integer_quantized_nn_amd import binding
    binding.lib()
    return torch


def to_bytes(codes, t):
    """Oracle codes -> packed bytes (oracle packing).  INT32 -> little-endian bytes."""
    if t == 4:
        return np.ascontiguousarray(codes.astype(np.int32)).view(np.uint8).reshape(codes.shape[:-1] + (-1,))
    return O.pack(codes, otype(t))


def describe_mismatch(got, want):
    got = np.asarray(got)
    want = np.asarray(want)
    if got.shape != want.shape:
        return "shape %s != %s" % (got.shape, want.shape)
    bad = np.nonzero(got.reshape(-1) != want.reshape(-1))[0]
    if bad.size == 0:
        return "equal"
    i = bad[0]
    return "%d of %d bytes differ; first at flat %d (unravel %s): got %d want %d" % (
        bad.size, got.size, i, np.unravel_index(i, got.shape), got.reshape(-1)[i], want.reshape(-1)[i])


def assert_bytes_equal(got, want, what=""):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape and np.array_equal(got, want), what + ": " + describe_mismatch(got, want)


# -------------------------------------------------------------------- conv


def conv_codes(case):
    """Oracle-quantized codes of a synth.ConvCase: (x, w, res) int32 codes."""
    x = O.quantize(case.x, case.s_in, case.z_in, otype(case.x_type))
    w = O.quantize(case.w, case.s_w, 0, otype(case.w_type), axis=0)
    res = None
    if case.res is not None:
        res = O.quantize(case.res, case.s_res, case.z_res, otype(case.res_type))
    return x, w, res


def oracle_conv(case, x, w, res, images=None, z_w=0, s_w=None):
    """Oracle output codes (int32) for the given images (default: all).  z_w / s_w:
    weight zero point and scale when the weight codes are not case.w_type symmetric."""
    if images is not None:
        x = x[images]
        res = res[images] if res is not None else None
    return O.qconv(x, case.z_in, case.s_in, w, case.s_w if s_w is None else s_w, case.bias, case.s_out,
                   case.z_out, otype(case.y_type), oepi(case.epi), case.stride, case.pad, res, case.s_res,
                   case.z_res, z_w=z_w)


def gpu_conv(case, x, w, res, stream=None, w_type=None, z_w=0, s_w=None, cfg=None):
    """libiqnn output bytes (numpy) for the whole batch; cfg: (tile, xcd_groups) of the
    call (iqnn_qconv_fwd_cfg), None for the automatic choice."""
    import torch
    from integer_quantized_nn_amd.layers import QConv
    n, h, wd, ci = x.shape
    co, kh, kw, _ = w.shape
    wt = case.w_type if w_type is None else w_type
    conv = QConv(n, h, wd, ci, co, kh, case.stride, case.pad, case.x_type, wt, case.y_type, case.epi,
                 case.z_in, case.z_out, to_bytes(w, wt), case.bias, case.s_in, case.s_w if s_w is None else s_w,
                 case.s_out, res_type=case.res_type, z_res=case.z_res, s_res=case.s_res, kw=kw, stream=stream,
                 z_w=z_w)
    xd = torch.from_numpy(to_bytes(x, case.x_type)).cuda()
    rd = torch.from_numpy(to_bytes(res, case.res_type)).cuda() if res is not None else None
    y = conv(xd, res=rd, stream=stream, cfg=cfg)
    torch.cuda.synchronize()
    return y.cpu().numpy()


# -------------------------------------------------------------------- gemm


def gemm_codes(case):
    a = case.a_codes if case.a_codes is not None else O.quantize(case.a, case.s_a, case.z_a, otype(case.a_type))
    b = case.b_codes if case.b_codes is not None else O.quantize(case.b, case.s_b, 0, otype(case.b_type), axis=0)
    return a, b


def oracle_gemm(case, a, b, rows=None):
    if rows is not None:
        a = a[rows]
    return O.qgemm(a, case.z_a, case.s_a, b, case.s_b, case.bias, case.s_out, case.z_out, otype(case.c_type),
                   oepi(case.epi))


def gpu_gemm(case, a, b, stream=None, cfg=None):
    import torch
    from integer_quantized_nn_amd.layers import QGemm
    m, k = a.shape
    n = b.shape[0]
    g = QGemm(m, n, k, case.a_type, case.b_type, case.c_type, case.epi, case.z_a, case.z_out,
              to_bytes(b, case.b_type), case.bias, case.s_a, case.s_b, case.s_out, stream=stream)
    ad = torch.from_numpy(to_bytes(a, case.a_type)).cuda()
    c = g(ad, stream=stream, cfg=cfg)
    torch.cuda.synchronize()
    return c.cpu().numpy()
