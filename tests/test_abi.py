"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/iqnn.h declares, rejects invalid arguments with the documented status
before any device work, and its host prepack computes the folded bias,
multipliers and weight layout the oracle's own qparam functions imply."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from integer_quantized_nn_amd import binding as B
from parity_util import otype, to_bytes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libiqnn.so is not built (run __graft_entry__.build())")
    return B.lib()


def test_exports_every_declared_symbol(lib):
    header = open(os.path.join(ROOT, "include", "iqnn.h")).read()
    names = set(re.findall(r"\b(iqnn_[a-z0-9_]+)\s*\(", header))
    assert len(names) >= 14
    raw = ctypes.CDLL(B.LIB_PATH)
    missing = [n for n in sorted(names) if not hasattr(raw, n)]
    assert not missing, missing


def test_version_and_status_strings(lib):
    assert B.iqnn_abi_version() == 5
    assert lib.iqnn_status_str(0) == b"IQNN_OK"
    assert lib.iqnn_status_str(4) == b"IQNN_ERR_OVERFLOW"


def test_kernel_cfg_is_validated_before_launch(lib):
    """iqnn_qconv_fwd_cfg / iqnn_qgemm_fwd_cfg reject a tile outside -1..23 and an XCD
    group count other than 0, 1, 2, 4, 8 before touching any pointer (null device
    pointers here: reaching a launch would fail differently), and the library exports
    no process-wide tuning knob any more."""
    d = conv_desc()
    g = B.GemmDesc()
    g.m, g.n, g.k = 64, 64, 64
    g.a_type, g.b_type, g.c_type, g.res_type, g.epilogue = B.INT8, B.INT8, B.INT8, B.INT8, B.EPI_NONE
    for bad, word in (((-2, 0), "tile"), ((24, 0), "tile"), ((-1, 3), "xcd_groups"), ((10, 16), "xcd_groups")):
        with pytest.raises(B.IqnnError) as ei:
            B.iqnn_qconv_fwd_cfg(d, 0, 0, None, 0, bad, stream=0)
        assert ei.value.status == 1 and word in str(ei.value), str(ei.value)
        with pytest.raises(B.IqnnError) as ei:
            B.iqnn_qgemm_fwd_cfg(g, 0, 0, None, 0, bad, stream=0)
        assert ei.value.status == 1 and word in str(ei.value), str(ei.value)
    # a valid configuration passes validation and fails on the null pointers instead
    for ok in ((-1, 0), (0, 1), (23, 8), (19, 2)):
        with pytest.raises(B.IqnnError) as ei:
            B.iqnn_qconv_fwd_cfg(d, 0, 0, None, 0, ok, stream=0)
        assert ei.value.status == 1 and "null" in str(ei.value), str(ei.value)
    assert not hasattr(lib, "iqnn_set_conv_tile")


def conv_desc(**kw):
    d = B.ConvDesc()
    base = dict(n=1, h=8, w=8, c_in=16, c_out=32, kh=3, kw=3, stride_h=1, stride_w=1, pad_h=1, pad_w=1,
                x_type=B.UINT8, w_type=B.INT8, y_type=B.UINT8, res_type=B.UINT8, epilogue=B.EPI_RELU,
                z_in=3, z_out=5, z_res=0, z_w=0)
    base.update(kw)
    for k, v in base.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("kw,status", [
    (dict(n=0), 1), (dict(c_out=0), 1), (dict(kh=11, pad_h=0), 1), (dict(x_type=7), 1),
    (dict(w_type=9), 1), (dict(w_type=B.UINT8, z_w=256), 1), (dict(w_type=B.INT4, z_w=8), 1),
    # a weight zero point other than the kernel's weight shift needs the streaming path
    (dict(w_type=B.UINT8), 2), (dict(w_type=B.INT8, z_w=5), 2),
    (dict(x_type=B.UINT4, c_in=64, w_type=B.UINT4, z_w=3), 2),
    (dict(c_in=64, w_type=B.UINT8, z_w=7, epilogue=B.EPI_ADD, res_type=B.UINT4), 2),
    (dict(y_type=B.INT32), 1), (dict(epilogue=B.EPI_RAW_INT32), 1),
    (dict(z_in=300), 1), (dict(z_out=-1), 1), (dict(x_type=B.UINT4, c_in=8, z_in=3), 2),
    (dict(epilogue=B.EPI_ADD, res_type=9), 1), (dict(y_type=B.UINT4, c_out=33, z_out=1), 1),
    (dict(stride_h=0), 1), (dict(pad_w=-1), 1),
])
def test_invalid_descriptors_are_rejected(lib, kw, status):
    d = conv_desc(**kw)
    assert lib.iqnn_qconv_packed_size(ctypes.byref(d)) == 0
    assert B.lib().iqnn_last_error().decode() != ""
    rc = lib.iqnn_qconv_fwd(ctypes.byref(d), ctypes.c_void_p(4096), ctypes.c_void_p(4096), None,
                            ctypes.c_void_p(4096), None)
    assert rc == status


def test_forward_argument_errors_before_launch(lib):
    d = conv_desc(epilogue=B.EPI_ADD_RELU)
    P = ctypes.c_void_p
    assert lib.iqnn_qconv_fwd(ctypes.byref(d), P(4096), P(4096), None, P(4096), None) == 1   # no residual
    d = conv_desc()
    assert lib.iqnn_qconv_fwd(ctypes.byref(d), P(4097), P(4096), None, P(4096), None) == 3   # misaligned x
    assert lib.iqnn_qconv_fwd(ctypes.byref(d), P(4096), P(4112), None, P(4096), None) == 3   # packed not 256-aligned
    assert lib.iqnn_qconv_fwd(ctypes.byref(d), None, P(4096), None, P(4096), None) == 1
    assert "null" in lib.iqnn_last_error().decode()


def test_fused_conv_pool_rejects_other_shapes_before_launch(lib):
    P = ctypes.c_void_p
    stem = conv_desc(n=2, h=38, w=38, c_in=4, c_out=64, kh=7, kw=7, stride_h=2, stride_w=2, pad_h=0, pad_w=0)
    d = conv_desc()   # a 3x3 16-channel layer: not the stem shape class
    assert lib.iqnn_qconv_maxpool_fwd(ctypes.byref(d), P(4096), P(4096), P(4096), 3, 2, 1, None) == 2
    assert "stem" in lib.iqnn_last_error().decode()
    assert lib.iqnn_qconv_maxpool_fwd(ctypes.byref(stem), P(4096), P(4096), P(4096), 2, 2, 0, None) == 2
    d = conv_desc(n=2, h=38, w=38, c_in=4, c_out=32, kh=7, kw=7, stride_h=2, stride_w=2, pad_h=0, pad_w=0)
    assert lib.iqnn_qconv_maxpool_fwd(ctypes.byref(d), P(4096), P(4096), P(4096), 3, 2, 1, None) == 2
    d = conv_desc(n=2, h=38, w=38, c_in=4, c_out=64, kh=7, kw=7, stride_h=2, stride_w=2, pad_h=0, pad_w=0,
                  epilogue=B.EPI_ADD_RELU)
    assert lib.iqnn_qconv_maxpool_fwd(ctypes.byref(d), P(4096), P(4096), P(4096), 3, 2, 1, None) == 2
    assert lib.iqnn_qconv_maxpool_fwd(ctypes.byref(stem), P(4100), P(4096), P(4096), 3, 2, 1, None) == 3
    assert lib.iqnn_qconv_maxpool_fwd(ctypes.byref(stem), P(4096), P(4096), None, 3, 2, 1, None) == 1


def test_pair_validated_before_launch(lib):
    """iqnn_qconv_pair_fwd checks both descriptors, that the second takes the first's
    output (N, H, W, C_in, type, zero point), and every pointer of both calls before
    anything is launched (fake device addresses here: a launch would fail otherwise)."""
    P = ctypes.c_void_p
    a = conv_desc(n=2, h=7, w=9, c_in=64, c_out=256, kh=1, kw=1, pad_h=0, pad_w=0, epilogue=B.EPI_ADD_RELU,
                  z_out=5)
    b = conv_desc(n=2, h=7, w=9, c_in=256, c_out=64, kh=1, kw=1, pad_h=0, pad_w=0, z_in=5)
    x, pk, r, y = P(4096), P(8192), P(4096), P(4096)

    def call(da, db, *ptrs):
        return lib.iqnn_qconv_pair_fwd(ctypes.byref(da), ctypes.byref(db), *ptrs, None)

    for bad in (dict(c_in=128), dict(h=8), dict(n=3), dict(z_in=6), dict(x_type=B.INT8)):
        kb = dict(n=2, h=7, w=9, c_in=256, c_out=64, kh=1, kw=1, pad_h=0, pad_w=0, z_in=5)
        kb.update(bad)
        assert call(a, conv_desc(**kb), x, pk, r, pk, y, y) == 1, bad
        assert "first conv's output" in lib.iqnn_last_error().decode()
    assert call(a, b, x, pk, None, pk, y, y) == 1                       # ADD_RELU without residual
    assert call(a, b, x, pk, r, None, y, y) == 1                        # second packed buffer
    assert call(a, b, x, pk, r, pk, y, None) == 1                       # second output
    assert call(a, b, P(4100), pk, r, pk, y, y) == 3                    # misaligned x
    assert call(a, b, x, pk, r, pk, y, P(4104)) == 3                    # misaligned second output
    assert call(a, b, x, pk, r, P(8208), y, y) == 3                     # second packed not 256-aligned
    assert call(conv_desc(n=0), b, x, pk, r, pk, y, y) == 1             # invalid first descriptor
    assert call(a, conv_desc(c_out=0), x, pk, r, pk, y, y) == 1         # invalid second descriptor


def test_empty_and_oversized_inputs(lib):
    P = ctypes.c_void_p
    # empty tensors: nothing to read or write, no launch, no pointer needed
    assert lib.iqnn_quantize(None, None, 0, 3, 1, None, None, 0, B.UINT8, None) == 0
    assert lib.iqnn_dequantize(None, None, 0, 3, 1, None, None, 0, B.INT4, None) == 0
    assert lib.iqnn_quantize_pad(None, None, 0, 8, 8, 3, 3, 4, None, None, 0, B.UINT8, None) == 0
    # an empty batch or GEMM has no valid descriptor
    g = B.GemmDesc()
    g.m, g.n, g.k = 0, 16, 64
    g.a_type, g.b_type, g.c_type, g.res_type, g.epilogue = B.UINT8, B.INT8, B.INT8, B.UINT8, B.EPI_NONE
    assert lib.iqnn_qgemm_fwd(ctypes.byref(g), P(4096), P(4096), None, P(4096), None) == 1
    # size limits, all reported before any launch
    assert lib.iqnn_qconv_fwd(ctypes.byref(conv_desc(c_out=(1 << 24) + 16, kh=1, kw=1, pad_h=0, pad_w=0)),
                              P(4096), P(4096), None, P(4096), None) == 2
    huge = conv_desc(n=1 << 20, h=1 << 11, w=1 << 11, kh=1, kw=1, pad_h=0, pad_w=0)   # 2^42 output pixels
    assert lib.iqnn_qconv_fwd(ctypes.byref(huge), P(4096), P(4096), None, P(4096), None) == 2
    assert lib.iqnn_maxpool2d(P(4096), P(4096), 1 << 16, 512, 512, 16, 3, 1, 1, B.UINT8, None) == 2
    assert lib.iqnn_quantize_pad(P(4096), P(4096), 1 << 16, 256, 256, 3, 0, 4, P(4096), P(4096), 0, B.UINT8,
                                 None) == 2
    g.m, g.k, g.b_type, g.z_b = 256, 96, B.UINT8, 9   # Z_B term needs K % 64 == 0
    assert lib.iqnn_qgemm_fwd(ctypes.byref(g), P(4096), P(4096), None, P(4096), None) == 2


def test_quantize_and_pool_argument_errors(lib):
    P = ctypes.c_void_p
    assert lib.iqnn_quantize(P(4096), P(4096), 1, 3, 1, P(4096), P(4096), 0, 9, None) == 1
    assert lib.iqnn_quantize(P(4096), P(4096), 1, 3, 1, P(4096), P(4096), 0, B.UINT4, None) == 1   # odd count
    assert lib.iqnn_quantize(P(4100), P(4096), 1, 4, 1, P(4096), P(4096), 0, B.INT8, None) == 3
    assert lib.iqnn_dequantize(P(4096), P(4096), 1, 0, 1, P(4096), P(4096), 0, B.INT8, None) == 1
    assert lib.iqnn_maxpool2d(P(4096), P(4096), 1, 8, 8, 16, 3, 2, 2, B.UINT8, None) == 1   # 2p > k-1
    assert lib.iqnn_maxpool2d(P(4096), P(4096), 1, 8, 8, 12, 3, 2, 1, B.UINT8, None) == 2   # C % 16
    assert lib.iqnn_maxpool2d(P(4096), P(4096), 1, 8, 8, 16, 3, 2, 1, B.UINT4, None) == 2


def _host_pack(d, w_codes, wt, bias, s_in, s_w, s_out, s_res=1.0):
    size = B.iqnn_qconv_packed_size(d)
    buf = np.zeros(size, np.uint8)
    B.iqnn_qconv_prepack_host(d, to_bytes(w_codes, wt), bias, s_in, s_w, np.size(s_w) > 1, s_out, s_res, buf)
    return buf


def _unpack_layout(buf, c_out, k, act4, stream4=False):
    ocp = (c_out + 255) // 256 * 256
    kp = (k + 63) // 64 * 64
    bias = buf[:4 * ocp].view(np.int32)
    mult = buf[4 * ocp:8 * ocp].view(np.float32)
    mres = buf[8 * ocp:8 * ocp + 4].view(np.float32)[0]
    pad = buf[8 * ocp + 64:8 * ocp + 128]
    w = buf[8 * ocp + 256:8 * ocp + 256 + ocp * kp].view(np.int8).reshape(ocp, kp)
    rows = []
    for c in range(c_out):
        b, r32 = divmod(c, 32)
        h, j, r = r32 // 16, (r32 // 4) % 4, r32 % 4
        rows.append(32 * b + 8 * j + 4 * h + r)
    w = w[rows][:, :k]
    if act4:
        # nibble unpack order inside every 16 K positions; with the streaming kernel's
        # 4-bit layout (C_in % 64 == 0) also blocks 1 and 2 of every 64 trade places
        order = [0, 2, 4, 6, 1, 3, 5, 7, 8, 10, 12, 14, 9, 11, 13, 15]
        logical = np.empty_like(w)
        for s0 in range(0, k, 16):
            blk = (s0 // 16) % 4
            src0 = s0 - 16 * blk + 16 * ({1: 2, 2: 1}.get(blk, blk) if stream4 else blk)
            for p, e in enumerate(order):
                logical[:, s0 + e] = w[:, src0 + p]
        w = logical
    return bias[:c_out], mult[:c_out], mres, w, pad


@pytest.mark.parametrize("x_type,w_type,c_in,c_out,epi", [
    (B.UINT8, B.INT8, 16, 96, B.EPI_RELU),
    (B.INT8, B.INT8, 32, 64, B.EPI_NONE),
    (B.UINT4, B.INT4, 32, 48, B.EPI_ADD_RELU),
    (B.INT4, B.INT4, 16, 16, B.EPI_ADD),
    (B.UINT4, B.INT4, 64, 64, B.EPI_ADD_RELU),
    (B.UINT8, B.INT8, 3, 64, B.EPI_RELU),
])
def test_host_prepack_matches_oracle_qparams(lib, x_type, w_type, c_in, c_out, epi):
    rng = np.random.default_rng(c_in * 1000 + c_out)
    lo, hi = O.qrange(otype(w_type))
    w = rng.integers(lo, hi + 1, size=(c_out, 3, 3, c_in)).astype(np.int32)
    xlo, xhi = O.qrange(otype(x_type))
    z_in = int(rng.integers(xlo, xhi + 1)) if x_type in (B.UINT8, B.UINT4) else 0
    s_in = np.float32(0.013)
    s_w = rng.uniform(0.001, 0.01, c_out).astype(np.float32)
    bias = rng.normal(0, 0.3, c_out).astype(np.float32)
    s_out, s_res = np.float32(0.07), np.float32(0.031)
    y_type = B.UINT8 if x_type == B.UINT8 else (B.INT8 if x_type == B.INT8 else B.UINT4)
    d = conv_desc(x_type=x_type, w_type=w_type, y_type=y_type, c_in=c_in, c_out=c_out, epilogue=epi, z_in=z_in,
                  z_out=1, res_type=B.UINT4, z_res=2)
    buf = _host_pack(d, w, w_type, bias, s_in, s_w, s_out, s_res)
    act4 = x_type in (B.UINT4, B.INT4)
    fold, mult, mres, wl, pad = _unpack_layout(buf, c_out, 9 * c_in, act4, stream4=act4 and c_in % 64 == 0)
    # the padding row holds the raw input zero-point code (two per byte for 4-bit codes)
    assert np.all(pad == ((z_in & 0xF) * 0x11 if act4 else z_in & 0xFF))
    # weights: exactly the codes, back in OHWI order after undoing the documented permutations
    assert np.array_equal(wl.astype(np.int32), w.reshape(c_out, -1))
    # multipliers: the oracle's requant_multiplier / residual_multiplier
    assert np.array_equal(mult, O.requant_multiplier(s_in, s_w, s_out))
    if epi in (B.EPI_ADD, B.EPI_ADD_RELU):
        assert mres == O.residual_multiplier(s_res, s_out)
    # folded bias: the oracle's bias quantization minus the zero-point term, checked through
    # the fold identity on a one-pixel input where every tap reads the input value q:
    # sum_k (q - Z) w + bias_q == sum_k (q - shift) w + fold.
    shift = 128 if x_type == B.UINT8 else 0
    bq = O.quantize_bias(bias, s_in, s_w).astype(np.int64)
    for q in (xlo, z_in, xhi):
        lhs = (q - z_in) * w.reshape(c_out, -1).astype(np.int64).sum(1) + bq
        rhs = (q - shift) * w.reshape(c_out, -1).astype(np.int64).sum(1) + fold.astype(np.int64)
        assert np.array_equal(lhs, rhs)


@pytest.mark.parametrize("x_type,w_type,z_w,c_in,epi", [
    (B.UINT8, B.UINT8, 131, 64, B.EPI_RELU),
    (B.INT8, B.UINT8, 0, 128, B.EPI_NONE),
    (B.UINT8, B.INT8, -7, 64, B.EPI_ADD_RELU),
    (B.UINT8, B.UINT4, 6, 64, B.EPI_RELU),
    (B.UINT8, B.UINT8, 128, 16, B.EPI_RELU),   # z_w == the weight shift: no per-pixel term, any path
])
def test_host_prepack_asymmetric_weights(lib, x_type, w_type, z_w, c_in, epi):
    # MegEngine 4-bit article, section 緩解精度下降: with Z_W != 0 only the Z_I and Z_I*Z_W
    # terms are known before inference; the Z_W * sum Q(I) term stays per pixel.
    rng = np.random.default_rng(c_in + 7 * z_w % 1000)
    c_out = 48
    lo, hi = O.qrange(otype(w_type))
    w = rng.integers(lo, hi + 1, size=(c_out, 3, 3, c_in)).astype(np.int32)
    xlo, xhi = O.qrange(otype(x_type))
    z_in = int(rng.integers(xlo, xhi + 1)) if x_type == B.UINT8 else -5
    s_in, s_out, s_res = np.float32(0.02), np.float32(0.09), np.float32(0.04)
    s_w = rng.uniform(0.001, 0.01, c_out).astype(np.float32)
    bias = rng.normal(0, 0.3, c_out).astype(np.float32)
    d = conv_desc(x_type=x_type, w_type=w_type, z_w=z_w, c_in=c_in, c_out=c_out, epilogue=epi, z_in=z_in,
                  y_type=B.UINT8, z_out=2, res_type=B.UINT8, z_res=9)
    buf = _host_pack(d, w, w_type, bias, s_in, s_w, s_out, s_res)
    fold, mult, _, wl, _ = _unpack_layout(buf, c_out, 9 * c_in, False)
    s_w_shift = 128 if w_type == B.UINT8 else 0
    assert np.array_equal(wl.astype(np.int32), w.reshape(c_out, -1) - s_w_shift)
    assert np.array_equal(mult, O.requant_multiplier(s_in, s_w, s_out))
    # every tap reads q: sum_k (q - Z_in)(w - Z_w) + bias_q
    #   == sum_k (q - s)(w - s_w) + fold + (s_w - Z_w) * K * (q - s)
    s = 128 if x_type == B.UINT8 else 0
    k = 9 * c_in
    bq = O.quantize_bias(bias, s_in, s_w).astype(np.int64)
    wf = w.reshape(c_out, -1).astype(np.int64)
    for q in (xlo, z_in, xhi):
        lhs = (q - z_in) * (wf - z_w).sum(1) + bq
        rhs = (q - s) * (wf - s_w_shift).sum(1) + fold.astype(np.int64) + (s_w_shift - z_w) * k * (q - s)
        assert np.array_equal(lhs, rhs)


@pytest.mark.parametrize("kw", [dict(epilogue=B.EPI_ADD_RELU | B.EPI_INT_REQUANT),
                                dict(epilogue=B.EPI_RAW_INT32 | B.EPI_INT_REQUANT, y_type=B.INT32),
                                dict(epilogue=B.EPI_RELU | B.EPI_INT_REQUANT, c_in=64, w_type=B.UINT8, z_w=3)])
def test_integer_requant_unsupported_combinations(lib, kw):
    d = conv_desc(**kw)
    rc = lib.iqnn_qconv_fwd(ctypes.byref(d), ctypes.c_void_p(4096), ctypes.c_void_p(4096), ctypes.c_void_p(4096),
                            ctypes.c_void_p(4096), None)
    assert rc == 2


def test_host_prepack_integer_multipliers(lib):
    # the packed multiplier slot holds M * 2^-N (exact in binary32) with (M, N) =
    # get_MN(M[c]) (FQ-ViT article, LayerNorm code), checked against the oracle's get_mn
    rng = np.random.default_rng(21)
    c_out, c_in = 40, 32
    w = rng.integers(-127, 128, size=(c_out, 3, 3, c_in)).astype(np.int32)
    s_w = np.exp(rng.uniform(np.log(1e-5), np.log(1e-1), c_out)).astype(np.float32)
    s_in, s_out = np.float32(0.013), np.float32(0.07)
    d = conv_desc(c_in=c_in, c_out=c_out, epilogue=B.EPI_RELU | B.EPI_INT_REQUANT)
    buf = _host_pack(d, w, B.INT8, None, s_in, s_w, s_out)
    ocp = 256
    slots = buf[4 * ocp:8 * ocp].view(np.float32)[:c_out]
    want = [O.get_mn(m) for m in O.requant_multiplier(s_in, s_w, s_out)]
    assert [float(v) for v in slots] == [float(mm) * 2.0 ** -nn for mm, nn in want]
    assert lib.iqnn_qconv_maxpool_fwd(ctypes.byref(conv_desc(n=2, h=38, w=38, c_in=4, c_out=64, kh=7, kw=7,
                                                             stride_h=2, stride_w=2, pad_h=0, pad_w=0,
                                                             epilogue=B.EPI_RELU | B.EPI_INT_REQUANT)),
                                      ctypes.c_void_p(4096), ctypes.c_void_p(4096), ctypes.c_void_p(4096), 3, 2, 1,
                                      None) == 2


def test_prepack_overflow_and_bad_scales(lib):
    d = conv_desc(c_in=16, c_out=16)
    w = np.full((16, 3, 3, 16), 127, np.int32)
    with pytest.raises(B.IqnnError) as e:
        _host_pack(d, w, B.INT8, np.full(16, 1e9, np.float32), np.float32(1e-3), np.full(16, 1e-3, np.float32), 1.0)
    assert e.value.status == 4
    with pytest.raises(B.IqnnError) as e:
        _host_pack(d, w, B.INT8, None, np.float32(-1.0), np.full(16, 1e-3, np.float32), 1.0)
    assert e.value.status == 1
    with pytest.raises(B.IqnnError) as e:   # multiplier underflows to a denormal
        _host_pack(d, w, B.INT8, None, np.float32(1e-20), np.full(16, 1e-20, np.float32), 1e10)
    assert e.value.status == 1


def _bf6_value(code):
    """Real value of a BF6 (e3m2) code: sign, 3 exponent bits (bias 3), 2 mantissa bits."""
    sign = -1 if code & 32 else 1
    e, m = (code >> 2) & 7, code & 3
    return sign * (m / 4 * 2.0 ** -2 if e == 0 else (1 + m / 4) * 2.0 ** (e - 3))


@pytest.mark.parametrize("x_type,c_out", [(B.UINT4, 96), (B.INT4, 64)])
def test_host_prepack_fp6_region(lib, x_type, c_out):
    """4-bit streaming layers with INT4 weights carry a BF6 copy of the weights and a
    bias for the FP6 path after the standard layout: the copy decodes to the weight
    codes, and the bias is the folded bias plus 8 * sum(W) for UINT4 activations (the
    path contracts q - 8)."""
    rng = np.random.default_rng(c_out)
    c_in, k = 64, 9 * 64
    w = rng.integers(-8, 8, size=(c_out, 3, 3, c_in)).astype(np.int32)
    bias = rng.normal(0, 0.3, c_out).astype(np.float32)
    s_w = rng.uniform(0.01, 0.05, c_out).astype(np.float32)
    z_in = 5 if x_type == B.UINT4 else 0
    d = conv_desc(x_type=x_type, w_type=B.INT4, y_type=B.UINT4, c_in=c_in, c_out=c_out, epilogue=B.EPI_RELU,
                  z_in=z_in, z_out=1)
    buf = _host_pack(d, w, B.INT4, bias, np.float32(0.05), s_w, np.float32(0.07))
    ocp, kp = 256, (k + 63) // 64 * 64
    std_bytes = 8 * ocp + 256 + 2 * ocp * kp
    assert buf.size == std_bytes + 4 * ocp + ocp * kp
    folded = buf[:4 * ocp].view(np.int32)[:c_out].astype(np.int64)
    bias_f6 = buf[std_bytes:std_bytes + 4 * ocp].view(np.int32)[:c_out]
    shift = 8 if x_type == B.UINT4 else 0
    assert np.array_equal(bias_f6, folded + shift * w.reshape(c_out, -1).sum(axis=1))
    # blocks: 4 KB per (64-row group, stage); row R's 8-byte unit u at u ^ ((R >> 2) & 7)
    nst = kp // 64
    blocks = buf[std_bytes + 4 * ocp:].reshape(ocp // 64, nst, 64, 64)
    rows = []
    for c in range(c_out):
        b, r32 = divmod(c, 32)
        h, j, r = r32 // 16, (r32 // 4) % 4, r32 % 4
        rows.append(32 * b + 8 * j + 4 * h + r)
    logical = w.reshape(c_out, -1)
    for c in range(0, c_out, 7):
        R = rows[c]
        for s in range(nst):
            rowbytes = blocks[R // 64, s, R % 64]
            for h in range(2):
                half = b"".join(bytes(rowbytes[8 * ((3 * h + i) ^ ((R >> 2) & 7)):][:8]) for i in range(3))
                bits = int.from_bytes(half, "little")
                vals = [_bf6_value((bits >> (6 * v)) & 63) for v in range(32)]
                assert vals == list(logical[c, s * 64 + 32 * h:s * 64 + 32 * h + 32]), (c, s, h)


def test_fused_stem_pool_rejects_inputs_of_partial_16_byte_units(lib):
    """iqnn_qconv_maxpool_fwd moves its input in whole 16-byte units, so an input of
    N*H*W*4 = 8 mod 16 bytes (N = 1, 37x38x4) is UNSUPPORTED, decided from the
    descriptor before any pointer is used (the addresses here are aligned stand-ins
    that are never dereferenced)."""
    d = conv_desc(n=1, h=37, w=38, c_in=4, c_out=64, kh=7, kw=7, stride_h=2, stride_w=2, pad_h=0, pad_w=0,
                  y_type=B.UINT8, epilogue=B.EPI_RELU)
    fake = 1 << 20
    with pytest.raises(B.IqnnError) as ei:
        B.iqnn_qconv_maxpool_fwd(d, fake, fake, fake, 3, 2, 1, stream=0)
    assert ei.value.status == 2 and "16" in str(ei.value), str(ei.value)


@pytest.mark.parametrize("x_type,c_out,epi", [(B.UINT4, 96, B.EPI_RELU), (B.INT4, 128, B.EPI_ADD_RELU)])
def test_host_prepack_packed_int4_weights(lib, x_type, c_out, epi):
    """4-bit streaming layers with INT4 weights and more than 64 output channels keep the
    weights packed (two codes per byte) in the tile-order copy the kernel reads: 2 KB per
    (64-row group, 64-K stage), 32 bytes per row in K order with the low nibble first,
    the row's 16-byte halves swapped on rows with bit 3 set.  Decoding the blocks gives
    back every weight code (in the documented row permutation)."""
    rng = np.random.default_rng(c_out + 7)
    c_in, k = 64, 9 * 64
    w = rng.integers(-8, 8, size=(c_out, 3, 3, c_in)).astype(np.int32)
    d = conv_desc(x_type=x_type, w_type=B.INT4, y_type=B.UINT4, c_in=c_in, c_out=c_out, epilogue=epi,
                  z_in=3 if x_type == B.UINT4 else 0, z_out=1, res_type=B.UINT4, z_res=2)
    buf = _host_pack(d, w, B.INT4, None, np.float32(0.05), np.full(c_out, 0.02, np.float32), np.float32(0.07),
                     np.float32(0.03))
    ocp, kp = 256, k
    t_off = 8 * ocp + 256 + ocp * kp
    nst = kp // 64
    blocks = buf[t_off:t_off + ocp * kp // 2].reshape(ocp // 64, nst, 64, 32)
    logical = w.reshape(c_out, -1)
    for c in range(c_out):
        b, r32 = divmod(c, 32)
        h, j, r = r32 // 16, (r32 // 4) % 4, r32 % 4
        R = 32 * b + 8 * j + 4 * h + r
        for s in range(nst):
            row = blocks[R // 64, s, R % 64]
            sw = (R >> 3) & 1
            nat = np.concatenate([row[16 * (0 ^ sw):16 * (0 ^ sw) + 16], row[16 * (1 ^ sw):16 * (1 ^ sw) + 16]])
            codes = np.empty(64, np.int32)
            codes[0::2] = nat & 0xF
            codes[1::2] = nat >> 4
            codes[codes >= 8] -= 16
            assert np.array_equal(codes, logical[c, 64 * s:64 * s + 64]), (c, s)
    # the rest of the tile-order region and the padding rows stay zero
    assert not buf[t_off + ocp * kp // 2:t_off + ocp * kp].any()
