"""CPU oracle for integer-quantized convolution and GEMM (numpy front end).

TEST INFRASTRUCTURE ONLY.  This package is the checker: the test suite, the
smoke check and the benchmark's CPU-baseline leg call it; the product path
(the GPU library and its binding) never imports it, and it imports nothing
from the product.  Every function forwards to the plain C implementation in
iqo.c (direct loops, strict binary32, no fused multiply-add); see that file
for the page passage each step follows.

Codes are numpy int32 arrays holding one logical code per element (4-bit codes
unpacked); pack()/unpack() convert to and from the byte layout.  The integer-only
requantization (get_mn, requant_int) is written here directly in numpy int64 /
Python integers, and choose_qparams in numpy binary32 scalars.

Parity pins: every function here is pinned by tests/test_oracle_*.py against
worked values printed on the pages, closed forms, library routines
(torch conv2d / max_pool2d / quantize_per_tensor, numpy matmul) and
invariants.  Functions without such a pin would be marked "parity unpinned";
there are none.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# IQO_LIB: another build of the oracle (the sanitized CPU-hygiene build, say)
_LIB_PATH = os.environ.get("IQO_LIB") or os.path.join(_HERE, "libiqo.so")

INT8, UINT8, INT4, UINT4, INT32 = 0, 1, 2, 3, 4
EPI_NONE, EPI_RELU, EPI_ADD, EPI_ADD_RELU, EPI_RAW = 0, 1, 2, 3, 4

_QRANGE = {INT8: (-128, 127), UINT8: (0, 255), INT4: (-8, 7), UINT4: (0, 15)}

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    I64 = ctypes.c_int64
    I32 = ctypes.c_int32
    F = ctypes.c_float
    sig = {
        "iqo_num_threads": (I, []),
        "iqo_set_num_threads": (None, [I]),
        "iqo_quantize": (I, [P, P, I64, I64, I64, P, P, I, I]),
        "iqo_dequantize": (I, [P, P, I64, I64, I64, P, P, I]),
        "iqo_pack": (I, [P, P, I64, I]),
        "iqo_unpack": (I, [P, P, I64, I]),
        "iqo_requant_multiplier": (F, [F, F, F]),
        "iqo_residual_multiplier": (F, [F, F]),
        "iqo_quantize_bias": (I, [F, F, F, P]),
        "iqo_conv2d_acc": (I, [P, I, I, I, I, I32, P, I, I, I, I32, I, I, I, I, P, P]),
        "iqo_gemm_acc": (I, [P, I64, I64, I32, P, I64, I32, P, P]),
        "iqo_requant": (I, [P, I64, I64, P, I, P, I32, F, I32, I, P]),
        "iqo_maxpool2d": (I, [P, I, I, I, I, I, I, I, P]),
        "iqo_im2col": (I, [P, I, I, I, I, I32, I, I, I, I, I, I, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class OracleError(RuntimeError):
    pass


def _check(rc, what):
    if rc != 0:
        raise OracleError("%s failed with code %d" % (what, rc))


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads():
    return _load().iqo_num_threads()


def set_num_threads(n):
    """Threads of the oracle's OpenMP loops from now on (timing only; results are the same)."""
    _load().iqo_set_num_threads(int(n))


def qrange(qtype):
    return _QRANGE[qtype]


def _per_channel_arrays(scale, zp, ch):
    scale = np.atleast_1d(np.asarray(scale, dtype=np.float32))
    zp = np.atleast_1d(np.asarray(zp, dtype=np.int32))
    per_channel = scale.size > 1 or zp.size > 1
    if per_channel:
        scale = np.broadcast_to(scale, (ch,)).astype(np.float32)
        zp = np.broadcast_to(zp, (ch,)).astype(np.int32)
    return _c(scale, np.float32), _c(zp, np.int32), int(per_channel)


def choose_qparams(vmin, vmax, qtype, symmetric=False):
    """Quantization parameters from a real range (FQ-ViT article, §3.1, MinMax uniform
    quantization; Horizon QAT talk, section 三: a fixed scale from the real min / max
    over the code range).  Each step is one binary32 operation (numpy float32 scalars,
    round to nearest even):
      symmetric (signed types): S = max(|min|, |max|) / Q_MAX, Z = 0;
      asymmetric: widen the range to hold 0, S = (max - min) / (Q_MAX - Q_MIN),
      Z = clip(Q_MIN - rne(min / S)), so the real 0 gets the exact code Z.
    A scale that is zero or below the smallest normal binary32 becomes 1 (every value
    of a zero-range tensor is then the code Z).  Returns (np.float32 S, int Z)."""
    f = np.float32
    q_min, q_max = qrange(qtype)
    lo_real, hi_real = f(vmin), f(vmax)
    if symmetric:
        assert q_min < 0, "symmetric parameters need a signed type"
        scale = f(max(abs(lo_real), abs(hi_real))) / f(q_max)
    else:
        lo_real = lo_real if lo_real < f(0) else f(0)
        hi_real = hi_real if hi_real > f(0) else f(0)
        scale = (hi_real - lo_real) / f(q_max - q_min)
    if not scale >= np.finfo(np.float32).tiny:
        scale = f(1)
    if symmetric:
        return f(scale), 0
    zero = q_min - int(np.rint(lo_real / scale))
    return f(scale), int(min(max(zero, q_min), q_max))


def _axis_view(shape, axis):
    axis = axis % len(shape)
    outer = int(np.prod(shape[:axis], dtype=np.int64))
    inner = int(np.prod(shape[axis + 1:], dtype=np.int64))
    return outer, int(shape[axis]), inner


def quantize(x, scale, zp, qtype, axis=-1):
    """q = clip(rne(x / S) + Z); scale/zp scalar (per tensor) or [ch] along `axis`."""
    x = _c(x, np.float32)
    outer, ch, inner = _axis_view(x.shape, axis)
    s, z, pc = _per_channel_arrays(scale, zp, ch)
    q = np.empty(x.shape, np.int32)
    _check(_load().iqo_quantize(_ptr(x), _ptr(q), outer, ch, inner, _ptr(s), _ptr(z), pc, qtype),
           "quantize")
    return q


def dequantize(q, scale, zp, axis=-1):
    q = _c(q, np.int32)
    outer, ch, inner = _axis_view(q.shape, axis)
    s, z, pc = _per_channel_arrays(scale, zp, ch)
    x = np.empty(q.shape, np.float32)
    _check(_load().iqo_dequantize(_ptr(q), _ptr(x), outer, ch, inner, _ptr(s), _ptr(z), pc),
           "dequantize")
    return x


def pack(q, qtype):
    """Codes -> bytes; 4-bit types halve the last axis."""
    q = _c(q, np.int32)
    if qtype in (INT4, UINT4):
        shape = q.shape[:-1] + (q.shape[-1] // 2,)
    else:
        shape = q.shape
    out = np.empty(shape, np.uint8)
    _check(_load().iqo_pack(_ptr(q), _ptr(out), q.size, qtype), "pack")
    return out


def unpack(b, qtype):
    b = _c(b, np.uint8)
    if qtype in (INT4, UINT4):
        shape = b.shape[:-1] + (b.shape[-1] * 2,)
    else:
        shape = b.shape
    q = np.empty(shape, np.int32)
    _check(_load().iqo_unpack(_ptr(b), _ptr(q), q.size, qtype), "unpack")
    return q


def requant_multiplier(s_in, s_w, s_out):
    """M[c] = (S_in * S_w[c]) / S_out in binary32."""
    lib = _load()
    s_w = np.atleast_1d(np.asarray(s_w, np.float32))
    return np.array([lib.iqo_requant_multiplier(float(np.float32(s_in)), float(v), float(np.float32(s_out)))
                     for v in s_w], dtype=np.float32)


def residual_multiplier(s_res, s_out):
    return np.float32(_load().iqo_residual_multiplier(float(np.float32(s_res)), float(np.float32(s_out))))


def quantize_bias(b, s_in, s_w):
    """bias_q[c] = rne(B[c] / (S_in * S_w[c])) as int32."""
    lib = _load()
    b = np.atleast_1d(np.asarray(b, np.float32))
    s_w = np.broadcast_to(np.atleast_1d(np.asarray(s_w, np.float32)), b.shape)
    out = np.empty(b.shape, np.int32)
    for i in range(b.size):
        v = ctypes.c_int32()
        _check(lib.iqo_quantize_bias(float(b[i]), float(np.float32(s_in)), float(s_w[i]), ctypes.byref(v)),
               "quantize_bias")
        out[i] = v.value
    return out


def conv_out_hw(h, w, kh, kw, stride, pad):
    sh, sw = (stride, stride) if np.isscalar(stride) else stride
    ph, pw = (pad, pad) if np.isscalar(pad) else pad
    return (h + 2 * ph - kh) // sh + 1, (w + 2 * pw - kw) // sw + 1


def conv2d_acc(x, z_in, w, z_w=0, stride=1, pad=0, bias_q=None):
    """Direct-conv accumulator, NHWC x [n,h,w,ci], OHWI w [co,kh,kw,ci] -> int64 [n,oh,ow,co]."""
    x = _c(x, np.int32)
    w = _c(w, np.int32)
    n, h, wd, ci = x.shape
    co, kh, kw, ci2 = w.shape
    assert ci == ci2
    sh, sw = (stride, stride) if np.isscalar(stride) else stride
    ph, pw = (pad, pad) if np.isscalar(pad) else pad
    oh, ow = conv_out_hw(h, wd, kh, kw, (sh, sw), (ph, pw))
    acc = np.empty((n, oh, ow, co), np.int64)
    b = _c(bias_q, np.int32) if bias_q is not None else None
    _check(_load().iqo_conv2d_acc(_ptr(x), n, h, wd, ci, int(z_in), _ptr(w), co, kh, kw, int(z_w),
                                  sh, sw, ph, pw, _ptr(b), _ptr(acc)), "conv2d_acc")
    return acc


def gemm_acc(a, z_a, b, z_b=0, bias_q=None):
    """acc[m,n] = bias_q[n] + sum_k (a[m,k]-z_a)(b[n,k]-z_b) as int64."""
    a = _c(a, np.int32)
    b = _c(b, np.int32)
    m, k = a.shape
    n, k2 = b.shape
    assert k == k2
    acc = np.empty((m, n), np.int64)
    bq = _c(bias_q, np.int32) if bias_q is not None else None
    _check(_load().iqo_gemm_acc(_ptr(a), m, k, int(z_a), _ptr(b), n, int(z_b), _ptr(bq), _ptr(acc)),
           "gemm_acc")
    return acc


def requant(acc, mult, epi, z_out, out_qtype, res=None, z_res=0, m_res=0.0):
    """Fused epilogue over acc [..., ch]; mult [ch] (or scalar)."""
    acc = _c(acc, np.int64)
    ch = acc.shape[-1]
    mult = _c(np.broadcast_to(np.asarray(mult, np.float32), (ch,)), np.float32)
    r = _c(res, np.int32) if res is not None else None
    if r is not None:
        assert r.shape == acc.shape
    out = np.empty(acc.shape, np.int32)
    _check(_load().iqo_requant(_ptr(acc), acc.size // ch, ch, _ptr(mult), epi, _ptr(r), int(z_res),
                               float(np.float32(m_res)), int(z_out), out_qtype, _ptr(out)), "requant")
    return out


# ---------------------------------------------------------------------------
# Integer-only requantization: the multiplier M[c] as an integer mantissa and a
# power-of-two shift, for targets without floating point ("Quantization" blog,
# 量化模式: integer quantization replaces float arithmetic by a power-of-two
# scale; FQ-ViT article, section 2 / LayerNorm code: get_MN).


def get_mn(x, bit=8):
    """(M, N) with x ~ M * 2^-N: N = clamp(bit - 1 - floor(log2 x), 0, 31),
    M = clamp(floor(x * 2^N), 0, 2^bit - 1) (FQ-ViT's get_MN).  floor(log2 x) is the
    exact binary exponent of the binary32 value x (frexp), not a rounded log."""
    import math
    x = float(np.float32(x))
    assert x > 0.0
    mant, e = math.frexp(x)           # x = mant * 2^e, mant in [0.5, 1)
    n = min(max(bit - 1 - (e - 1), 0), 31)
    m = min(max(math.floor(math.ldexp(x, n)), 0), (1 << bit) - 1)
    return int(m), int(n)


def requant_int(acc, m, n, epi, z_out, out_qtype):
    """y = clip(rne(acc * M[c] / 2^N[c]) + Z_out) with ReLU as the clamp at Z_out
    (passive); acc [..., ch] int64, m / n [ch].  rne = round half to even (the blog's
    round_fn).  Epilogues NONE and RELU only."""
    assert epi in (EPI_NONE, EPI_RELU)
    acc = np.asarray(acc, np.int64)
    ch = acc.shape[-1]
    m = np.broadcast_to(np.asarray(m, np.int64), (ch,))
    n = np.broadcast_to(np.asarray(n, np.int64), (ch,))
    t = acc * m                                   # |t| < 2^62 for |acc| < 2^31, M < 2^31
    q = t.copy()
    for c in range(ch):
        if n[c] == 0:
            continue
        tc = t[..., c]
        q0 = tc >> n[c]                           # floor (arithmetic shift)
        rem = tc - (q0 << n[c])                   # in [0, 2^N)
        half = np.int64(1) << (n[c] - 1)
        up = (rem > half) | ((rem == half) & ((q0 & 1) == 1))
        q[..., c] = q0 + up.astype(np.int64)
    lo, hi = qrange(out_qtype)
    if epi == EPI_RELU:
        q = np.maximum(q, 0)
    return np.clip(q + z_out, lo, hi).astype(np.int32)


def maxpool2d(x, k, stride, pad):
    x = _c(x, np.int32)
    n, h, w, c = x.shape
    oh, ow = conv_out_hw(h, w, k, k, stride, pad)
    y = np.empty((n, oh, ow, c), np.int32)
    _check(_load().iqo_maxpool2d(_ptr(x), n, h, w, c, k, stride, pad, _ptr(y)), "maxpool2d")
    return y


def im2col(x, z_in, kh, kw, stride=1, pad=0):
    x = _c(x, np.int32)
    n, h, w, ci = x.shape
    sh, sw = (stride, stride) if np.isscalar(stride) else stride
    ph, pw = (pad, pad) if np.isscalar(pad) else pad
    oh, ow = conv_out_hw(h, w, kh, kw, (sh, sw), (ph, pw))
    cols = np.empty((n * oh * ow, kh * kw * ci), np.int32)
    _check(_load().iqo_im2col(_ptr(x), n, h, w, ci, int(z_in), kh, kw, sh, sw, ph, pw, _ptr(cols)), "im2col")
    return cols


# ---------------------------------------------------------------------------
# Whole operators, composed from the steps above in the pages' order.


def qconv(x, z_in, s_in, w, s_w, bias, s_out, z_out, out_qtype, epi, stride=1, pad=0,
          res=None, s_res=1.0, z_res=0, z_w=0):
    """Quantized conv with fused epilogue: codes in, codes out (int32 acc for EPI_RAW).

    x: NHWC input codes; w: OHWI weight codes with per-tensor zero point z_w (0:
    symmetric); s_w: scalar or [co]; bias: float32 [co] or None; res: NHWC residual
    codes for ADD / ADD_RELU.  The accumulator is the plain definition
    sum (x - Z_in)(w - Z_w) (MegEngine 4-bit article, 緩解精度下降).
    """
    co = w.shape[0]
    s_w_c = np.broadcast_to(np.atleast_1d(np.asarray(s_w, np.float32)), (co,))
    bias_q = quantize_bias(bias, s_in, s_w_c) if bias is not None else None
    acc = conv2d_acc(x, z_in, w, z_w, stride, pad, bias_q)
    if epi == EPI_RAW:
        return requant(acc, np.ones(co, np.float32), EPI_RAW, 0, INT32)
    mult = requant_multiplier(s_in, s_w_c, s_out)
    m_res = residual_multiplier(s_res, s_out) if res is not None else 0.0
    return requant(acc, mult, epi, z_out, out_qtype, res, z_res, m_res)


def qgemm(a, z_a, s_a, b, s_b, bias, s_out, z_out, out_qtype, epi, res=None, s_res=1.0, z_res=0, z_b=0):
    """Quantized GEMM C = A B^T (B stored [n][k], zero point z_b) with fused epilogue."""
    n = b.shape[0]
    s_b_c = np.broadcast_to(np.atleast_1d(np.asarray(s_b, np.float32)), (n,))
    bias_q = quantize_bias(bias, s_a, s_b_c) if bias is not None else None
    acc = gemm_acc(a, z_a, b, z_b, bias_q)
    if epi == EPI_RAW:
        return requant(acc, np.ones(n, np.float32), EPI_RAW, 0, INT32)
    mult = requant_multiplier(s_a, s_b_c, s_out)
    m_res = residual_multiplier(s_res, s_out) if res is not None else 0.0
    return requant(acc, mult, epi, z_out, out_qtype, res, z_res, m_res)
