"""ctypes binding of libiqnn (include/iqnn.h): argument marshalling only.

Every function has the name of the C entry point it calls.  Device buffers are
passed as torch tensors (their data_ptr()) or raw integer addresses; host
buffers as numpy arrays.  `stream` defaults to torch's current stream on the
tensor's device.  A non-OK status raises IqnnError carrying the library's
message.  There is no fallback: if libiqnn.so is missing, every call raises.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# IQNN_LIB: another build of the library (the sanitized CPU-hygiene build, say)
LIB_PATH = os.environ.get("IQNN_LIB") or os.path.join(_HERE, "libiqnn.so")

INT8, UINT8, INT4, UINT4, INT32 = 0, 1, 2, 3, 4
INT8_2OF4 = 5          # weights only: 2:4-sparse symmetric int8 codes
EPI_NONE, EPI_RELU, EPI_ADD, EPI_ADD_RELU, EPI_RAW_INT32 = 0, 1, 2, 3, 4
EPI_INT_REQUANT = 16   # flag: integer-only requantization (with NONE or RELU)
STATUS = {0: "IQNN_OK", 1: "IQNN_ERR_INVALID_ARG", 2: "IQNN_ERR_UNSUPPORTED", 3: "IQNN_ERR_ALIGNMENT",
          4: "IQNN_ERR_OVERFLOW", 5: "IQNN_ERR_HIP"}


class IqnnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s: %s" % (STATUS.get(status, status), message))
        self.status = status


class ConvDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n", "h", "w", "c_in", "c_out", "kh", "kw", "stride_h", "stride_w", "pad_h", "pad_w",
        "x_type", "w_type", "y_type", "res_type", "epilogue", "z_in", "z_out", "z_res", "z_w")]

    def out_hw(self):
        return ((self.h + 2 * self.pad_h - self.kh) // self.stride_h + 1,
                (self.w + 2 * self.pad_w - self.kw) // self.stride_w + 1)


class KernelCfg(ctypes.Structure):
    """iqnn_kernel_cfg: tile (-1 automatic) and xcd_groups (0 automatic) of one call."""
    _fields_ = [("tile", ctypes.c_int32), ("xcd_groups", ctypes.c_int32)]


def kernel_cfg(tile=-1, xcd_groups=0):
    return KernelCfg(int(tile), int(xcd_groups))


class GemmDesc(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int64), ("n", ctypes.c_int64), ("k", ctypes.c_int64)] + \
               [(n, ctypes.c_int32) for n in ("a_type", "b_type", "c_type", "res_type", "epilogue",
                                              "z_a", "z_out", "z_res", "z_b")]


_lib = None


def lib():
    """The loaded libiqnn.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libiqnn.so not found at %s: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P, I, I32, I64, F, SZ = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int32, ctypes.c_int64,
                             ctypes.c_float, ctypes.c_size_t)
    CD, GD, KC = ctypes.POINTER(ConvDesc), ctypes.POINTER(GemmDesc), ctypes.POINTER(KernelCfg)
    sig = {
        "iqnn_abi_version": (I, []),
        "iqnn_status_str": (ctypes.c_char_p, [I]),
        "iqnn_last_error": (ctypes.c_char_p, []),
        "iqnn_choose_qparams": (I, [F, F, I32, I, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int32)]),
        "iqnn_quantize": (I, [P, P, I64, I64, I64, P, P, I, I32, P]),
        "iqnn_dequantize": (I, [P, P, I64, I64, I64, P, P, I, I32, P]),
        "iqnn_quantize_pad": (I, [P, P, I32, I32, I32, I32, I32, I32, P, P, I, I32, P]),
        "iqnn_qconv_packed_size": (SZ, [CD]),
        "iqnn_qconv_prepack": (I, [CD, P, P, F, P, I, F, F, P, SZ, P]),
        "iqnn_qconv_prepack_host": (I, [CD, P, P, F, P, I, F, F, P, SZ]),
        "iqnn_qconv_fwd": (I, [CD, P, P, P, P, P]),
        "iqnn_qconv_fwd_cfg": (I, [CD, P, P, P, P, KC, P]),
        "iqnn_qconv_maxpool_fwd": (I, [CD, P, P, P, I32, I32, I32, P]),
        "iqnn_qconv_pair_fwd": (I, [CD, CD, P, P, P, P, P, P, P]),
        "iqnn_qgemm_packed_size": (SZ, [GD]),
        "iqnn_qgemm_prepack": (I, [GD, P, P, F, P, I, F, F, P, SZ, P]),
        "iqnn_qgemm_prepack_host": (I, [GD, P, P, F, P, I, F, F, P, SZ]),
        "iqnn_qgemm_fwd": (I, [GD, P, P, P, P, P]),
        "iqnn_qgemm_fwd_cfg": (I, [GD, P, P, P, P, KC, P]),
        "iqnn_maxpool2d": (I, [P, P, I32, I32, I32, I32, I32, I32, I32, I32, P]),
        "iqnn_probe_empty": (I, [P]),
        "iqnn_probe_mfma_rate": (I, [I32, I32, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(status):
    if status != 0:
        raise IqnnError(status, lib().iqnn_last_error().decode())


def _dev(t):
    """Device address of a torch tensor (or an int address, or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    return ctypes.c_void_p(t.data_ptr())


def _host(a, dtype):
    if a is None:
        return None, None
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, ctypes.c_void_p(a.ctypes.data)


def _stream(stream, like=None):
    if stream is None:
        import torch
        dev = like.device if like is not None and hasattr(like, "device") else None
        return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def iqnn_abi_version():
    return lib().iqnn_abi_version()


def iqnn_choose_qparams(vmin, vmax, qtype, symmetric=False):
    """(scale, zero point) of a real range [vmin, vmax]: binary32 scale, int zero point."""
    s, z = ctypes.c_float(), ctypes.c_int32()
    _check(lib().iqnn_choose_qparams(float(vmin), float(vmax), int(qtype), int(bool(symmetric)),
                                     ctypes.byref(s), ctypes.byref(z)))
    return np.float32(s.value), int(z.value)


def iqnn_quantize(x, q, outer, ch, inner, scale, zp, per_channel, qtype, stream=None):
    _check(lib().iqnn_quantize(_dev(x), _dev(q), outer, ch, inner, _dev(scale), _dev(zp), int(per_channel),
                               qtype, _stream(stream, x)))


def iqnn_dequantize(q, x, outer, ch, inner, scale, zp, per_channel, qtype, stream=None):
    _check(lib().iqnn_dequantize(_dev(q), _dev(x), outer, ch, inner, _dev(scale), _dev(zp), int(per_channel),
                                 qtype, _stream(stream, x)))


def iqnn_quantize_pad(x, q, n, h, w, c, pad, c_pad, scale, zp, per_channel, qtype, stream=None):
    _check(lib().iqnn_quantize_pad(_dev(x), _dev(q), n, h, w, c, pad, c_pad, _dev(scale), _dev(zp), int(per_channel),
                                   qtype, _stream(stream, x)))


def iqnn_qconv_packed_size(desc):
    n = lib().iqnn_qconv_packed_size(ctypes.byref(desc))
    if n == 0:
        raise IqnnError(1, lib().iqnn_last_error().decode())
    return n


def iqnn_qconv_prepack(desc, w_host, bias_host, s_in, s_w_host, per_channel, s_out, s_res, packed, stream=None):
    w_arr, w_ptr = _host(w_host, np.uint8)
    b_arr, b_ptr = _host(bias_host, np.float32)
    s_arr, s_ptr = _host(np.atleast_1d(np.asarray(s_w_host, np.float32)), np.float32)
    _check(lib().iqnn_qconv_prepack(ctypes.byref(desc), w_ptr, b_ptr, float(s_in), s_ptr, int(per_channel),
                                    float(s_out), float(s_res), _dev(packed), packed.numel() * packed.element_size(),
                                    _stream(stream, packed)))


def iqnn_qconv_prepack_host(desc, w_host, bias_host, s_in, s_w_host, per_channel, s_out, s_res, packed_host):
    """Host prepack into a numpy uint8 array of iqnn_qconv_packed_size bytes."""
    w_arr, w_ptr = _host(w_host, np.uint8)
    b_arr, b_ptr = _host(bias_host, np.float32)
    s_arr, s_ptr = _host(np.atleast_1d(np.asarray(s_w_host, np.float32)), np.float32)
    assert packed_host.dtype == np.uint8 and packed_host.flags.c_contiguous
    _check(lib().iqnn_qconv_prepack_host(ctypes.byref(desc), w_ptr, b_ptr, float(s_in), s_ptr, int(per_channel),
                                         float(s_out), float(s_res), ctypes.c_void_p(packed_host.ctypes.data),
                                         packed_host.nbytes))


def iqnn_qconv_fwd(desc, x, packed, res, y, stream=None):
    _check(lib().iqnn_qconv_fwd(ctypes.byref(desc), _dev(x), _dev(packed), _dev(res), _dev(y), _stream(stream, y)))


def iqnn_qconv_fwd_cfg(desc, x, packed, res, y, cfg, stream=None):
    """cfg: a KernelCfg, a (tile, xcd_groups) pair, or None (automatic)."""
    _check(lib().iqnn_qconv_fwd_cfg(ctypes.byref(desc), _dev(x), _dev(packed), _dev(res), _dev(y), _cfg(cfg),
                                    _stream(stream, y)))


def _cfg(cfg):
    if cfg is None:
        return None
    if not isinstance(cfg, KernelCfg):
        cfg = KernelCfg(*(int(v) for v in cfg))
    return ctypes.byref(cfg)


def iqnn_qconv_maxpool_fwd(desc, x, packed, y, pool_k, pool_stride, pool_pad, stream=None):
    _check(lib().iqnn_qconv_maxpool_fwd(ctypes.byref(desc), _dev(x), _dev(packed), _dev(y), pool_k, pool_stride,
                                        pool_pad, _stream(stream, y)))


def iqnn_qconv_pair_fwd(desc_a, desc_b, x, packed_a, res, packed_b, y_a, y_b, stream=None):
    _check(lib().iqnn_qconv_pair_fwd(ctypes.byref(desc_a), ctypes.byref(desc_b), _dev(x), _dev(packed_a), _dev(res),
                                     _dev(packed_b), _dev(y_a), _dev(y_b), _stream(stream, y_b)))


def iqnn_qgemm_packed_size(desc):
    n = lib().iqnn_qgemm_packed_size(ctypes.byref(desc))
    if n == 0:
        raise IqnnError(1, lib().iqnn_last_error().decode())
    return n


def iqnn_qgemm_prepack(desc, b_host, bias_host, s_a, s_b_host, per_channel, s_out, s_res, packed, stream=None):
    b_arr, b_ptr = _host(b_host, np.uint8)
    bias_arr, bias_ptr = _host(bias_host, np.float32)
    s_arr, s_ptr = _host(np.atleast_1d(np.asarray(s_b_host, np.float32)), np.float32)
    _check(lib().iqnn_qgemm_prepack(ctypes.byref(desc), b_ptr, bias_ptr, float(s_a), s_ptr, int(per_channel),
                                    float(s_out), float(s_res), _dev(packed), packed.numel() * packed.element_size(),
                                    _stream(stream, packed)))


def iqnn_qgemm_prepack_host(desc, b_host, bias_host, s_a, s_b_host, per_channel, s_out, s_res, packed_host):
    b_arr, b_ptr = _host(b_host, np.uint8)
    bias_arr, bias_ptr = _host(bias_host, np.float32)
    s_arr, s_ptr = _host(np.atleast_1d(np.asarray(s_b_host, np.float32)), np.float32)
    assert packed_host.dtype == np.uint8 and packed_host.flags.c_contiguous
    _check(lib().iqnn_qgemm_prepack_host(ctypes.byref(desc), b_ptr, bias_ptr, float(s_a), s_ptr, int(per_channel),
                                         float(s_out), float(s_res), ctypes.c_void_p(packed_host.ctypes.data),
                                         packed_host.nbytes))


def iqnn_qgemm_fwd(desc, a, packed, res, c, stream=None):
    _check(lib().iqnn_qgemm_fwd(ctypes.byref(desc), _dev(a), _dev(packed), _dev(res), _dev(c), _stream(stream, c)))


def iqnn_qgemm_fwd_cfg(desc, a, packed, res, c, cfg, stream=None):
    _check(lib().iqnn_qgemm_fwd_cfg(ctypes.byref(desc), _dev(a), _dev(packed), _dev(res), _dev(c), _cfg(cfg),
                                    _stream(stream, c)))


def iqnn_probe_empty(stream=None):
    _check(lib().iqnn_probe_empty(_stream(stream)))


def iqnn_probe_mfma_rate(iters, blocks, sink, stream=None):
    _check(lib().iqnn_probe_mfma_rate(int(iters), int(blocks), _dev(sink), _stream(stream, sink)))


def iqnn_maxpool2d(x, y, n, h, w, c, k, stride, pad, dtype, stream=None):
    _check(lib().iqnn_maxpool2d(_dev(x), _dev(y), n, h, w, c, k, stride, pad, dtype, _stream(stream, y)))
