"""Layer objects over the C ABI: torch supplies device memory and streams, every
step runs in libiqnn's kernels.

  QConv / QGemm   prepack a layer once (iqnn_*_prepack), then run it (iqnn_*_fwd)
  quantize / dequantize / maxpool2d   allocate the output and call the kernel
"""
import numpy as np
import torch

from . import binding as B


def code_bytes(shape, qtype):
    """Byte shape of a code tensor: 4-bit types pack pairs along the last axis."""
    shape = tuple(int(s) for s in shape)
    if qtype in (B.INT4, B.UINT4):
        assert shape[-1] % 2 == 0, "4-bit tensors need an even innermost size"
        return shape[:-1] + (shape[-1] // 2,)
    if qtype == B.INT32:
        return shape[:-1] + (shape[-1] * 4,)
    return shape


def empty_codes(shape, qtype, device="cuda"):
    return torch.empty(code_bytes(shape, qtype), dtype=torch.uint8, device=device)


def _scalar_or_vec(v, dtype, device):
    return torch.as_tensor(np.atleast_1d(np.asarray(v)), dtype=dtype, device=device).contiguous()


def quantize(x, scale, zp, qtype, axis=-1, out=None, stream=None):
    """Codes of float tensor x (device); scale/zp scalars or per-channel along `axis`."""
    axis = axis % x.dim()
    outer = int(np.prod(x.shape[:axis], dtype=np.int64))
    ch = int(x.shape[axis])
    inner = int(np.prod(x.shape[axis + 1:], dtype=np.int64))
    s = scale if torch.is_tensor(scale) else _scalar_or_vec(scale, torch.float32, x.device)
    z = zp if torch.is_tensor(zp) else _scalar_or_vec(zp, torch.int32, x.device)
    per_channel = s.numel() > 1 or z.numel() > 1
    if per_channel and s.numel() == 1:
        s = s.expand(ch).contiguous()
    if per_channel and z.numel() == 1:
        z = z.expand(ch).contiguous()
    if out is None:
        out = empty_codes(x.shape, qtype, x.device)
    B.iqnn_quantize(x, out, outer, ch, inner, s, z, per_channel, qtype, stream)
    return out


def quantize_pad(x, scale, zp, qtype, pad, c_pad, out=None, stream=None):
    """Codes of NHWC float x with a border of `pad` pixels and channels padded to c_pad,
    all padding holding the zero-point code."""
    n, h, w, c = (int(v) for v in x.shape)
    s = scale if torch.is_tensor(scale) else _scalar_or_vec(scale, torch.float32, x.device)
    z = zp if torch.is_tensor(zp) else _scalar_or_vec(zp, torch.int32, x.device)
    per_channel = s.numel() > 1 or z.numel() > 1
    if out is None:
        out = torch.empty((n, h + 2 * pad, w + 2 * pad, c_pad), dtype=torch.uint8, device=x.device)
    B.iqnn_quantize_pad(x, out, n, h, w, c, pad, c_pad, s, z, per_channel, qtype, stream)
    return out


def dequantize(q, shape, scale, zp, qtype, axis=-1, out=None, stream=None):
    shape = tuple(shape)
    axis = axis % len(shape)
    outer = int(np.prod(shape[:axis], dtype=np.int64))
    ch = int(shape[axis])
    inner = int(np.prod(shape[axis + 1:], dtype=np.int64))
    s = scale if torch.is_tensor(scale) else _scalar_or_vec(scale, torch.float32, q.device)
    z = zp if torch.is_tensor(zp) else _scalar_or_vec(zp, torch.int32, q.device)
    per_channel = s.numel() > 1 or z.numel() > 1
    if per_channel and s.numel() == 1:
        s = s.expand(ch).contiguous()
    if per_channel and z.numel() == 1:
        z = z.expand(ch).contiguous()
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=q.device)
    B.iqnn_dequantize(q, out, outer, ch, inner, s, z, per_channel, qtype, stream)
    return out


def maxpool2d(x, n, h, w, c, k, stride, pad, dtype, out=None, stream=None):
    oh = (h + 2 * pad - k) // stride + 1
    ow = (w + 2 * pad - k) // stride + 1
    if out is None:
        out = torch.empty((n, oh, ow, c), dtype=torch.uint8, device=x.device)
    B.iqnn_maxpool2d(x, out, n, h, w, c, k, stride, pad, dtype, stream)
    return out


class QConv:
    """One prepacked quantized conv layer (NHWC, OHWI weights)."""

    def __init__(self, n, h, w, c_in, c_out, k, stride, pad, x_type, w_type, y_type, epi, z_in, z_out,
                 w_bytes, bias, s_in, s_w, s_out, res_type=B.UINT8, z_res=0, s_res=1.0, kw=None,
                 device="cuda", stream=None, z_w=0):
        kw = k if kw is None else kw
        d = B.ConvDesc()
        d.n, d.h, d.w, d.c_in, d.c_out = n, h, w, c_in, c_out
        d.kh, d.kw, d.stride_h, d.stride_w, d.pad_h, d.pad_w = k, kw, stride, stride, pad, pad
        d.x_type, d.w_type, d.y_type, d.res_type, d.epilogue = x_type, w_type, y_type, res_type, epi
        d.z_in, d.z_out, d.z_res, d.z_w = z_in, z_out, z_res, z_w
        self.desc = d
        self.out_shape = (n,) + d.out_hw() + (c_out,)
        s_w = np.atleast_1d(np.asarray(s_w, np.float32))
        self.packed = torch.empty(B.iqnn_qconv_packed_size(d), dtype=torch.uint8, device=device)
        B.iqnn_qconv_prepack(d, w_bytes, bias, s_in, s_w, s_w.size > 1, s_out, s_res, self.packed, stream)
        self.y_type = y_type

    def __call__(self, x, res=None, out=None, stream=None, cfg=None):
        """cfg: kernel configuration (tile, xcd_groups) of this call; None: automatic."""
        if out is None:
            out = empty_codes(self.out_shape, self.y_type, x.device)
        if cfg is None:
            B.iqnn_qconv_fwd(self.desc, x, self.packed, res, out, stream)
        else:
            B.iqnn_qconv_fwd_cfg(self.desc, x, self.packed, res, out, cfg, stream)
        return out

    def pool_shape(self, k=3, stride=2, pad=1):
        n, oh, ow, c = self.out_shape
        return (n, (oh + 2 * pad - k) // stride + 1, (ow + 2 * pad - k) // stride + 1, c)

    def conv_maxpool(self, x, k=3, stride=2, pad=1, out=None, stream=None):
        """maxpool(conv(x)) in one fused launch (iqnn_qconv_maxpool_fwd)."""
        if out is None:
            out = empty_codes(self.pool_shape(k, stride, pad), self.y_type, x.device)
        B.iqnn_qconv_maxpool_fwd(self.desc, x, self.packed, out, k, stride, pad, stream)
        return out


def conv_pair(conv_a, conv_b, x, res=None, out_a=None, out_b=None, stream=None):
    """y_a = conv_a(x, res) and y_b = conv_b(y_a) in one call (iqnn_qconv_pair_fwd):
    conv_b's input is conv_a's output.  Returns (y_a, y_b)."""
    if out_a is None:
        out_a = empty_codes(conv_a.out_shape, conv_a.y_type, x.device)
    if out_b is None:
        out_b = empty_codes(conv_b.out_shape, conv_b.y_type, x.device)
    B.iqnn_qconv_pair_fwd(conv_a.desc, conv_b.desc, x, conv_a.packed, res, conv_b.packed, out_a, out_b, stream)
    return out_a, out_b


class QGemm:
    """One prepacked quantized GEMM: C[M][N] = epilogue(A[M][K] B[N][K]^T)."""

    def __init__(self, m, n, k, a_type, b_type, c_type, epi, z_a, z_out, b_bytes, bias, s_a, s_b, s_out,
                 res_type=B.UINT8, z_res=0, s_res=1.0, device="cuda", stream=None, z_b=0):
        d = B.GemmDesc()
        d.m, d.n, d.k = m, n, k
        d.a_type, d.b_type, d.c_type, d.res_type, d.epilogue = a_type, b_type, c_type, res_type, epi
        d.z_a, d.z_out, d.z_res, d.z_b = z_a, z_out, z_res, z_b
        self.desc = d
        self.out_shape = (m, n)
        s_b = np.atleast_1d(np.asarray(s_b, np.float32))
        self.packed = torch.empty(B.iqnn_qgemm_packed_size(d), dtype=torch.uint8, device=device)
        B.iqnn_qgemm_prepack(d, b_bytes, bias, s_a, s_b, s_b.size > 1, s_out, s_res, self.packed, stream)
        self.c_type = c_type

    def __call__(self, a, res=None, out=None, stream=None, cfg=None):
        if out is None:
            out = empty_codes(self.out_shape, self.c_type, a.device)
        if cfg is None:
            B.iqnn_qgemm_fwd(self.desc, a, self.packed, res, out, stream)
        else:
            B.iqnn_qgemm_fwd_cfg(self.desc, a, self.packed, res, out, cfg, stream)
        return out
