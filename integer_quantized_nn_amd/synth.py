"""Seeded synthetic workloads: float tensors and quantization parameters.

This module is the one thing the tests, the benchmark and the CPU oracle's
callers share.  It holds none of the quantized method's arithmetic: it draws
float activations, weights, biases and residuals from numpy's PCG64 generator
(draws in a fixed order per case), and picks scales and zero points with the
max / min-max calibration rule the pages describe for real ranges (Horizon QAT
talk, section 三: a fixed scale from the real min/max divided by the integer
range; FQ-ViT article, section 3.1: MinMax uniform quantization for Conv /
Linear / MatMul).  Output scales are calibrated on the float (unquantized)
operator over a calibration slice (batch element 0, or the first 197 rows of a
GEMM).  Turning floats into codes is left to the caller: the oracle's quantize
in the tests, the library's iqnn_quantize in the benchmark.

Workloads (shapes and distributions):
  gemm_int8_256      256x256x256, codes drawn uniformly over [-128, 127]
  conv3x3_int8       ResNet 3x3 conv, N=32 56x56 64->64, uint8 half-normal input
  conv3x3_4bit       N=64 28x28 128->128 uint4 input, int4 weights, uint4 residual
  vitl_fc1           ViT-L MLP fc1 as a GEMM, 12608x1024 -> 4096, outlier channels
  resnet50_trunk     the 53 convolutions of ResNet-50 at batch 256 (plus max pooling)
"""
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

INT8, UINT8, INT4, UINT4, INT32 = 0, 1, 2, 3, 4
EPI_NONE, EPI_RELU, EPI_ADD, EPI_ADD_RELU, EPI_RAW = 0, 1, 2, 3, 4
_QMAX = {INT8: 127, UINT8: 255, INT4: 7, UINT4: 15}


def f32(v):
    return np.float32(v)


def sym_scales(w, axis=0, qtype=INT8):
    """Per-output-channel symmetric scale amax / Q_MAX (weights)."""
    amax = np.abs(w).reshape(w.shape[axis], -1).max(1).astype(np.float64)
    amax = np.maximum(amax, 1e-8)
    return (amax / _QMAX[qtype]).astype(np.float32)


def relu_scale(vmax, z, qtype):
    """Asymmetric scale for a non-negative tensor: max / (Q_MAX - Z)."""
    return f32(max(float(vmax), 1e-6) / (_QMAX[qtype] - z))


def minmax_qparams(vmin, vmax, qtype=UINT8):
    """Asymmetric min-max parameters: S = (max - min) / (Q_MAX - Q_MIN), Z from -min / S."""
    vmin, vmax = min(float(vmin), 0.0), max(float(vmax), 0.0)
    s = max(vmax - vmin, 1e-6) / _QMAX[qtype]
    z = int(np.clip(np.rint(-vmin / s), 0, _QMAX[qtype]))
    return f32(s), z


@dataclass
class ConvCase:
    """One quantized conv layer: float tensors plus every quantization parameter."""
    name: str
    x: Optional[np.ndarray]         # NHWC float input (None inside a trunk: it comes from the previous layer)
    w: np.ndarray                   # OHWI float weights
    bias: np.ndarray                # [C_out] float32
    s_in: np.float32
    z_in: int
    s_w: np.ndarray                 # [C_out] float32
    s_out: np.float32
    z_out: int
    x_type: int
    w_type: int
    y_type: int
    epi: int
    stride: int
    pad: int
    res: Optional[np.ndarray] = None  # float residual (standalone 4-bit case)
    s_res: np.float32 = f32(1.0)
    z_res: int = 0
    res_type: int = UINT8

    @property
    def c_out(self):
        return self.w.shape[0]

    def ops(self, n, h, w):
        co, kh, kw, ci = self.w.shape
        oh = (h + 2 * self.pad - kh) // self.stride + 1
        ow = (w + 2 * self.pad - kw) // self.stride + 1
        return 2 * n * oh * ow * co * kh * kw * ci


@dataclass
class GemmCase:
    name: str
    a: Optional[np.ndarray]         # float [M][K] (None when codes are drawn directly)
    a_codes: Optional[np.ndarray]   # int codes [M][K] (config drawn as codes)
    b: Optional[np.ndarray]         # float [N][K]
    b_codes: Optional[np.ndarray]
    bias: Optional[np.ndarray]
    s_a: np.float32
    z_a: int
    s_b: np.ndarray
    s_out: np.float32
    z_out: int
    a_type: int
    b_type: int
    c_type: int
    epi: int

    @property
    def shape(self):
        src_a = self.a if self.a is not None else self.a_codes
        src_b = self.b if self.b is not None else self.b_codes
        return src_a.shape[0], src_b.shape[0], src_a.shape[1]


def _float_conv(x_nhwc, w_ohwi, bias, stride, pad):
    """Float32 reference conv (NHWC) used only to calibrate output scales."""
    import torch
    import torch.nn.functional as F
    xt = torch.from_numpy(np.ascontiguousarray(x_nhwc, np.float32)).permute(0, 3, 1, 2)
    wt = torch.from_numpy(np.ascontiguousarray(w_ohwi, np.float32)).permute(0, 3, 1, 2)
    y = F.conv2d(xt, wt, torch.from_numpy(bias.astype(np.float32)), stride=stride, padding=pad)
    return y.permute(0, 2, 3, 1).numpy()


# ------------------------------------------------------------------ workloads


def gemm_int8_256(seed=0, m=256, n=256, k=256):
    """256^3 int8 symmetric GEMM: codes uniform on [-128, 127]; S_A 0.02, S_B 0.01, S_out 0.5."""
    rng = np.random.default_rng(seed)
    a = rng.integers(-128, 128, size=(m, k), dtype=np.int64).astype(np.int32)
    b = rng.integers(-128, 128, size=(n, k), dtype=np.int64).astype(np.int32)
    return GemmCase("gemm_int8_256", None, a, None, b, None, f32(0.02), 0, np.full(n, 0.01, np.float32),
                    f32(0.5), 0, INT8, INT8, INT8, EPI_NONE)


def conv_case(seed, n, h, w, c_in, c_out, k, stride, pad, x_type=UINT8, w_type=INT8, y_type=UINT8,
              epi=EPI_RELU, w_sigma=0.05, bias_sigma=0.1, res_type=UINT4, name="conv"):
    """A standalone conv layer with half-normal (post-ReLU-like) input.

    Draw order: input, weights, bias, input zero point, output zero point,
    then (ADD epilogues) the residual and its zero point.
    """
    rng = np.random.default_rng(seed)
    x = np.abs(rng.standard_normal((n, h, w, c_in), dtype=np.float32))
    wt = (rng.standard_normal((c_out, k, k, c_in), dtype=np.float32) * np.float32(w_sigma))
    bias = (rng.standard_normal(c_out, dtype=np.float32) * np.float32(bias_sigma))
    zmax_in = 16 if _QMAX[x_type] == 255 else 3
    z_in = int(rng.integers(0, zmax_in + 1)) if x_type in (UINT8, UINT4) else 0
    zmax_out = 16 if _QMAX.get(y_type, 0) == 255 else 3
    z_out = int(rng.integers(0, zmax_out + 1)) if y_type in (UINT8, UINT4) else 0
    s_in = relu_scale(x.max(), z_in, x_type) if x_type in (UINT8, UINT4) else f32(np.abs(x).max() / _QMAX[x_type])
    s_w = sym_scales(wt, 0, w_type)
    res = None
    s_res, z_res = f32(1.0), 0
    if epi in (EPI_ADD, EPI_ADD_RELU):
        res = np.abs(rng.standard_normal((n,) + _out_hw(h, w, k, stride, pad) + (c_out,), dtype=np.float32))
        z_res = int(rng.integers(0, (16 if _QMAX[res_type] == 255 else 3) + 1))
        s_res = relu_scale(res.max(), z_res, res_type)
    # output scale: max rule on the float operator, calibration slice = batch element 0
    y = _float_conv(x[:1], wt, bias, stride, pad)
    if res is not None:
        y = y + res[:1]
    if epi in (EPI_RELU, EPI_ADD_RELU):
        y = np.maximum(y, 0)
    if y_type in (UINT8, UINT4):
        if epi in (EPI_RELU, EPI_ADD_RELU):
            s_out = relu_scale(y.max(), z_out, y_type)
        else:
            s_out, z_out = minmax_qparams(y.min(), y.max(), y_type)
    elif y_type in (INT8, INT4):
        s_out = f32(max(float(np.abs(y).max()), 1e-6) / _QMAX[y_type])
    else:
        s_out = f32(1.0)
    return ConvCase(name, x, wt, bias, s_in, z_in, s_w, s_out, z_out, x_type, w_type, y_type, epi, stride, pad,
                    res, s_res, z_res, res_type)


def _out_hw(h, w, k, stride, pad):
    return (h + 2 * pad - k) // stride + 1, (w + 2 * pad - k) // stride + 1


def conv3x3_int8(seed=0, n=32, hw=56, c=64):
    """ResNet-50-style 3x3 conv: uint8 asymmetric half-normal input (Z in [0,16]), int8
    per-channel weights N(0, 0.05), fp32 bias folded to int32, Conv_Relu to uint8."""
    return conv_case(seed, n, hw, hw, c, c, 3, 1, 1, UINT8, INT8, UINT8, EPI_RELU, name="conv3x3_int8")


def conv3x3_4bit(seed=0, n=64, hw=28, c=128):
    """4-bit conv: UINT4 input/output/residual (Z in [0,3]), INT4 per-channel weights,
    fp32 bias, Conv_Add_Relu with a uint4 residual of the output's shape."""
    return conv_case(seed, n, hw, hw, c, c, 3, 1, 1, UINT4, INT4, UINT4, EPI_ADD_RELU, res_type=UINT4,
                     name="conv3x3_4bit")


def prune_2of4(w):
    """Magnitude pruning to 2:4 structured sparsity along the last axis: in every group
    of four consecutive entries the two of largest |w| are kept (the earlier one on a
    tie), the other two set to 0.  The last axis must be a multiple of 4."""
    g = w.reshape(-1, 4)
    order = np.argsort(-np.abs(g), axis=1, kind="stable")
    keep = np.zeros(g.shape, bool)
    np.put_along_axis(keep, order[:, :2], True, axis=1)
    return np.where(keep, g, np.float32(0)).reshape(w.shape).astype(w.dtype)


def vitl_fc1(seed=0, m=64 * 197, k=1024, n=4096, outlier_frac=0.02, outlier_max=40.0, sparse_2of4=False):
    """ViT-L MLP fc1 as a GEMM: N(0,1) activations with 2% of channels scaled by U[1,40]
    (the FQ-ViT article's inter-channel range observation), uint8 per-tensor min-max;
    int8 per-channel weights N(0, 0.02); per-channel requant to int8, no activation.
    sparse_2of4: the float weights magnitude-pruned to 2:4 along K before quantization."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((m, k), dtype=np.float32)
    n_out = int(round(outlier_frac * k))
    ch = rng.choice(k, size=n_out, replace=False)
    a[:, ch] *= rng.uniform(1.0, outlier_max, size=n_out).astype(np.float32)
    b = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    if sparse_2of4:
        b = prune_2of4(b)
    bias = rng.standard_normal(n, dtype=np.float32) * np.float32(0.1)
    s_a, z_a = minmax_qparams(a.min(), a.max(), UINT8)
    s_b = sym_scales(b, 0, INT8)
    cal = a[:197].astype(np.float64) @ b.astype(np.float64).T + bias
    s_out = f32(float(np.abs(cal).max()) / 127)
    return GemmCase("vitl_fc1_2of4" if sparse_2of4 else "vitl_fc1", a, None, b, None, bias, s_a, z_a, s_b, s_out, 0,
                    UINT8, INT8, INT8, EPI_NONE)


# ------------------------------------------------------------ ResNet-50 trunk


@dataclass
class TrunkLayer:
    name: str
    case: ConvCase
    src: str                 # name of the tensor this layer reads
    res_src: Optional[str]   # residual tensor for Conv_Add_Relu
    in_hw: tuple
    out: str                 # name of the tensor it writes


@dataclass
class Trunk:
    batch: int
    x: np.ndarray            # float input NHWC [batch, 224, 224, 3]
    s_in: np.float32
    z_in: int
    layers: List[TrunkLayer] = field(default_factory=list)
    pool_after: str = "stem"
    qparams: dict = field(default_factory=dict)   # tensor name -> (scale, zero point)

    def ops(self):
        return sum(l.case.ops(self.batch, *l.in_hw) for l in self.layers)


def resnet50_trunk(seed=0, batch=256, hw=224, calib_images=1, sparse_2of4=False):
    """The 53 convolutions of ResNet-50 (bottleneck stages 3-4-6-3, stride on the 3x3
    conv, 1x1 stride-s downsample without ReLU), random He-normal weights, uint8
    activations and int8 per-channel weights.

    Output scales come from a float forward of the unquantized trunk over the first
    `calib_images` images (max rule; min-max for the downsample outputs).
    sparse_2of4: the float weights of every conv after the stem are magnitude-pruned
    to 2:4 along the input channels as they are drawn (before calibration)."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((batch, hw, hw, 3), dtype=np.float32)
    s_in, z_in = minmax_qparams(x.min(), x.max(), UINT8)
    tr = Trunk(batch, x, s_in, z_in)
    tr.qparams["input"] = (s_in, z_in)

    specs = []   # (name, src, res_src, c_in, c_out, k, stride, pad, epi, out)
    specs.append(("stem", "input", None, 3, 64, 7, 2, 3, EPI_RELU, "stem"))
    cur, c_cur = "pool", 64
    for si, (blocks, width, stride) in enumerate([(3, 64, 1), (4, 128, 2), (6, 256, 2), (3, 512, 2)]):
        out_c = width * 4
        for bi in range(blocks):
            s = stride if bi == 0 else 1
            pre = "l%d.%d" % (si + 1, bi)
            if bi == 0:
                specs.append((pre + ".down", cur, None, c_cur, out_c, 1, s, 0, EPI_NONE, pre + ".down"))
                shortcut = pre + ".down"
            else:
                shortcut = cur
            specs.append((pre + ".c1", cur, None, c_cur, width, 1, 1, 0, EPI_RELU, pre + ".c1"))
            specs.append((pre + ".c2", pre + ".c1", None, width, width, 3, s, 1, EPI_RELU, pre + ".c2"))
            specs.append((pre + ".c3", pre + ".c2", shortcut, width, out_c, 1, 1, 0, EPI_ADD_RELU, pre + ".out"))
            cur, c_cur = pre + ".out", out_c

    # weights and biases in layer order, then zero points in layer order
    params = []
    for (name, src, res_src, ci, co, k, st, pd, epi, out) in specs:
        fan_in = k * k * ci
        sigma = np.float32(np.sqrt(2.0 / fan_in))
        w = rng.standard_normal((co, k, k, ci), dtype=np.float32) * sigma
        b = rng.standard_normal(co, dtype=np.float32) * np.float32(0.1) * sigma
        if sparse_2of4 and name != "stem":
            w = prune_2of4(w)
        params.append((w, b))
    zps = [int(rng.integers(0, 17)) for _ in specs]

    # float calibration forward over the calibration images
    act = {"input": torch.from_numpy(x[:calib_images]).permute(0, 3, 1, 2)}
    hw_of = {"input": (hw, hw)}
    for (spec, (w, b), z) in zip(specs, params, zps):
        name, src, res_src, ci, co, k, st, pd, epi, out = spec
        xin = act[src]
        y = F.conv2d(xin, torch.from_numpy(w).permute(0, 3, 1, 2), torch.from_numpy(b), stride=st, padding=pd)
        if res_src is not None:
            y = y + act[res_src]
        if epi in (EPI_RELU, EPI_ADD_RELU):
            y = torch.relu(y)
            s_out, z_out = relu_scale(float(y.max()), z, UINT8), z
        else:
            s_out, z_out = minmax_qparams(float(y.min()), float(y.max()), UINT8)
        act[out] = y
        hw_of[out] = (y.shape[2], y.shape[3])
        if name == "stem":
            act["pool"] = F.max_pool2d(y, 3, 2, 1)
            hw_of["pool"] = (act["pool"].shape[2], act["pool"].shape[3])
            tr.qparams["pool"] = (s_out, z_out)   # max pooling is passive
        s_src, z_src = tr.qparams[src]
        s_res, z_res = tr.qparams[res_src] if res_src is not None else (f32(1.0), 0)
        case = ConvCase(name, None, w, b, s_src, z_src, sym_scales(w, 0, INT8), s_out, z_out, UINT8, INT8, UINT8,
                        epi, st, pd, None, s_res, z_res, UINT8)
        tr.qparams[out] = (s_out, z_out)
        tr.layers.append(TrunkLayer(name, case, src, res_src, hw_of[src], out))
    return tr
