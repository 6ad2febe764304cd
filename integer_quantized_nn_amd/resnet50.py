"""ResNet-50 convolution trunk on libiqnn: every layer a fused quantized conv.

The schedule follows the fused ResNet-50 graph of the MegEngine 4-bit article
(section 算子融合優化, Fig. 3 and 4): Conv_Relu for the stem and the first two
convs of each bottleneck, Conv_Add_Relu for the third (the residual add and ReLU
absorbed into the conv), a plain Conv for the stride-s 1x1 downsample of each
stage's first block, and a passive max pooling after the stem ("Quantization"
blog, 量化激活函数).  One forward step is: quantize the fp32 input, 53 convs and
one max pooling on one stream, dequantize the final output.  Every activation
tensor keeps its own HBM buffer (the trunk needs a few GB at batch 256).  Where a
64-channel block ends, its last conv and the next block's first conv are one launch
(iqnn_qconv_pair_fwd): the block output is written once and read by the second conv
from LDS, so 50 launches carry the 53 convs.

Activations are uint8 codes with a per-tensor zero point (the article's asymmetric
activation quantization).  With offset_codes the trunk stores every such code q as the
int8 byte q - 128 with zero point Z - 128: the same real values, the same q - Z in every
contraction, the same rounding decisions (rne(t) + Z and the clip bounds shift by the
same 128), so every buffer holds the uint8 trunk's bytes XOR 0x80.  The kernels then
take the activation bytes as signed MFMA operands directly instead of flipping the sign
bit of every fragment.
"""
import numpy as np
import torch

from . import binding as B
from .layers import QConv, conv_pair, dequantize, empty_codes, maxpool2d, quantize, quantize_pad

STEM_PAD_CHANNELS = 4


def _pair_first(layer):
    """The last conv of a 64-channel bottleneck block: 1x1, 64 -> 256, residual add."""
    c = layer.case
    return c.w.shape == (256, 1, 1, 64) and c.stride == 1 and c.pad == 0 and layer.res_src is not None


def _pair_second(layer):
    """A block's first conv reading 256 channels: 1x1, 256 -> 64 or 128, no residual."""
    c = layer.case
    return c.w.shape[1:] == (1, 1, 256) and c.w.shape[0] in (64, 128) and c.stride == 1 and c.pad == 0 and \
        layer.res_src is None


class QuantResNet50Trunk:
    """The trunk's 3-channel image enters through iqnn_quantize_pad: the stem's zero
    padding (3 pixels) and a 4th channel are written as the input zero-point code, so
    the stem runs as a padding-free 4-channel conv whose loads take 4 taps x 4
    channels at a time.  A zero weight on the extra channel and the real-0 border make
    it the same convolution as the 3-channel padded one."""

    def __init__(self, trunk, device="cuda", weight_codes=None, stream=None, fuse_stem_pool=True,
                 offset_codes=False, sparse_2of4=False, fuse_pairs=True):
        """trunk: synth.Trunk.  weight_codes: optional {layer name: OHWI int8 bytes};
        by default the float weights are quantized per output channel on the GPU.
        fuse_stem_pool: run the stem and the max pooling as one launch
        (iqnn_qconv_maxpool_fwd), never writing the stem's output.  offset_codes:
        store the uint8 activation codes as int8 bytes q - 128 (zero points Z - 128).
        sparse_2of4: run the convs after the stem with their weights as 2:4-sparse
        codes (IQNN_INT8_2OF4; the trunk's weights must be 2:4, as drawn by
        synth.resnet50_trunk(sparse_2of4=True)).  fuse_pairs: launch the last conv of
        each 64-channel block together with the next block's first conv
        (iqnn_qconv_pair_fwd), which then reads the block output from LDS instead of
        HBM (dense weights only)."""
        self.trunk = trunk
        self.fuse_stem_pool = fuse_stem_pool
        self.offset_codes = offset_codes
        act, off = (B.INT8, 128) if offset_codes else (B.UINT8, 0)
        self.act_type = act
        self.device = device
        n = trunk.batch
        self.convs = {}
        stem = trunk.layers[0]
        self.stem_pad = stem.case.pad
        hin, win, cin = trunk.x.shape[1:]
        self.shapes = {"input": (n, hin + 2 * self.stem_pad, win + 2 * self.stem_pad, STEM_PAD_CHANNELS)}
        for layer in trunk.layers:
            c = layer.case
            co, kh, kw, ci = c.w.shape
            if weight_codes is not None:
                w_bytes = np.ascontiguousarray(weight_codes[layer.name]).view(np.uint8)
            else:
                w_dev = torch.from_numpy(c.w).to(device)
                w_bytes = quantize(w_dev, c.s_w, 0, B.INT8, axis=0, stream=stream).cpu().numpy()
            h, w = layer.in_hw
            pad = c.pad
            if layer is stem:   # padded 4-channel input, zero weights on the extra channel
                w_bytes = np.pad(w_bytes.reshape(co, kh, kw, ci), ((0, 0), (0, 0), (0, 0), (0, STEM_PAD_CHANNELS - ci)))
                h, w, ci, pad = h + 2 * pad, w + 2 * pad, STEM_PAD_CHANNELS, 0
            w_type = B.INT8_2OF4 if (sparse_2of4 and layer is not stem) else B.INT8
            conv = QConv(n, h, w, ci, co, kh, c.stride, pad, act, w_type, act, c.epi, c.z_in - off, c.z_out - off,
                         w_bytes, c.bias, c.s_in, c.s_w, c.s_out, res_type=act, z_res=c.z_res - off,
                         s_res=c.s_res, device=device, stream=stream)
            self.convs[layer.name] = conv
            self.shapes[layer.out] = conv.out_shape
            if layer.name == "stem":
                oh, ow = conv.out_shape[1:3]
                self.shapes["pool"] = (n, (oh + 2 - 3) // 2 + 1, (ow + 2 - 3) // 2 + 1, co)
        self.bufs = {name: empty_codes(shape, act, device) for name, shape in self.shapes.items()
                     if not (fuse_stem_pool and name == "stem")}
        self.units = self._launch_units(fuse_pairs and not sparse_2of4)
        self.final = trunk.layers[-1].out
        s_f, z_f = trunk.qparams[self.final]
        self.final_scale = torch.tensor([s_f], dtype=torch.float32, device=device)
        self.final_zp = torch.tensor([z_f - off], dtype=torch.int32, device=device)
        self.in_scale = torch.tensor([trunk.s_in], dtype=torch.float32, device=device)
        self.in_zp = torch.tensor([trunk.z_in - off], dtype=torch.int32, device=device)
        self.out_f32 = torch.empty(self.shapes[self.final], dtype=torch.float32, device=device)

    def _launch_units(self, fuse):
        """The step's conv launches in order: (i,) for layer i alone, (i, j) for layer i
        with layer j, the next block's first conv reading layer i's output, run right
        behind it in one launch (j's other neighbours never read j's output before it)."""
        layers = self.trunk.layers
        units, moved = [], set()
        for i, la in enumerate(layers):
            if i in moved:
                continue
            j = None
            if fuse and _pair_first(la):
                j = next((k for k in range(i + 1, len(layers))
                          if layers[k].src == la.out and _pair_second(layers[k])), None)
            if j is None:
                units.append((i,))
            else:
                units.append((i, j))
                moved.add(j)
        return units

    def unit_name(self, u):
        return "+".join(self.trunk.layers[i].name for i in self.units[u])

    def launch_unit(self, u, stream=None):
        """Launch conv unit u of the step (one conv, the stem with its fused pooling when
        the trunk fuses it, or a fused pair) on the buffers of the step."""
        b = self.bufs
        layers = [self.trunk.layers[i] for i in self.units[u]]
        la = layers[0]
        conv = self.convs[la.name]
        res = b[la.res_src] if la.res_src is not None else None
        if len(layers) == 2:
            lb = layers[1]
            conv_pair(conv, self.convs[lb.name], b[la.src], res=res, out_a=b[la.out], out_b=b[lb.out], stream=stream)
        elif la.name == "stem" and self.fuse_stem_pool:
            conv.conv_maxpool(b[la.src], 3, 2, 1, out=b["pool"], stream=stream)
        else:
            conv(b[la.src], res=res, out=b[la.out], stream=stream)
            if la.name == "stem":
                n, h, w, c = self.shapes["stem"]
                maxpool2d(b["stem"], n, h, w, c, 3, 2, 1, self.act_type, out=b["pool"], stream=stream)

    def run_codes(self, stream=None, events=None):
        """The 53 convs + max pooling on the codes already in bufs['input'].  events:
        optional list of (start, end) torch events per launch unit, recorded around it."""
        for u in range(len(self.units)):
            if events is not None:
                events[u][0].record()
            self.launch_unit(u, stream)
            if events is not None:
                events[u][1].record()
        return self.bufs[self.final]

    def quantize_input(self, x_f32, stream=None):
        """The step's first launch: the fp32 image into the stem's padded 4-channel codes."""
        quantize_pad(x_f32, self.in_scale, self.in_zp, self.act_type, self.stem_pad, STEM_PAD_CHANNELS,
                     out=self.bufs["input"], stream=stream)

    def dequantize_output(self, stream=None):
        """The step's last launch: the final codes back to fp32 (self.out_f32)."""
        dequantize(self.bufs[self.final], self.shapes[self.final], self.final_scale, self.final_zp, self.act_type,
                   out=self.out_f32, stream=stream)
        return self.out_f32

    def step(self, x_f32, stream=None, events=None):
        """One full forward: quantize -> trunk -> dequantize.  Returns fp32 NHWC output."""
        self.quantize_input(x_f32, stream)
        self.run_codes(stream, events)
        return self.dequantize_output(stream)

    def capture(self, x_f32):
        """Record one step on x_f32 (a fixed device buffer) into a HIP graph, so a
        step is one graph launch instead of one per kernel.  Replay with
        graph.replay(); the result lands in self.out_f32 as with step().  Every
        launch of the step is a plain kernel on the capture stream (no memsets, no
        host synchronisation, no allocation)."""
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):   # warm the capture stream once, eagerly
            self.step(x_f32)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            self.step(x_f32)
        return g

    def capture_parts(self, x_f32):
        """The step as three HIP graphs -- quantize, the convs with the pooling, and
        dequantize -- so a caller can record events between them and time the conv
        section of each replayed step on its own.  Replaying the three in order equals
        one step."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):   # warm the capture stream once, eagerly
            self.step(x_f32)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = [torch.cuda.CUDAGraph() for _ in range(3)]
        with torch.cuda.graph(graphs[0]):
            self.quantize_input(x_f32)
        with torch.cuda.graph(graphs[1]):
            self.run_codes()
        with torch.cuda.graph(graphs[2]):
            self.dequantize_output()
        return graphs

    def launches(self):
        """(kernel family, algorithmic ops, algorithmic bytes) of every launch in one step.
        Ops and bytes are those of the unpadded layer (the stem's 3 channels, K = 147); a
        fused pair counts its first conv's output once, as written, not as read again."""
        out = []
        n = self.trunk.batch
        n_in = int(np.prod(self.trunk.x.shape))
        out.append(("quantize", 0, n_in * 4 + n_in))
        for u, unit in enumerate(self.units):
            ops = by = 0
            for k, i in enumerate(unit):
                layer = self.trunk.layers[i]
                c = layer.case
                co, kh, kw, ci = c.w.shape
                h, w = layer.in_hw
                oh = (h + 2 * c.pad - kh) // c.stride + 1
                ow = (w + 2 * c.pad - kw) // c.stride + 1
                ops += 2 * n * oh * ow * co * kh * kw * ci
                out_elems = n * oh * ow * co
                if layer.name == "stem" and self.fuse_stem_pool:
                    out_elems = int(np.prod(self.shapes["pool"]))   # only the pooled codes are written
                by += (n * h * w * ci if k == 0 else 0) + co * kh * kw * ci + out_elems
                if layer.res_src is not None:
                    by += n * oh * ow * co
            out.append(("qconv:" + self.unit_name(u), ops, by))
            if self.trunk.layers[unit[0]].name == "stem" and not self.fuse_stem_pool:
                _, sh, sw, sc = self.shapes["stem"]
                out.append(("maxpool", 0, n * sh * sw * sc + int(np.prod(self.shapes["pool"]))))
        n_out = int(np.prod(self.shapes[self.final]))
        out.append(("dequantize", 0, n_out + 4 * n_out))
        return out
