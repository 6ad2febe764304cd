"""GPU parity of the ResNet-50 conv trunk (53 fused quantized convs + max pooling).

The oracle runs the same chain layer by layer on the CPU from the same input and
weight codes: its inputs come only from the oracle's own quantize, never from a
GPU result.  At batch 256 every image's final output is compared; the oracle walks
the batch in chunks of images (batch elements are independent)."""
import numpy as np
import pytest

import oracle as O
from integer_quantized_nn_amd import synth
from parity_util import assert_bytes_equal, require_gpu

pytestmark = pytest.mark.gpu


def oracle_trunk(tr, x_codes, w_codes, images):
    acts = {"input": x_codes[images]}
    for layer in tr.layers:
        c = layer.case
        res = acts[layer.res_src] if layer.res_src is not None else None
        acts[layer.out] = O.qconv(acts[layer.src], c.z_in, c.s_in, w_codes[layer.name], c.s_w, c.bias, c.s_out,
                                  c.z_out, O.UINT8, c.epi, c.stride, c.pad, res, c.s_res, c.z_res)
        if layer.name == "stem":
            acts["pool"] = O.maxpool2d(acts["stem"], 3, 2, 1)
    return acts


def _codes(tr):
    x = O.quantize(tr.x, tr.s_in, tr.z_in, O.UINT8)
    w = {l.name: O.quantize(l.case.w, l.case.s_w, 0, O.INT8, axis=0) for l in tr.layers}
    return x, w


def _run_gpu(tr, x, w, offset=False, sparse=False, fuse_pairs=True):
    import torch
    from integer_quantized_nn_amd.resnet50 import QuantResNet50Trunk
    net = QuantResNet50Trunk(tr, weight_codes={k: O.pack(v, O.INT8) for k, v in w.items()}, offset_codes=offset,
                             sparse_2of4=sparse, fuse_pairs=fuse_pairs)
    # the trunk's input buffer is the image with the stem's border and a 4th channel,
    # all holding the input zero-point code
    p = net.stem_pad
    xp = np.pad(x, ((0, 0), (p, p), (p, p), (0, 1)), constant_values=tr.z_in)
    net.bufs["input"].copy_(torch.from_numpy(O.pack(xp, O.UINT8) ^ np.uint8(0x80 if offset else 0)))
    net.run_codes()
    torch.cuda.synchronize()
    return net


@pytest.mark.parametrize("offset,fuse", [(False, True), (True, True), (True, False)],
                         ids=["uint8", "offset_int8", "offset_int8_unfused"])
def test_trunk_every_layer_small_batch(offset, fuse):
    """Batch 2 at 224x224: every intermediate tensor of both images, byte for byte.
    With offset codes (uint8 code q stored as the int8 byte q - 128, zero points
    shifted alike) every buffer holds the uint8 oracle's bytes XOR 0x80.  The trunk
    runs its block hand-offs fused (one launch per pair) or as separate launches."""
    require_gpu()
    tr = synth.resnet50_trunk(seed=3, batch=2)
    x, w = _codes(tr)
    net = _run_gpu(tr, x, w, offset, fuse_pairs=fuse)
    assert len(net.units) == (50 if fuse else 53)
    ref = oracle_trunk(tr, x, w, [0, 1])
    flip = np.uint8(0x80 if offset else 0)
    for name, buf in net.bufs.items():
        if name == "input":
            continue
        assert_bytes_equal(buf.cpu().numpy(), O.pack(ref[name], O.UINT8) ^ flip, name)


def test_trunk_2of4_every_layer_small_batch():
    """The trunk with 2:4-pruned weights after the stem, every conv after the stem on the
    sparse kernels, offset int8 storage, batch 3: every intermediate tensor against the
    oracle's dense convolutions of the same codes."""
    require_gpu()
    tr = synth.resnet50_trunk(seed=6, batch=3, sparse_2of4=True)
    x, w = _codes(tr)
    for l in tr.layers[1:]:
        assert np.all((w[l.name].reshape(-1, 4) != 0).sum(axis=1) <= 2), l.name
    net = _run_gpu(tr, x, w, True, sparse=True)
    ref = oracle_trunk(tr, x, w, [0, 1, 2])
    for name, buf in net.bufs.items():
        if name == "input":
            continue
        assert_bytes_equal(buf.cpu().numpy(), O.pack(ref[name], O.UINT8) ^ np.uint8(0x80), name)
    for name in ("l1.0.out", "l3.5.out", tr.layers[-1].out):
        assert len(np.unique(ref[name])) >= 32, name


def oracle_trunk_final(tr, x_codes, w_codes, chunk=32):
    """The oracle chain over every image of the batch, `chunk` images at a time (the
    images are independent); returns the final output codes and, for the first chunk,
    every intermediate tensor (for the discrimination check)."""
    final = tr.layers[-1].out
    out, first = [], None
    for i0 in range(0, tr.batch, chunk):
        acts = oracle_trunk(tr, x_codes, w_codes, list(range(i0, min(i0 + chunk, tr.batch))))
        out.append(acts[final])
        if first is None:
            first = acts
    return np.concatenate(out), first


def test_trunk_full_batch_every_image():
    """Batch 256 (the benchmark configuration): the step as the benchmark runs it
    (float input, GPU quantize -> 53 convs + max pooling -> dequantize, GPU-quantized
    weights), with uint8 codes and with the offset int8 storage the benchmark uses.
    Every final output code of all 256 images and every dequantized float (as bits)
    against the oracle chain (about 1 T multiply-adds on the host cores)."""
    torch = require_gpu()
    from integer_quantized_nn_amd.resnet50 import QuantResNet50Trunk
    tr = synth.resnet50_trunk(seed=0, batch=256)
    x, w = _codes(tr)
    final = tr.layers[-1].out
    ref_final, first = oracle_trunk_final(tr, x, w)
    s_f, z_f = tr.qparams[final]
    want_f = O.dequantize(ref_final, s_f, z_f)
    xd = torch.from_numpy(tr.x).cuda()
    for offset in (False, True):
        net = QuantResNet50Trunk(tr, offset_codes=offset)
        y = net.step(xd)
        torch.cuda.synchronize()
        got_codes = net.bufs[final].cpu().numpy()
        flip = np.uint8(0x80 if offset else 0)
        assert_bytes_equal(got_codes, O.pack(ref_final, O.UINT8) ^ flip, "trunk output codes, offset %s" % offset)
        assert np.array_equal(y.cpu().numpy().view(np.uint32), want_f.view(np.uint32)), offset
        del net, y
        torch.cuda.empty_cache()
    # discrimination: the outputs span many codes and rarely saturate
    for name in ("stem", "l1.0.out", "l3.5.out", final):
        q = first[name]
        assert len(np.unique(q)) >= 32 and (q == 255).mean() < 0.02, name


@pytest.mark.parametrize("offset", [False, True], ids=["uint8", "offset_int8"])
def test_trunk_graph_replay_matches_eager(offset):
    """The step captured in a HIP graph and replayed three times, with other eager
    work and synchronisations in between, gives the eager step's bytes each time."""
    torch = require_gpu()
    from integer_quantized_nn_amd.resnet50 import QuantResNet50Trunk
    tr = synth.resnet50_trunk(seed=5, batch=2)
    net = QuantResNet50Trunk(tr, offset_codes=offset)
    x = torch.from_numpy(tr.x).cuda()
    want = net.step(x).clone()
    want_codes = net.bufs[tr.layers[-1].out].clone()
    g = net.capture(x)
    for i in range(3):
        net.out_f32.fill_(-1.0)
        net.bufs[tr.layers[-1].out].fill_(0)
        junk = torch.randn(1 << 16, device="cuda").sum()   # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(net.bufs[tr.layers[-1].out], want_codes), "replay %d codes" % i
        assert torch.equal(net.out_f32.view(torch.int32), want.view(torch.int32)), "replay %d floats" % i
        del junk
