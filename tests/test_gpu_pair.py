"""GPU parity of iqnn_qconv_pair_fwd: y_a = conv_a(x, residual) and y_b = conv_b(y_a)
against the oracle's two convs (conv_b on the oracle's own y_a), every byte of both
outputs, and against the two separate iqnn_qconv_fwd calls.  The fused launch takes
conv_a 64 -> 256 channels with a residual (Conv_Add / Conv_Add_Relu) and conv_b 256 ->
64 or 128 (Conv / Conv_Relu); other pairs run as the two calls.  Shapes: one partial
tile, several tiles with a ragged last one, and more tiles than workgroups (each walks
several); activations stored as uint8 codes and as offset int8 bytes q - 128 (zero
points Z - 128), as the ResNet-50 trunk stores them."""
import numpy as np
import pytest

import oracle as O
from integer_quantized_nn_amd import synth
from parity_util import assert_bytes_equal, require_gpu, to_bytes

pytestmark = pytest.mark.gpu

U8, I8 = synth.UINT8, synth.INT8
NONE, RELU, ADD, ADD_RELU = synth.EPI_NONE, synth.EPI_RELU, synth.EPI_ADD, synth.EPI_ADD_RELU
OEPI = {NONE: O.EPI_NONE, RELU: O.EPI_RELU, ADD: O.EPI_ADD, ADD_RELU: O.EPI_ADD_RELU}


def pair_run(seed, n, h, w, ca, cb, cc, epi_a, epi_b, offset):
    """Oracle codes of both outputs and the library's bytes of both (fused call and the
    two separate calls)."""
    torch = require_gpu()
    from integer_quantized_nn_amd.layers import QConv, conv_pair
    a = synth.conv_case(seed, n, h, w, ca, cb, 1, 1, 0, U8, I8, U8, epi_a, res_type=U8)
    b = synth.conv_case(seed + 7, n, h, w, cb, cc, 1, 1, 0, U8, I8, U8, epi_b)
    off = 128 if offset else 0
    t_lib, t_orc = (I8, O.INT8) if offset else (U8, O.UINT8)
    za_in, za_out, z_res = a.z_in - off, a.z_out - off, a.z_res - off
    x = O.quantize(a.x, a.s_in, za_in, t_orc)
    res = O.quantize(a.res, a.s_res, z_res, t_orc) if a.res is not None else None
    wa = O.quantize(a.w, a.s_w, 0, O.INT8, axis=0)
    wb = O.quantize(b.w, b.s_w, 0, O.INT8, axis=0)
    ya = O.qconv(x, za_in, a.s_in, wa, a.s_w, a.bias, a.s_out, za_out, t_orc, OEPI[epi_a], 1, 0, res, a.s_res, z_res)
    # conv_b's input is y_a (scale a.s_out, zero point za_out); its output scale from
    # the float conv of y_a's real values, so the codes span the range
    yf = O.dequantize(ya, a.s_out, za_out).reshape(-1, cb) @ b.w.reshape(cc, cb).T + b.bias
    if epi_b == RELU:
        yf = np.maximum(yf, 0)
    s_out_b = np.float32(max(float(np.abs(yf).max()), 1e-6) / 200.0)
    zb_out = (b.z_out if epi_b == RELU else 100) - off
    yb = O.qconv(ya, za_out, a.s_out, wb, b.s_w, b.bias, s_out_b, zb_out, t_orc, OEPI[epi_b])
    conv_a = QConv(n, h, w, ca, cb, 1, 1, 0, t_lib, I8, t_lib, epi_a, za_in, za_out, to_bytes(wa, I8), a.bias,
                   a.s_in, a.s_w, a.s_out, res_type=t_lib, z_res=z_res, s_res=a.s_res)
    conv_b = QConv(n, h, w, cb, cc, 1, 1, 0, t_lib, I8, t_lib, epi_b, za_out, zb_out, to_bytes(wb, I8), b.bias,
                   a.s_out, b.s_w, s_out_b)
    xd = torch.from_numpy(to_bytes(x, t_lib)).cuda()
    rd = torch.from_numpy(to_bytes(res, t_lib)).cuda() if res is not None else None
    ga, gb = conv_pair(conv_a, conv_b, xd, res=rd)
    sa = conv_a(xd, res=rd)
    sb = conv_b(sa)
    torch.cuda.synchronize()
    return (to_bytes(ya, t_lib), to_bytes(yb, t_lib), ga.cpu().numpy(), gb.cpu().numpy(), sa.cpu().numpy(),
            sb.cpu().numpy())


FUSED = [
    # seed, n, h, w, C_out of conv_b, conv_a epilogue, conv_b epilogue, offset int8 storage
    (1, 1, 7, 9, 64, ADD_RELU, RELU, False),      # 63 pixels: one partial tile
    (2, 2, 13, 17, 64, ADD_RELU, RELU, True),     # 442 pixels: 4 tiles, ragged last
    (3, 2, 11, 15, 128, ADD_RELU, RELU, False),
    (4, 1, 19, 23, 128, ADD, NONE, True),         # plain Conv_Add, Conv
    (5, 3, 160, 150, 64, ADD_RELU, RELU, True),   # 72000 pixels: 563 tiles, more than the 512 workgroups
    (6, 2, 150, 170, 128, ADD_RELU, RELU, False),
]


@pytest.mark.parametrize("case", FUSED, ids=lambda c: "s%dn%dh%dw%dcc%de%d%d%s" % (c[:7] + ("_off" if c[7] else "",)))
def test_pair_fused(case):
    seed, n, h, w, cc, ea, eb, off = case
    ya, yb, ga, gb, sa, sb = pair_run(seed, n, h, w, 64, 256, cc, ea, eb, off)
    assert_bytes_equal(ga, ya, "fused pair y_a")
    assert_bytes_equal(gb, yb, "fused pair y_b")
    assert_bytes_equal(sa, ya, "separate conv_a")
    assert_bytes_equal(sb, yb, "separate conv_b")
    # discrimination: both outputs span many codes
    assert len(np.unique(ga)) >= 64 and len(np.unique(gb)) >= 64


@pytest.mark.parametrize("ca,cb,cc,ea", [(128, 512, 128, ADD_RELU), (64, 256, 256, ADD_RELU), (64, 256, 64, RELU)])
def test_pair_as_two_calls(ca, cb, cc, ea):
    """Pairs outside the fused shapes (the stage-2 hand-off 128 -> 512 -> 128, a 256-
    channel conv_b, conv_a without a residual) give the same bytes as the oracle."""
    ya, yb, ga, gb, _, _ = pair_run(ca + cb + cc + ea, 2, 9, 11, ca, cb, cc, ea, RELU, True)
    assert_bytes_equal(ga, ya, "pair y_a")
    assert_bytes_equal(gb, yb, "pair y_b")


def test_pair_rejects_mismatched_input():
    """conv_b's descriptor must take conv_a's output (channels, type, zero point)."""
    torch = require_gpu()
    from integer_quantized_nn_amd import binding as B
    from integer_quantized_nn_amd.layers import QConv, conv_pair
    rng = np.random.default_rng(0)
    wa = rng.integers(-20, 20, (256, 1, 1, 64)).astype(np.int8).view(np.uint8)
    wb = rng.integers(-20, 20, (64, 1, 1, 256)).astype(np.int8).view(np.uint8)
    bias_a, bias_b = np.zeros(256, np.float32), np.zeros(64, np.float32)
    conv_a = QConv(1, 4, 4, 64, 256, 1, 1, 0, U8, I8, U8, ADD_RELU, 3, 5, wa, bias_a, 0.1, 0.01, 0.2, z_res=2)
    x = torch.zeros((1, 4, 4, 64), dtype=torch.uint8, device="cuda")
    r = torch.zeros((1, 4, 4, 256), dtype=torch.uint8, device="cuda")
    for z_in, xt in [(6, U8), (5, I8)]:   # wrong zero point, wrong type
        conv_b = QConv(1, 4, 4, 256, 64, 1, 1, 0, xt, I8, U8, RELU, z_in, 0, wb, bias_b, 0.2, 0.01, 0.3)
        with pytest.raises(B.IqnnError) as ei:
            conv_pair(conv_a, conv_b, x, res=r)
        assert ei.value.status == 1
    torch.cuda.synchronize()
