"""GPU parity of the implicit-GEMM quantized conv: every output byte equals the
oracle's (direct 7-loop conv, explicit zero-point subtraction, strict fp32
requant).  Small shapes cover several tiles, ragged pixel / channel tails, every
epilogue, activation / weight / output type and the stride / padding / kernel
sizes of the workloads; the two standalone conv workloads run at full size and
are compared on every output byte."""
import numpy as np
import pytest

import oracle as O
from integer_quantized_nn_amd import synth
from parity_util import (assert_bytes_equal, conv_codes, gpu_conv, oracle_conv, otype, require_gpu,
                         to_bytes)

pytestmark = pytest.mark.gpu

U8, I8, U4, I4, I32 = synth.UINT8, synth.INT8, synth.UINT4, synth.INT4, synth.INT32
NONE, RELU, ADD, ADD_RELU, RAW = synth.EPI_NONE, synth.EPI_RELU, synth.EPI_ADD, synth.EPI_ADD_RELU, synth.EPI_RAW

SMALL = [
    # n, h, w, c_in, c_out, k, stride, pad, x_type, w_type, y_type, epi, res_type
    (2, 9, 11, 64, 64, 3, 1, 1, U8, I8, U8, RELU, U8),
    (3, 7, 7, 32, 128, 3, 2, 1, U8, I8, U8, ADD_RELU, U8),
    (1, 13, 5, 16, 80, 1, 1, 0, I8, I8, I8, NONE, U8),
    (2, 6, 9, 48, 192, 1, 2, 0, U8, I8, U8, NONE, U8),
    (1, 10, 10, 128, 48, 3, 1, 1, U8, I8, I32, RAW, U8),
    (2, 8, 8, 32, 64, 3, 1, 1, U4, I4, U4, ADD_RELU, U4),
    (1, 9, 7, 64, 96, 1, 1, 0, U4, I4, U4, RELU, U4),
    (2, 5, 5, 16, 32, 3, 2, 1, I4, I4, I8, ADD, I8),
    (1, 12, 12, 32, 64, 3, 1, 1, U4, I8, U8, ADD_RELU, U4),
    (2, 15, 15, 3, 64, 7, 2, 3, U8, I8, U8, RELU, U8),
    (1, 8, 8, 8, 24, 3, 1, 1, U8, I8, U8, RELU, U8),
    (1, 4, 4, 256, 256, 3, 1, 1, U8, I8, U8, RELU, U8),
    (1, 3, 3, 64, 40, 3, 1, 2, U8, I8, U8, NONE, U8),
    (1, 1, 1, 1024, 2048, 1, 1, 0, U8, I8, U8, ADD_RELU, U8),
    # degenerate: one input and one output channel on a 1x1 image, a kernel wider than
    # its one-pixel-wide input, two 4-bit channels
    (1, 1, 1, 1, 1, 1, 1, 0, U8, I8, U8, NONE, U8),
    (2, 3, 1, 3, 5, 3, 1, 1, U8, I8, I8, RELU, U8),
    (1, 1, 2, 16, 2, 1, 1, 0, U4, I4, U4, NONE, U4),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "n%dh%dw%dci%dco%dk%ds%dp%d_x%dw%dy%de%d" % c[:12])
def test_conv_small_shapes(case):
    require_gpu()
    n, h, w, ci, co, k, s, p, xt, wt, yt, epi, rt = case
    c = synth.conv_case(hash(case) % 2 ** 31, n, h, w, ci, co, k, s, p, xt, wt, yt, epi, res_type=rt)
    x, wc, res = conv_codes(c)
    want = to_bytes(oracle_conv(c, x, wc, res), yt)
    got = gpu_conv(c, x, wc, res)
    assert_bytes_equal(got, want, str(case))


@pytest.mark.parametrize("hw,k,stride,co", [((23, 23), 7, 2, 64), ((20, 17), 7, 2, 128), ((12, 12), 3, 1, 64),
                                             ((9, 14), 5, 2, 96),
                                             # direct stem kernel: even padded width, whole 128-pixel tiles
                                             ((32, 32), 7, 2, 64), ((32, 32), 7, 2, 32), ((64, 48), 7, 2, 64)])
def test_conv_four_channel_padded_input(hw, k, stride, co):
    """The 4-channel gather (image stems): a 3-channel image quantized into a border
    of Z_in codes plus a 4th Z_in channel, convolved without padding, equals the
    oracle's padded 3-channel convolution."""
    torch = require_gpu()
    from integer_quantized_nn_amd.layers import QConv
    h, w = hw
    pad = k // 2
    c = synth.conv_case(hash((hw, k, stride, co)) % 2 ** 31, 2, h, w, 3, co, k, stride, pad, U8, I8, U8, RELU)
    x, wc, _ = conv_codes(c)
    want = to_bytes(oracle_conv(c, x, wc, None), U8)
    xp = np.pad(x, ((0, 0), (pad, pad), (pad, pad), (0, 1)), constant_values=c.z_in)
    wp = np.pad(wc, ((0, 0), (0, 0), (0, 0), (0, 1)))
    conv = QConv(2, h + 2 * pad, w + 2 * pad, 4, co, k, stride, 0, U8, I8, U8, RELU, c.z_in, c.z_out,
                 to_bytes(wp, I8), c.bias, c.s_in, c.s_w, c.s_out)
    y = conv(torch.from_numpy(to_bytes(xp, U8)).cuda())
    torch.cuda.synchronize()
    assert_bytes_equal(y.cpu().numpy(), want, "c4 %s" % ((hw, k, stride, co),))


@pytest.mark.parametrize("n", [1, 2])
def test_stem_input_not_whole_16_byte_units(n):
    """A 31x32 image padded to 37x38x4: with N = 1 the input is 5624 bytes (8 mod 16),
    which the slab kernels of the stem cannot read in whole 16-byte units, so
    iqnn_qconv_fwd takes the 4-channel streaming gather and iqnn_qconv_maxpool_fwd
    reports UNSUPPORTED; with N = 2 (11248 bytes) both run the stem kernels.  Every
    computed byte against the oracle, including the last pixel of the last image."""
    torch = require_gpu()
    from integer_quantized_nn_amd import binding as B
    from integer_quantized_nn_amd.layers import QConv
    h, w = 31, 32
    c = synth.conv_case(3700 + n, n, h, w, 3, 64, 7, 2, 3, U8, I8, U8, RELU)
    x, wc, _ = conv_codes(c)
    conv_ref = oracle_conv(c, x, wc, None)
    xp = np.pad(x, ((0, 0), (3, 3), (3, 3), (0, 1)), constant_values=c.z_in)
    wp = np.pad(wc, ((0, 0), (0, 0), (0, 0), (0, 1)))
    conv = QConv(n, h + 6, w + 6, 4, 64, 7, 2, 0, U8, I8, U8, RELU, c.z_in, c.z_out,
                 to_bytes(wp, I8), c.bias, c.s_in, c.s_w, c.s_out)
    xd = torch.from_numpy(to_bytes(xp, U8)).cuda()
    y = conv(xd)
    torch.cuda.synchronize()
    assert_bytes_equal(y.cpu().numpy(), to_bytes(conv_ref, U8), "stem n=%d" % n)
    if n == 1:
        with pytest.raises(B.IqnnError) as ei:
            conv.conv_maxpool(xd)
        assert ei.value.status == 2 and "16" in str(ei.value)
    else:
        yp = conv.conv_maxpool(xd)
        torch.cuda.synchronize()
        assert_bytes_equal(yp.cpu().numpy(), to_bytes(O.maxpool2d(conv_ref, 3, 2, 1), U8), "stem+pool n=%d" % n)


@pytest.mark.parametrize("n,hw,y_type,epi", [(2, (32, 32), U8, RELU), (3, (48, 64), I8, NONE), (1, (16, 224), U8, NONE),
                                          (2, (224, 224), U8, RELU), (1, (40, 64), I8, RELU),
                                          (1, (20, 36), I8, NONE), (2, (16, 248), U8, RELU),
                                          (3, (100, 132), I8, RELU), (1, (28, 124), U8, NONE)])
def test_stem_fused_max_pooling(n, hw, y_type, epi):
    """iqnn_qconv_maxpool_fwd (the stem conv and 3x3/2 pad 1 max pooling in one launch)
    equals the oracle's conv followed by the oracle's max pooling, byte for byte.  The
    shapes span one to three waves of 31 pooled columns (pooled widths 8, 9, 16, 31,
    33, 56, 62), bands of pooled rows whose first row takes its upper stem row from the
    band above, a short last band, and signed codes whose window maxima are negative."""
    torch = require_gpu()
    from integer_quantized_nn_amd.layers import QConv
    h, w = hw
    c = synth.conv_case(hash((n, hw, y_type, epi)) % 2 ** 31, n, h, w, 3, 64, 7, 2, 3, U8, I8, y_type, epi)
    x, wc, _ = conv_codes(c)
    conv_ref = oracle_conv(c, x, wc, None)
    want = to_bytes(O.maxpool2d(conv_ref, 3, 2, 1), y_type)
    xp = np.pad(x, ((0, 0), (3, 3), (3, 3), (0, 1)), constant_values=c.z_in)
    wp = np.pad(wc, ((0, 0), (0, 0), (0, 0), (0, 1)))
    conv = QConv(n, h + 6, w + 6, 4, 64, 7, 2, 0, U8, I8, y_type, epi, c.z_in, c.z_out,
                 to_bytes(wp, I8), c.bias, c.s_in, c.s_w, c.s_out)
    y = conv.conv_maxpool(torch.from_numpy(to_bytes(xp, U8)).cuda())
    torch.cuda.synchronize()
    assert y.shape == want.shape
    assert_bytes_equal(y.cpu().numpy(), want, "stem+pool %s" % ((n, hw, y_type, epi),))


@pytest.mark.parametrize("kh,kw", [(3, 8), (5, 7), (8, 8)])
def test_stem_fused_max_pooling_other_filter_sizes(kh, kw):
    """Stride-2 stems with 3x8, 5x7 and 8x8 filters on the 4-channel input (7 taps are
    widened to 8): the fused kernel's variant that reads the filter-row count at run
    time, against the oracle's conv and max pooling, every pooled byte.  The 4-channel
    gather reads 8 taps per filter row, so the fused path takes widths of 7 and 8 only."""
    torch = require_gpu()
    from integer_quantized_nn_amd.layers import QConv
    n = 2
    # even stem output height and width, an even input width, whole 16-byte units
    h = next(v for v in range(30, 40) if ((v - kh) // 2 + 1) % 2 == 0)
    w = next(v for v in range(64, 80) if v % 2 == 0 and ((v - kw) // 2 + 1) % 2 == 0 and (n * h * v) % 4 == 0)
    c = synth.conv_case(6000 + 10 * kh + kw, n, h, w, 3, 64, 8, 2, 0, U8, I8, U8, RELU)
    x, wc, _ = conv_codes(c)
    wc = np.ascontiguousarray(wc[:, :kh, :kw, :])
    conv_ref = oracle_conv(c, x, wc, None)
    want = to_bytes(O.maxpool2d(conv_ref, 3, 2, 1), U8)
    xp = np.pad(x, ((0, 0), (0, 0), (0, 0), (0, 1)), constant_values=c.z_in)
    wp = np.pad(wc, ((0, 0), (0, 0), (0, 0), (0, 1)))
    conv = QConv(n, h, w, 4, 64, kh, 2, 0, U8, I8, U8, RELU, c.z_in, c.z_out, to_bytes(wp, I8), c.bias,
                 c.s_in, c.s_w, c.s_out, kw=kw)
    y = conv.conv_maxpool(torch.from_numpy(to_bytes(xp, U8)).cuda())
    torch.cuda.synchronize()
    assert y.shape == want.shape
    assert_bytes_equal(y.cpu().numpy(), want, "stem+pool %dx%d" % (kh, kw))


@pytest.mark.parametrize("z_odd", [0, 1])
@pytest.mark.parametrize("n,hw", [(2, (64, 96)), (3, (28, 224))])
def test_stem_fused_max_pooling_signed_input(n, hw, z_odd):
    """The image stem as the trunk runs it -- signed input codes, 7 filter rows -- takes
    the fused kernel whose choices are fixed at compile time, including the odd part of
    Z_out (both parities here); every pooled byte against the oracle."""
    torch = require_gpu()
    from integer_quantized_nn_amd.layers import QConv
    h, w = hw
    c = synth.conv_case(5100 + 7 * n + z_odd, n, h, w, 3, 64, 7, 2, 3, I8, I8, U8, RELU)
    c.z_out = (c.z_out & ~1) | z_odd
    x, wc, _ = conv_codes(c)
    conv_ref = oracle_conv(c, x, wc, None)
    want = to_bytes(O.maxpool2d(conv_ref, 3, 2, 1), U8)
    xp = np.pad(x, ((0, 0), (3, 3), (3, 3), (0, 1)), constant_values=c.z_in)
    wp = np.pad(wc, ((0, 0), (0, 0), (0, 0), (0, 1)))
    conv = QConv(n, h + 6, w + 6, 4, 64, 7, 2, 0, I8, I8, U8, RELU, c.z_in, c.z_out,
                 to_bytes(wp, I8), c.bias, c.s_in, c.s_w, c.s_out)
    y = conv.conv_maxpool(torch.from_numpy(to_bytes(xp, I8)).cuda())
    torch.cuda.synchronize()
    assert_bytes_equal(y.cpu().numpy(), want, "stem+pool signed input %s" % ((n, hw, z_odd),))


# 64-channel 3x3 / stride 1 / pad 1 layers on 56-pixel rows (the direct kernel, forced at
# any batch through tile 18: one slab of input rows per two output rows): odd heights (a
# tile's second row outside the image), several 64-channel output blocks, signed codes,
# raw accumulators, padding-dominated two-row images, and batches with more two-row tiles
# than workgroups (each workgroup walks several tiles through its three slab buffers;
# the oracle checks the listed images)
DIRECT = [
    # n, h, c_out, x_type, y_type, epi, images checked (None: all)
    (2, 56, 64, U8, U8, RELU, None),
    (1, 7, 128, U8, I8, NONE, None),
    (3, 2, 64, I8, U8, RELU, None),
    (1, 5, 192, U8, U8, NONE, None),
    (2, 3, 64, U8, I32, RAW, None),
    (20, 56, 64, U8, I32, RAW, (0, 19)),
    (45, 55, 128, U8, U8, RELU, (0, 22, 44)),
]


@pytest.mark.parametrize("case", DIRECT, ids=lambda c: "n%dh%dco%d_x%dy%de%d" % c[:6])
def test_conv_direct3x3_64ch(case):
    require_gpu()
    from integer_quantized_nn_amd import binding as B
    n, h, co, xt, yt, epi, images = case
    c = synth.conv_case(hash(case[:6]) % 2 ** 31, n, h, 56, 64, co, 3, 1, 1, xt, I8, yt, epi)
    x, wc, _ = conv_codes(c)
    got = gpu_conv(c, x, wc, None, cfg=(18, 0))
    sel = list(images) if images is not None else None
    want = to_bytes(oracle_conv(c, x, wc, None, sel), yt)
    assert_bytes_equal(got if sel is None else got[sel], want, str(case))


def test_conv_direct3x3_automatic_large_batch():
    """From 512 two-row tiles the automatic choice takes the direct kernel: batch 80
    of the 56x56 64->64 Conv_Relu layer, every output byte against the oracle and
    against the streaming kernel (tile 11)."""
    require_gpu()
    from integer_quantized_nn_amd import binding as B
    c = synth.conv_case(4242, 80, 56, 56, 64, 64, 3, 1, 1, U8, I8, U8, RELU)
    x, wc, _ = conv_codes(c)
    got = gpu_conv(c, x, wc, None)
    assert_bytes_equal(got, to_bytes(oracle_conv(c, x, wc, None), U8), "direct, batch 80")
    other = gpu_conv(c, x, wc, None, cfg=(11, 0))
    assert_bytes_equal(got, other, "direct vs streaming kernel, batch 80")


# 8-bit layers with C_in % 64 == 0 (the pipelined kernel): ring depths that do not
# divide the stage count, one-stage contractions, ragged pixel tails and channel
# counts that are not multiples of any block
PIPE = [
    # n, h, w, c_in, c_out, k, stride, pad, epi
    (2, 13, 11, 64, 64, 1, 1, 0, RELU),          # one stage
    (2, 13, 11, 64, 256, 1, 1, 0, ADD_RELU),     # residual prefetch
    (1, 17, 9, 320, 96, 1, 1, 0, ADD_RELU),      # 5 stages
    (2, 9, 10, 64, 64, 3, 1, 1, RELU),           # 9 stages, padding taps
    (1, 15, 15, 128, 320, 3, 2, 1, NONE),        # stride 2, 18 stages
    (3, 7, 7, 512, 128, 1, 2, 0, NONE),          # strided 1x1 downsample
]


@pytest.mark.parametrize("tile", list(range(18)) + [20, 21, 22, 23])
def test_conv_every_tile(tile):
    """Each block tile of the pipelined and streaming kernels (forced per call through
    iqnn_qconv_fwd_cfg) gives the oracle's bytes on the same layers, and so does the
    4-channel gather on the tiles it is built for."""
    torch = require_gpu()
    from integer_quantized_nn_amd.layers import QConv
    for i, (n, h, w, ci, co, k, s, p, epi) in enumerate(PIPE):
        c = synth.conv_case(1000 + 17 * i, n, h, w, ci, co, k, s, p, U8, I8, U8, epi, res_type=U8)
        x, wc, res = conv_codes(c)
        want = to_bytes(oracle_conv(c, x, wc, res), U8)
        assert_bytes_equal(gpu_conv(c, x, wc, res, cfg=(tile, 0)), want, "tile %d %s" % (tile, PIPE[i]))
    if tile in (0, 1, 6, 8, 10, 12):
        h, w, k, st, co = 21, 19, 7, 2, 64 if tile != 1 else 128
        c = synth.conv_case(77 + tile, 2, h, w, 3, co, k, st, 3, U8, I8, U8, RELU)
        x, wc, _ = conv_codes(c)
        want = to_bytes(oracle_conv(c, x, wc, None), U8)
        xp = np.pad(x, ((0, 0), (3, 3), (3, 3), (0, 1)), constant_values=c.z_in)
        wp = np.pad(wc, ((0, 0), (0, 0), (0, 0), (0, 1)))
        conv = QConv(2, h + 6, w + 6, 4, co, k, st, 0, U8, I8, U8, RELU, c.z_in, c.z_out,
                     to_bytes(wp, I8), c.bias, c.s_in, c.s_w, c.s_out)
        y = conv(torch.from_numpy(to_bytes(xp, U8)).cuda(), cfg=(tile, 0))
        torch.cuda.synchronize()
        assert_bytes_equal(y.cpu().numpy(), want, "tile %d four-channel gather" % tile)


@pytest.mark.parametrize("tile", list(range(18)) + [20, 21, 22, 23])
def test_conv_every_tile_signed_codes(tile):
    """The same layers, and a 3x3 Conv_Add_Relu, with signed 8-bit activations,
    residuals and outputs: the streaming configurations of the automatic choice run
    their variant without the activation sign flip on these, the others the flipping
    one with x_xor = 0; every tile gives the oracle's bytes."""
    require_gpu()
    layers = PIPE + [(2, 9, 10, 64, 128, 3, 1, 1, ADD_RELU), (1, 11, 13, 128, 64, 3, 2, 1, ADD)]
    for i, (n, h, w, ci, co, k, s, p, epi) in enumerate(layers):
        c = synth.conv_case(2000 + 13 * i, n, h, w, ci, co, k, s, p, I8, I8, I8, epi, res_type=I8)
        x, wc, res = conv_codes(c)
        want = to_bytes(oracle_conv(c, x, wc, res), I8)
        got = gpu_conv(c, x, wc, res, cfg=(tile, 0))
        assert_bytes_equal(got, want, "tile %d %s" % (tile, layers[i]))
        assert len(np.unique(got)) >= 32   # the codes span the range


# 3x3 layers without a residual with more pixel tiles per XCD share than a share has
# persistent blocks, for every configuration (over 64 tiles of 256 pixels per share),
# so blocks run more than one tile and the streaming kernel's split stage loop hands
# its issue side over to the next tile inside the loop: 9 and 27 stages per tile,
# against ring depths that divide them (the loop in rounds) and ones that do not.
MULTI_TILE = [
    (64, 48, 48, 64, 64, 3, 1, 1, RELU),      # 147456 pixels, 9 stages
    (24, 76, 76, 192, 64, 3, 1, 1, NONE),     # 138624 pixels, 27 stages
]
_multi_tile_cases = {}


def _multi_tile_case(i):
    if i not in _multi_tile_cases:
        n, h, w, ci, co, k, s, p, epi = MULTI_TILE[i]
        c = synth.conv_case(3000 + 7 * i, n, h, w, ci, co, k, s, p, I8, I8, I8, epi)
        x, wc, _ = conv_codes(c)
        _multi_tile_cases[i] = (c, x, wc, to_bytes(oracle_conv(c, x, wc, None), I8))
    return _multi_tile_cases[i]


@pytest.mark.parametrize("tile", list(range(18)) + [20, 21, 22, 23])
def test_conv_every_tile_several_tiles_per_block(tile):
    """Every block configuration on signed 8-bit codes with several tiles per
    persistent block; every output byte against the oracle."""
    require_gpu()
    for i in range(len(MULTI_TILE)):
        c, x, wc, want = _multi_tile_case(i)
        got = gpu_conv(c, x, wc, None, cfg=(tile, 0))
        assert_bytes_equal(got, want, "tile %d %s" % (tile, MULTI_TILE[i]))
        assert len(np.unique(got)) >= 32


# 4-bit activations with C_in % 64 == 0 (the streaming kernel's 4-bit path): both
# block heights (C_out <= 64 -> 64-channel blocks, 32-byte residual rows; else 128),
# UINT4 and INT4 codes, 4-bit residuals, stride 2, ragged pixel tails
B4S = [
    # n, h, w, c_in, c_out, k, stride, pad, x_type, y_type, epi, res_type
    (2, 9, 11, 64, 64, 3, 1, 1, U4, U4, ADD_RELU, U4),
    (1, 13, 7, 128, 128, 3, 1, 1, U4, U4, ADD_RELU, U4),
    (2, 8, 9, 64, 96, 1, 1, 0, I4, I4, ADD, I4),
    (1, 15, 15, 128, 64, 3, 2, 1, I4, U8, RELU, U4),
    (3, 7, 7, 192, 32, 1, 1, 0, U4, I8, NONE, U4),
    (1, 6, 5, 64, 256, 3, 1, 1, U4, U4, RELU, U4),
]


@pytest.mark.parametrize("case", B4S, ids=lambda c: "n%dh%dw%dci%dco%dk%ds%dp%d_x%dy%de%d" % c[:11])
def test_conv_4bit_streaming(case):
    require_gpu()
    n, h, w, ci, co, k, s, p, xt, yt, epi, rt = case
    c = synth.conv_case(hash(case) % 2 ** 31, n, h, w, ci, co, k, s, p, xt, I4, yt, epi, res_type=rt)
    x, wc, res = conv_codes(c)
    want = to_bytes(oracle_conv(c, x, wc, res), yt)
    assert_bytes_equal(gpu_conv(c, x, wc, res), want, str(case))


@pytest.mark.parametrize("case", B4S, ids=lambda c: "n%dh%dw%dci%dco%dk%ds%dp%d_x%dy%de%d" % c[:11])
def test_conv_4bit_fp6_path(case):
    """The same 4-bit layers on the FP6 MFMA path (forced through tile 19): INT4 weights
    and the activations as BF6 codes, fp32 accumulation of integers, every byte equal to
    the oracle's."""
    require_gpu()
    from integer_quantized_nn_amd import binding as B
    n, h, w, ci, co, k, s, p, xt, yt, epi, rt = case
    c = synth.conv_case(hash(case) % 2 ** 31 + 1, n, h, w, ci, co, k, s, p, xt, I4, yt, epi, res_type=rt)
    x, wc, res = conv_codes(c)
    want = to_bytes(oracle_conv(c, x, wc, res), yt)
    got = gpu_conv(c, x, wc, res, cfg=(19, 0))
    assert_bytes_equal(got, want, "fp6 " + str(case))


def test_conv_4bit_fp6_adversarial_codes():
    """Every 4-bit code, including -8 weights and the extreme activations 0 and 15, on
    the FP6 path."""
    require_gpu()
    from integer_quantized_nn_amd import binding as B
    rng = np.random.default_rng(43)
    for (xt, yt, rt) in [(U4, U4, U4), (I4, I4, I4)]:
        c = synth.conv_case(9, 3, 5, 6, 64, 64, 3, 1, 1, xt, I4, yt, ADD_RELU, res_type=rt)
        xlo, xhi = O.qrange(otype(xt))
        rlo, rhi = O.qrange(otype(rt))
        x = rng.integers(xlo, xhi + 1, size=c.x.shape).astype(np.int32)
        w = rng.integers(-8, 8, size=c.w.shape).astype(np.int32)
        r = rng.integers(rlo, rhi + 1, size=c.res.shape).astype(np.int32)
        c.z_in = int(xhi) if xt == U4 else 0
        want = to_bytes(oracle_conv(c, x, w, r), yt)
        got = gpu_conv(c, x, w, r, cfg=(19, 0))
        assert_bytes_equal(got, want, "fp6 adversarial x%d" % xt)


def test_conv_4bit_fp6_workload_full_size():
    """The 4-bit workload (N=64, 28x28, 128 -> 128, Conv_Add_Relu, UINT4 in / out /
    residual, INT4 weights) on the FP6 path: every output byte against the oracle and
    against the int8 path."""
    require_gpu()
    c = synth.conv3x3_4bit()
    x, wc, res = conv_codes(c)
    got = gpu_conv(c, x, wc, res, cfg=(19, 0))
    assert_bytes_equal(got, gpu_conv(c, x, wc, res), "fp6 vs int8 path")
    assert_bytes_equal(got, to_bytes(oracle_conv(c, x, wc, res), c.y_type), "fp6 vs oracle")


def test_conv_4bit_fp6_path_reads_only_its_own_region():
    """The FP6 path is the one that runs under tile 19: with the int8 weights and the
    int32 bias of the packed layer overwritten it still matches the oracle, and the
    default path still does with the BF6 region overwritten instead."""
    require_gpu()
    import torch
    from integer_quantized_nn_amd import binding as B
    from integer_quantized_nn_amd.layers import QConv
    c = synth.conv_case(77, 1, 13, 7, 128, 128, 3, 1, 1, U4, I4, U4, ADD_RELU, res_type=U4)
    x, wc, res = conv_codes(c)
    want = to_bytes(oracle_conv(c, x, wc, res), c.y_type)
    ocp, kp = 256, 9 * 128
    std_bytes = 8 * ocp + 256 + 2 * ocp * kp          # bias, multipliers, scalars, int8 weights, tile-order copy
    xd = torch.from_numpy(to_bytes(x, c.x_type)).cuda()
    rd = torch.from_numpy(to_bytes(res, c.res_type)).cuda()

    def layer():
        conv = QConv(1, 13, 7, 128, 128, 3, c.stride, c.pad, c.x_type, I4, c.y_type, c.epi, c.z_in, c.z_out,
                     to_bytes(wc, I4), c.bias, c.s_in, c.s_w, c.s_out, res_type=c.res_type, z_res=c.z_res,
                     s_res=c.s_res)
        assert conv.packed.numel() == std_bytes + 4 * ocp + ocp * kp
        return conv

    conv = layer()
    conv.packed[:4 * ocp].fill_(0x5A)
    conv.packed[8 * ocp + 256:std_bytes].fill_(0x5A)
    got = conv(xd, res=rd, cfg=(19, 0))
    torch.cuda.synchronize()
    assert_bytes_equal(got.cpu().numpy(), want, "fp6 path with the int8 region overwritten")
    conv = layer()
    conv.packed[std_bytes:].fill_(0x5A)
    got = conv(xd, res=rd)
    torch.cuda.synchronize()
    assert_bytes_equal(got.cpu().numpy(), want, "default path with the BF6 region overwritten")


def test_conv_adversarial_codes_and_padding():
    # every code of each type, including -128 / 255 / -8 / 15, on tiny images where
    # most taps read padding
    require_gpu()
    rng = np.random.default_rng(42)
    for (xt, wt, yt, rt, ci) in [(U8, I8, U8, U8, 32), (I8, I8, I8, I8, 16), (U4, I4, U4, U4, 32), (I4, I4, I4, I4, 16)]:
        c = synth.conv_case(7, 3, 2, 3, ci, 64, 3, 1, 2, xt, wt, yt, ADD_RELU, res_type=rt)
        xlo, xhi = O.qrange(otype(xt))
        wlo, whi = O.qrange(otype(wt))
        rlo, rhi = O.qrange(otype(rt))
        x = rng.integers(xlo, xhi + 1, size=c.x.shape).astype(np.int32)
        w = rng.integers(wlo, whi + 1, size=c.w.shape).astype(np.int32)
        r = rng.integers(rlo, rhi + 1, size=c.res.shape).astype(np.int32)
        c.z_in = int(xhi) if xt in (U8, U4) else 0
        want = to_bytes(oracle_conv(c, x, w, r), yt)
        got = gpu_conv(c, x, w, r)
        assert_bytes_equal(got, want, "adversarial x%d w%d" % (xt, wt))


def test_conv_relu_is_passive_clamp():
    # Conv_Relu == max(Conv, Z_out) byte for byte on the GPU too
    require_gpu()
    c = synth.conv_case(3, 2, 9, 9, 32, 64, 3, 1, 1, U8, I8, U8, RELU)
    x, w, _ = conv_codes(c)
    relu = gpu_conv(c, x, w, None)
    c.epi = NONE
    none = gpu_conv(c, x, w, None)
    assert np.array_equal(relu, np.maximum(none, np.uint8(c.z_out)))


def test_conv3x3_int8_full_size():
    """ResNet 3x3 conv workload: N=32 56x56 64->64, uint8 in, Conv_Relu to uint8.  Every
    output byte of the whole batch against the oracle."""
    require_gpu()
    c = synth.conv3x3_int8(seed=0)
    x, w, _ = conv_codes(c)
    got = gpu_conv(c, x, w, None)
    want = to_bytes(oracle_conv(c, x, w, None), c.y_type)
    assert_bytes_equal(got, want, "conv3x3_int8")
    # discrimination: the case exercises most output codes and rarely saturates
    q = got
    assert len(np.unique(q)) >= 64 and (q == 255).mean() < 0.01


def test_conv3x3_4bit_full_size():
    """4-bit workload: N=64 28x28 128->128, uint4 in/out/residual, int4 weights,
    Conv_Add_Relu.  Every output byte of the whole batch against the oracle."""
    require_gpu()
    c = synth.conv3x3_4bit(seed=0)
    x, w, res = conv_codes(c)
    got = gpu_conv(c, x, w, res)
    want = to_bytes(oracle_conv(c, x, w, res), c.y_type)
    assert_bytes_equal(got, want, "conv3x3_4bit")
    codes = O.unpack(got, O.UINT4)
    # ReLU clamps at Z_out, so exactly the codes Z_out..15 can occur: all of them should
    assert set(np.unique(codes)) == set(range(c.z_out, 16)) and (codes == 15).mean() < 0.01
