"""2:4-sparse weights (IQNN_INT8_2OF4) on the host, no GPU needed: prepack keeps two
codes per group of four K positions with their positions, the kept codes decode back
to the dense weights, the folded bias and multipliers equal those of the same codes
as dense INT8, and weights or layers the sparse path does not take are rejected
before any launch."""
import ctypes
import os

import numpy as np
import pytest

from integer_quantized_nn_amd import binding as B
from integer_quantized_nn_amd import synth
from parity_util import to_bytes


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libiqnn.so is not built (run __graft_entry__.build())")
    return B.lib()


def conv_desc(**kw):
    d = B.ConvDesc()
    base = dict(n=2, h=9, w=9, c_in=64, c_out=96, kh=3, kw=3, stride_h=1, stride_w=1, pad_h=1, pad_w=1,
                x_type=B.UINT8, w_type=B.INT8_2OF4, y_type=B.UINT8, res_type=B.UINT8, epilogue=B.EPI_RELU,
                z_in=7, z_out=3, z_res=0, z_w=0)
    base.update(kw)
    for k, v in base.items():
        setattr(d, k, v)
    return d


def sparse_codes(rng, c_out, k, full_groups=True):
    """int8 codes with at most two nonzero codes per group of four along K; some groups
    keep fewer than two (zeros among the kept, or all-zero groups)."""
    w = rng.integers(-128, 128, size=(c_out, k)).astype(np.int32)
    g = w.reshape(c_out, k // 4, 4)
    for row in g:
        for grp in row:
            drop = rng.choice(4, 2 if full_groups or rng.random() < 0.7 else 4, replace=False)
            grp[drop] = 0
    return g.reshape(c_out, k)


def packed_rows(c_out):
    """Packed row of each output channel (the MFMA accumulator permutation inside
    32-channel blocks: channel 32b + 16h + 4j + r sits at row 32b + 8j + 4h + r)."""
    rows = []
    for c in range(c_out):
        b, r32 = divmod(c, 32)
        h, j, r = r32 // 16, (r32 // 4) % 4, r32 % 4
        rows.append(32 * b + 8 * j + 4 * h + r)
    return np.array(rows)


def decode(buf, c_out, k):
    """Dense [c_out][k] codes and the raw positions from a 2:4 packed layer: blocks of
    5120 bytes per (128-row channel tile, 64-K stage), tile-major; in a block, 128 rows
    of 32 bytes of kept codes (K half h of row r at 16-byte slot h ^ ((r >> 3) & 1)),
    then 128 rows of two 32-bit position words."""
    ocp = (c_out + 255) // 256 * 256
    kp = (k + 63) // 64 * 64
    nst = kp // 64
    w_off = 8 * ocp + 256
    blocks = buf[w_off:w_off + ocp * kp * 5 // 8].reshape(ocp // 128, nst, 5120)
    codes = blocks[:, :, :4096].view(np.int8).reshape(ocp // 128, nst, 128, 2, 16).astype(np.int32)
    words = blocks[:, :, 4096:].copy().view(np.uint32).reshape(ocp // 128, nst, 128, 2).astype(np.int64)
    dense = np.zeros((ocp, kp), np.int32)
    p_all = np.zeros((ocp, kp // 4, 2), np.int64)
    for t in range(ocp // 128):
        for st in range(nst):
            for r in range(128):
                for h in range(2):
                    vals = codes[t, st, r, h ^ ((r >> 3) & 1)]
                    word = words[t, st, r, h]
                    for g in range(8):
                        for q in range(2):
                            pos = (word >> (4 * g + 2 * q)) & 3
                            dense[128 * t + r, st * 64 + h * 32 + 4 * g + pos] += vals[2 * g + q]
                            p_all[128 * t + r, (st * 64 + h * 32) // 4 + g, q] = pos
    rows = packed_rows(c_out)
    return dense[rows][:, :k], p_all[rows], buf[:4 * ocp].view(np.int32)[:c_out], \
        buf[4 * ocp:8 * ocp].view(np.float32)[:c_out]


def _pack(d, w, bias, s_w, s_out=0.05, s_res=1.0):
    buf = np.zeros(B.iqnn_qconv_packed_size(d), np.uint8)
    B.iqnn_qconv_prepack_host(d, to_bytes(w, B.INT8), bias, np.float32(0.02), s_w, np.size(s_w) > 1,
                              np.float32(s_out), np.float32(s_res), buf)
    return buf


@pytest.mark.parametrize("c_out,kh,c_in,full", [(96, 3, 64, True), (300, 1, 128, False), (32, 1, 64, False)])
def test_prepack_2of4_decodes_to_the_dense_codes(lib, c_out, kh, c_in, full):
    rng = np.random.default_rng(c_out + c_in)
    k = kh * kh * c_in
    w = sparse_codes(rng, c_out, k, full)
    s_w = rng.uniform(0.001, 0.01, c_out).astype(np.float32)
    bias = rng.normal(0, 0.3, c_out).astype(np.float32)
    d = conv_desc(c_out=c_out, kh=kh, kw=kh, c_in=c_in, pad_h=kh // 2, pad_w=kh // 2)
    buf = _pack(d, w.reshape(c_out, kh, kh, c_in), bias, s_w)
    dense, pos, bias_i32, mult = decode(buf, c_out, k)
    assert np.array_equal(dense, w)
    # the two positions of a group are distinct and increasing
    assert np.all(pos[..., 0] < pos[..., 1])
    # bias fold and multipliers are those of the same codes as dense INT8
    dd = conv_desc(c_out=c_out, kh=kh, kw=kh, c_in=c_in, pad_h=kh // 2, pad_w=kh // 2, w_type=B.INT8)
    ref = _pack(dd, w.reshape(c_out, kh, kh, c_in), bias, s_w)
    ocp = (c_out + 255) // 256 * 256
    assert np.array_equal(bias_i32, ref[:4 * ocp].view(np.int32)[:c_out])
    assert np.array_equal(mult.view(np.uint32), ref[4 * ocp:8 * ocp].view(np.uint32)[:c_out])


def test_prepack_2of4_gemm(lib):
    rng = np.random.default_rng(5)
    m, n, k = 100, 64, 192
    w = sparse_codes(rng, n, k)
    g = B.GemmDesc()
    g.m, g.n, g.k = m, n, k
    g.a_type, g.b_type, g.c_type, g.res_type, g.epilogue = B.UINT8, B.INT8_2OF4, B.INT8, B.UINT8, B.EPI_NONE
    g.z_a = 100
    buf = np.zeros(B.iqnn_qgemm_packed_size(g), np.uint8)
    B.iqnn_qgemm_prepack_host(g, to_bytes(w, B.INT8), None, np.float32(0.02), np.full(n, 0.01, np.float32), True,
                              np.float32(0.5), np.float32(1.0), buf)
    dense, _, _, _ = decode(buf, n, k)
    assert np.array_equal(dense, w)


def test_prepack_2of4_rejects_three_nonzero_codes(lib):
    rng = np.random.default_rng(1)
    w = sparse_codes(rng, 96, 576)
    w[37, 4 * 50:4 * 50 + 4] = [3, 0, -2, 9]   # channel 37, K 200..203: three nonzero codes
    d = conv_desc()
    with pytest.raises(B.IqnnError) as ei:
        _pack(d, w.reshape(96, 3, 3, 64), None, np.full(96, 0.01, np.float32))
    assert ei.value.status == 1 and "channel 37" in str(ei.value) and "200" in str(ei.value)


def test_synthetic_pruning_keeps_two_largest(lib):
    rng = np.random.default_rng(0)
    w = rng.standard_normal((8, 64)).astype(np.float32)
    w[0, :4] = [0.5, -0.5, 0.1, 0.5]   # a tie: the earlier ones are kept
    p = synth.prune_2of4(w)
    g, pg = w.reshape(-1, 4), p.reshape(-1, 4)
    assert np.all((pg != 0).sum(axis=1) == 2)
    for a, b in zip(g, pg):
        kept = np.flatnonzero(b)
        assert np.array_equal(b[kept], a[kept])
        assert np.sort(np.abs(a))[2:].sum() == np.abs(a[kept]).sum()
    assert np.array_equal(pg[0], np.float32([0.5, -0.5, 0, 0]))


def test_2of4_layers_the_sparse_path_does_not_take(lib):
    P = ctypes.c_void_p

    def status(**kw):
        return lib.iqnn_qconv_fwd(ctypes.byref(conv_desc(**kw)), P(4096), P(4096), P(4096), P(4096), None)

    assert status(z_w=1) == 1                                          # 2:4 weights are symmetric
    assert status(x_type=B.UINT4, z_in=3, y_type=B.UINT4) == 2          # 4-bit activations
    assert status(c_in=32) == 2                                         # C_in % 64
    assert status(epilogue=B.EPI_RELU | B.EPI_INT_REQUANT) == 2         # integer requantization
    assert status(epilogue=B.EPI_ADD_RELU, res_type=B.UINT4, z_res=1) == 2   # 4-bit residual
    assert status(epilogue=B.EPI_ADD_RELU, c_out=72) == 2              # residual with C_out % 16
