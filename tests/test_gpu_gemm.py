"""GPU parity of the quantized GEMM (the conv kernel with a 1x1 gather)."""
import numpy as np
import pytest

import oracle as O
from integer_quantized_nn_amd import synth
from parity_util import (assert_bytes_equal, gemm_codes, gpu_gemm, oracle_gemm, otype, require_gpu,
                         to_bytes)

pytestmark = pytest.mark.gpu


def test_gemm_int8_256_full():
    """256^3 int8 symmetric GEMM, per-tensor scales (0.02, 0.01, 0.5), int8 out."""
    require_gpu()
    c = synth.gemm_int8_256(seed=0)
    a, b = gemm_codes(c)
    got = gpu_gemm(c, a, b)
    want = to_bytes(oracle_gemm(c, a, b), c.c_type)
    assert_bytes_equal(got, want, "gemm 256")


@pytest.mark.parametrize("m,n,k,at,bt,ct,epi", [
    (1, 64, 64, synth.INT8, synth.INT8, synth.INT8, synth.EPI_NONE),
    (197, 192, 320, synth.UINT8, synth.INT8, synth.INT8, synth.EPI_NONE),
    (333, 256, 1024, synth.UINT8, synth.INT8, synth.UINT8, synth.EPI_RELU),
    (130, 96, 48, synth.UINT8, synth.INT8, synth.INT32, synth.EPI_RAW),
    (77, 64, 256, synth.UINT4, synth.INT4, synth.UINT4, synth.EPI_RELU),
    (50, 32, 37, synth.UINT8, synth.INT8, synth.INT8, synth.EPI_NONE),
])
def test_gemm_shapes(m, n, k, at, bt, ct, epi):
    require_gpu()
    rng = np.random.default_rng(m * 7 + n * 3 + k)
    alo, ahi = O.qrange(otype(at))
    blo, bhi = O.qrange(otype(bt))
    a = rng.integers(alo, ahi + 1, size=(m, k)).astype(np.int32)
    b = rng.integers(blo, bhi + 1, size=(n, k)).astype(np.int32)
    c = synth.GemmCase("g", None, a, None, b, rng.normal(0, 1, n).astype(np.float32), np.float32(0.01),
                       (int(rng.integers(alo, ahi + 1)) if at in (synth.UINT8, synth.UINT4) else 0),
                       rng.uniform(0.001, 0.01, n).astype(np.float32), np.float32(0.2 * np.sqrt(k) * 0.01),
                       3 if ct in (synth.UINT8, synth.UINT4) else 0, at, bt, ct, epi)
    got = gpu_gemm(c, a, b)
    want = to_bytes(oracle_gemm(c, a, b), ct)
    assert_bytes_equal(got, want, "gemm %dx%dx%d" % (m, n, k))


def test_gemm_epilogue_fma_canaries():
    # Accumulators and residuals for which a fused multiply-add would round to a
    # different code than the two rounded products and the rounded sum.  A has two
    # non-zero columns, B row 0 is [127, 1, 0...], so acc = 127*a0 + a1 hits each
    # chosen value exactly; M = 0.00731 and M_res = 0.0413 are exact in binary32.
    torch = require_gpu()
    from integer_quantized_nn_amd.layers import QGemm
    m_f, mres_f = np.float32(0.00731), np.float32(0.0413)
    acc, r = np.meshgrid(np.arange(-15000, 15000, dtype=np.int64), np.arange(256, dtype=np.int64))
    acc, r = acc.ravel(), r.ravel()
    t_unf = acc.astype(np.float32) * m_f + (r - 9).astype(np.float32) * mres_f
    t_fus = (acc * np.float64(m_f) + (r - 9) * np.float64(mres_f)).astype(np.float32)
    sel = np.nonzero((np.rint(t_unf) != np.rint(t_fus)) & (np.abs(t_unf) < 120))[0]
    assert sel.size >= 5
    acc, r = acc[sel], r[sel]
    a0 = np.floor_divide(acc, 127)
    a1 = acc - 127 * a0
    A = np.zeros((sel.size, 16), np.int32)
    A[:, 0], A[:, 1] = a0, a1
    Bm = np.zeros((16, 16), np.int32)
    Bm[0, 0], Bm[0, 1] = 127, 1
    res = np.zeros((sel.size, 16), np.int32)
    res[:, 0] = r
    g = QGemm(sel.size, 16, 16, synth.INT8, synth.INT8, synth.INT8, synth.EPI_ADD, 0, 0, to_bytes(Bm, 0), None,
              np.float32(1.0), np.float32(0.00731), np.float32(1.0), res_type=synth.UINT8, z_res=9,
              s_res=np.float32(0.0413))
    out = g(torch.from_numpy(to_bytes(A, 0)).cuda(), res=torch.from_numpy(to_bytes(res, 1)).cuda())
    got = O.unpack(out.cpu().numpy(), O.INT8)[:, 0]
    want = O.requant(acc[:, None], m_f, O.EPI_ADD, 0, O.INT8, res=r[:, None].astype(np.int32), z_res=9,
                     m_res=mres_f)[:, 0]
    assert np.array_equal(got, want)
    assert np.array_equal(got, np.rint(t_unf[sel]).astype(np.int32))


def test_vitl_fc1_full_size():
    """ViT-L fc1: 12608x1024 -> 4096, uint8 activations with outlier channels, int8
    per-channel weights, per-channel requant to int8.  Every output byte against the
    oracle (53 G multiply-adds on the host cores)."""
    require_gpu()
    c = synth.vitl_fc1(seed=0)
    a, b = gemm_codes(c)
    got = gpu_gemm(c, a, b)
    want = to_bytes(oracle_gemm(c, a, b), c.c_type)
    assert_bytes_equal(got, want, "vitl fc1")
    q = O.unpack(got, O.INT8)
    assert len(np.unique(q)) >= 64 and (np.abs(q) >= 127).mean() < 0.01


@pytest.mark.parametrize("n,k,sparse", [(4096, 2048, False), (8192, 2048, False), (3328, 2048, False),
                                        (8192, 2048, True)],
                         ids=["w8MB_4groups", "w16MB_8groups", "odd_tiles_1group", "sp10MB_8groups"])
def test_gemm_xcd_channel_groups(n, k, sparse):
    """Layers whose weights exceed 2 MB split their channel tiles across the XCDs (2, 4
    or 8 groups, so an XCD's share is at most 2 MB; a tile count the split does not
    divide keeps one group).  Every output byte of a 300-row GEMM against the oracle."""
    require_gpu()
    import torch
    from integer_quantized_nn_amd import binding as IB
    from integer_quantized_nn_amd.layers import QGemm
    g = synth.vitl_fc1(seed=n + k, m=300, k=k, n=n, sparse_2of4=sparse)
    a = O.quantize(g.a, g.s_a, g.z_a, O.UINT8)
    b = O.quantize(g.b, g.s_b, 0, O.INT8, axis=0)
    layer = QGemm(300, n, k, g.a_type, IB.INT8_2OF4 if sparse else IB.INT8, g.c_type, g.epi, g.z_a, g.z_out,
                  to_bytes(b, g.b_type), g.bias, g.s_a, g.s_b, g.s_out)
    got = layer(torch.from_numpy(to_bytes(a, g.a_type)).cuda())
    torch.cuda.synchronize()
    assert_bytes_equal(got.cpu().numpy(), to_bytes(oracle_gemm(g, a, b), g.c_type), "gemm 300x%dx%d" % (k, n))
