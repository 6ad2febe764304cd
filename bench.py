"""Benchmark of the quantized conv / GEMM hot path on one MI355X.

Default workload: the ResNet-50 conv trunk at batch 256 (224x224x3 input), one
step = quantize the fp32 input (resident in HBM) -> 53 fused quantized convs
(Conv_Relu / Conv / Conv_Add_Relu; the stem with the max pooling fused; where a
64-channel block ends, its last conv and the next block's first conv as one launch)
-> dequantize the output.  `value` is whole-step throughput in TOPS (2*M*N*K of every
conv, K = KH*KW*C_in without padding) over exactly --steps timed steps.

The step runs as three HIP graphs (quantize, the convs, dequantize) replayed back
to back with a pair of HIP events around the conv graph of every timed step, on the
launch stream.  The JSON line carries
  roofline      the implicit-GEMM conv kernel over its launches in the timed steps:
                algorithmic bytes (or ops) per launch / (conv-graph time per step /
                launches per step), against the MI355X peak that binds at the
                aggregate arithmetic intensity;
  layer_classes the same per class of layer (fused stem + pooling, HBM-bound,
                MFMA-bound by arithmetic intensity), each layer timed alone from a
                graph of back-to-back launches after the timed steps;
  calibration   what this GPU reaches in the same run: a register-only int8 MFMA
                loop, an empty launch, a device-to-device copy;
  configs       the four single-layer workloads (256^3 int8 GEMM, ResNet 3x3 int8
                conv, 4-bit conv, ViT-L fc1), each timed, with its roofline and the
                CPU oracle timed on its full output and compared with it byte for byte;
  cpu_baseline  the CPU oracle (plain C, OpenMP) on whole images of the trunk step for
                a bounded time on all host cores (and one image on one core), scaled
                to TOPS; the GPU output of those images is compared byte for byte.

Other workloads (--workload) time a single layer.
Only one GPU is supported: --gpus N with N > 1 exits with a message.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "int8/int4 quantized conv+GEMM TOPS and % of int8 MFMA peak, bit-exact"
PEAK_INT8_OPS = 5.0e15      # MI355X dense int8 MFMA, ops/s
PEAK_HBM = 8.0e12           # MI355X HBM3E, bytes/s
PEAK_FP6_OPS = 10.1e15      # MI355X dense FP6 MFMA, ops/s
RIDGE = PEAK_INT8_OPS / PEAK_HBM
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "qconv_resnet50_trunk_b256_traffic.md")
CONFIG_WORKLOADS = ["gemm_int8_256", "conv3x3_int8", "conv3x3_4bit", "vitl_fc1"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_tag():
    import hashlib
    h = hashlib.sha256()
    for f in ("qconv.hip", "iqnn_internal.h"):
        with open(os.path.join(ROOT, "integer_quantized_nn_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch from committed rocprofv3 PMC runs, if the kernel source is
    unchanged since they were taken; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    tag = kernel_source_tag()
    for line in open(TRAFFIC_FILE):
        if line.startswith("TRAFFIC "):
            rec = json.loads(line[len("TRAFFIC "):])
            if rec.get("workload") == workload and rec.get("kernel_source") == tag:
                return rec.get("bytes_per_launch")
    return None


def traffic_from_dbs(fetch_db, write_db, workload):
    """Per-launch HBM traffic of the conv kernels from two rocprofv3 --pmc databases (FETCH_SIZE,
    WRITE_SIZE; KiB per dispatch), each scaled by what the same counter reads for the
    calibration copy (--calib-copy-mib) whose true byte count is known."""
    import sqlite3

    def per_dispatch(path):
        cur = sqlite3.connect(path).cursor()
        return cur.execute("select dispatch_id, kernel_name, value from counters_collection").fetchall()

    out = {}
    for tag, path in (("fetch", fetch_db), ("write", write_db)):
        rows = per_dispatch(path)
        copies = [v for (_, n, v) in rows if "copyBuffer" in n or "copy" in n.lower()]
        calib_kib = max(copies)
        q = [v for (_, n, v) in rows if "qconv_" in n]
        out[tag] = (calib_kib, float(np.mean(q)), len(q))
    return out


def roofline(ops, nbytes, seconds, peak_ops=PEAK_INT8_OPS):
    """Roofline record of `ops` operations moving `nbytes` algorithmic bytes in `seconds`:
    bound by the arithmetic intensity against the ridge of the given peak."""
    if ops / nbytes < peak_ops / PEAK_HBM:
        r = {"bound": "hbm", "achieved": nbytes / seconds / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    else:
        r = {"bound": "mfma", "achieved": ops / seconds / 1e12, "peak": peak_ops / 1e12, "unit": "TOPS"}
    r["frac"] = r["achieved"] / r["peak"]
    return r


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------- calibration


def spin_time(torch, run, reps):
    """Average seconds per launch of `run`: a spin kernel holds the stream while `reps`
    launches are enqueued, then one pair of HIP events brackets them back to back (an
    event between launches would add its own few microseconds)."""
    stream = torch.cuda.current_stream()
    run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run()
    torch.cuda.synchronize()
    host = time.perf_counter() - t0
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    torch.cuda._sleep(1 << 20)
    b.record(stream)
    torch.cuda.synchronize()
    s_per_cycle = a.elapsed_time(b) * 1e-3 / (1 << 20)
    hold = 2.0 * reps * host + 2e-3
    t_begin, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    torch.cuda._sleep(int(hold / s_per_cycle))
    t0 = time.perf_counter()
    t_begin.record(stream)
    for _ in range(reps):
        run()
    t_end.record(stream)
    enqueued = time.perf_counter() - t0
    torch.cuda.synchronize()
    if a.elapsed_time(t_begin) * 1e-3 < enqueued:
        log("warning: the spin kernel ended before every timed launch was enqueued")
    return t_begin.elapsed_time(t_end) * 1e-3 / reps


def measure_copy_gbs(torch, mib=1024, reps=5):
    """Best rate of a device-to-device copy (bytes read + written per second, GB/s):
    the HBM rate a plain streaming kernel reaches on this GPU."""
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    best = float("inf")
    for _ in range(reps + 1):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b) * 1e-3)
    del src, dst
    return 2.0 * (mib << 20) / best / 1e9


def calibrate(torch):
    """Register-only int8 MFMA rate (2 workgroups of 4 waves per CU), empty-launch
    duration and copy rate of this GPU, measured now."""
    from integer_quantized_nn_amd import binding as B
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = 2 * n_cu, 4000
    sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    best = float("inf")
    for _ in range(4):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        B.iqnn_probe_mfma_rate(iters, blocks, sink)
        b.record()
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b) * 1e-3)
    mfma_ops = blocks * 4 * iters * 8 * 2 * 32 * 32 * 32
    empty = spin_time(torch, lambda: B.iqnn_probe_empty(), 200)
    return {"mfma_int8_tops": mfma_ops / best / 1e12,
            "mfma_int8_frac_of_spec": mfma_ops / best / PEAK_INT8_OPS,
            "mfma_note": "register-only loop of v_mfma_i32_32x32x32_i8, 8 accumulators per wave, "
                         "2 workgroups of 4 waves per CU",
            "empty_launch_us": empty * 1e6,
            "copy_gbs": measure_copy_gbs(torch),
            "compute_units": n_cu}


# --------------------------------------------------------- single layers


def make_layer(torch, wl, cfg=None):
    """One single-layer workload on the GPU plus the oracle's view of it.  Returns a dict
    with run(i, out), ins (input sets), out_shape / out_type, ops, nbytes, peak and
    oracle() -> expected output bytes of the full output (oracle codes from the
    oracle's own quantization of the same float data, never from the GPU)."""
    from integer_quantized_nn_amd import binding as IB
    from integer_quantized_nn_amd import synth
    from integer_quantized_nn_amd.layers import QConv, QGemm, quantize

    def oracle_names():
        # the oracle (the CPU baseline leg only) numbers types and epilogues on its own
        import oracle as O
        ot = {synth.INT8: O.INT8, synth.UINT8: O.UINT8, synth.INT4: O.INT4, synth.UINT4: O.UINT4}
        oe = {synth.EPI_NONE: O.EPI_NONE, synth.EPI_RELU: O.EPI_RELU, synth.EPI_ADD: O.EPI_ADD,
              synth.EPI_ADD_RELU: O.EPI_ADD_RELU}
        return O, ot, oe
    fp6 = wl == "conv3x3_4bit_fp6"   # the 4-bit layer on the FP6 MFMA (weights and activations as BF6)
    if fp6:
        cfg = (19, 0)
    rec = {"peak_ops": PEAK_FP6_OPS if fp6 else PEAK_INT8_OPS, "dtype": "bf6" if fp6 else "int8", "oracle": None}
    conv_wls = ("conv3x3_int8", "conv3x3_4bit", "conv3x3_4bit_fp6", "conv3x3_uint8w", "conv3x3_intrq",
                "conv3x3_2of4", "resnet50_l3_conv3x3", "resnet50_l3_conv3x3_intrq", "resnet50_l3_conv3x3_s8",
                "conv1x1_int8", "conv1x1_intrq")
    if wl in conv_wls:
        if wl.startswith("resnet50_l3_conv3x3"):   # the trunk's stage-3 3x3 layer: 256 x 14x14, 256 -> 256
            # _s8: signed 8-bit activation and output codes, the trunk's stored form (no sign flip)
            t8 = synth.INT8 if wl.endswith("_s8") else synth.UINT8
            c = synth.conv_case(31, 256, 14, 14, 256, 256, 3, 1, 1, t8, synth.INT8, t8, synth.EPI_RELU,
                                name="l3_conv3x3")
        elif wl.startswith("conv1x1"):   # the trunk's stage-1 expanding 1x1 layer: 256 x 56x56, 64 -> 256
            c = synth.conv_case(33, 256, 56, 56, 64, 256, 1, 1, 0, synth.UINT8, synth.INT8, synth.UINT8,
                                synth.EPI_RELU, name="conv1x1")
        else:
            c = synth.conv3x3_4bit() if wl.startswith("conv3x3_4bit") else synth.conv3x3_int8()
        if wl == "conv3x3_2of4":   # float weights magnitude-pruned to 2:4 along the input channels
            c.w = synth.prune_2of4(c.w)
        n, h, w, ci = c.x.shape
        co = c.c_out
        w_type, s_w, z_w = c.w_type, c.s_w, 0
        if wl == "conv3x3_uint8w":   # asymmetric weights: per-tensor min-max UINT8 codes
            w_type = synth.UINT8
            s_w, z_w = synth.minmax_qparams(c.w.min(), c.w.max(), w_type)
            wq = quantize(torch.from_numpy(c.w).cuda(), s_w, z_w, w_type).cpu().numpy()
        else:
            wq = quantize(torch.from_numpy(c.w).cuda(), c.s_w, 0, c.w_type, axis=0).cpu().numpy()
        epi = c.epi | (IB.EPI_INT_REQUANT if wl.endswith("intrq") else 0)
        lib_w_type = IB.INT8_2OF4 if wl == "conv3x3_2of4" else w_type
        kk = c.w.shape[1]
        layer = QConv(n, h, w, ci, co, kk, c.stride, c.pad, c.x_type, lib_w_type, c.y_type, epi, c.z_in, c.z_out,
                      wq, c.bias, c.s_in, s_w, c.s_out, res_type=c.res_type, z_res=c.z_res, s_res=c.s_res, z_w=z_w)
        xd = quantize(torch.from_numpy(c.x).cuda(), c.s_in, c.z_in, c.x_type)
        rd = quantize(torch.from_numpy(c.res).cuda(), c.s_res, c.z_res, c.res_type) if c.res is not None else None
        oh, ow = layer.out_shape[1:3]
        w_bytes = co * kk * kk * ci // (2 if c.w_type in (synth.UINT4, synth.INT4) else 1)
        if wl == "conv3x3_2of4":
            w_bytes = w_bytes * 5 // 8   # kept codes + positions
        y_bytes = n * oh * ow * co // (2 if c.y_type in (synth.UINT4, synth.INT4) else 1)
        rec.update(ops=c.ops(n, h, w), nbytes=xd.numel() + w_bytes + y_bytes + (rd.numel() if rd is not None else 0),
                   ins=[(xd, rd)], out_shape=layer.out_shape, out_type=c.y_type,
                   run=lambda i, o: layer(rec["ins"][i][0], res=rec["ins"][i][1], out=o, cfg=cfg))
        if wl in ("conv3x3_int8", "conv3x3_4bit", "resnet50_l3_conv3x3"):
            def oracle_out():
                O, OT, OE = oracle_names()
                xo = O.quantize(c.x, c.s_in, c.z_in, OT[c.x_type])
                wo = O.quantize(c.w, c.s_w, 0, OT[c.w_type], axis=0)
                ro = O.quantize(c.res, c.s_res, c.z_res, OT[c.res_type]) if c.res is not None else None
                t0 = time.perf_counter()
                y = O.qconv(xo, c.z_in, c.s_in, wo, c.s_w, c.bias, c.s_out, c.z_out, OT[c.y_type], OE[c.epi],
                            c.stride, c.pad, ro, c.s_res, c.z_res)
                return O.pack(y, OT[c.y_type]), time.perf_counter() - t0
            rec["oracle"] = oracle_out
    elif wl == "resnet50_stem_pool":
        # the trunk's stem with its max pooling fused: 256 x 224x224x3 -> 7x7/2 conv, 64
        # channels, ReLU -> 3x3/2 pad 1 pooling; the input as the trunk feeds it (padded
        # 4-channel offset codes q - 128 from iqnn_quantize_pad)
        from integer_quantized_nn_amd.layers import quantize_pad
        c = synth.conv_case(41, 256, 224, 224, 3, 64, 7, 2, 3, synth.UINT8, synth.INT8, synth.UINT8,
                            synth.EPI_RELU, name="stem")
        n, h, w, ci = c.x.shape
        wq = quantize(torch.from_numpy(c.w).cuda(), c.s_w, 0, c.w_type, axis=0).cpu().numpy()
        wq = np.pad(wq.reshape(64, 7, 7, ci), ((0, 0), (0, 0), (0, 0), (0, 1)))
        layer = QConv(n, h + 6, w + 6, 4, 64, 7, 2, 0, IB.INT8, IB.INT8, IB.INT8, c.epi, c.z_in - 128,
                      c.z_out - 128, wq, c.bias, c.s_in, c.s_w, c.s_out)
        xd = quantize_pad(torch.from_numpy(c.x).cuda(), c.s_in, c.z_in - 128, IB.INT8, 3, 4)
        pshape = layer.pool_shape(3, 2, 1)
        rec.update(ops=c.ops(n, h, w), nbytes=xd.numel() + 64 * 7 * 7 * 4 + int(np.prod(pshape)),
                   ins=[(xd, None)], out_shape=pshape, out_type=synth.INT8,
                   run=lambda i, o: layer.conv_maxpool(rec["ins"][i][0], out=o))
    elif wl == "resnet50_l1_pair":
        # the hand-off between two stage-1 bottleneck blocks of the trunk, batch 256 on
        # 56x56: 1x1 64 -> 256 with the residual add and ReLU, then the next block's 1x1
        # 256 -> 64 with ReLU on its output, one launch (iqnn_qconv_pair_fwd); the timed
        # output is the second conv's, the first's is written to its own buffer
        from integer_quantized_nn_amd.layers import conv_pair, empty_codes
        U8, I8 = synth.UINT8, synth.INT8
        a = synth.conv_case(35, 256, 56, 56, 64, 256, 1, 1, 0, U8, I8, U8, synth.EPI_ADD_RELU, res_type=U8,
                            name="l1_c3")
        b = synth.conv_case(36, 256, 56, 56, 256, 64, 1, 1, 0, U8, I8, U8, synth.EPI_RELU, name="l1_c1")
        wa = quantize(torch.from_numpy(a.w).cuda(), a.s_w, 0, I8, axis=0).cpu().numpy()
        wb = quantize(torch.from_numpy(b.w).cuda(), b.s_w, 0, I8, axis=0).cpu().numpy()
        conv_a = QConv(256, 56, 56, 64, 256, 1, 1, 0, U8, I8, U8, a.epi, a.z_in, a.z_out, wa, a.bias, a.s_in, a.s_w,
                       a.s_out, res_type=U8, z_res=a.z_res, s_res=a.s_res)
        conv_b = QConv(256, 56, 56, 256, 64, 1, 1, 0, U8, I8, U8, b.epi, a.z_out, b.z_out, wb, b.bias, a.s_out,
                       b.s_w, b.s_out)
        xd = quantize(torch.from_numpy(a.x).cuda(), a.s_in, a.z_in, U8)
        rd = quantize(torch.from_numpy(a.res).cuda(), a.s_res, a.z_res, U8)
        ya = empty_codes(conv_a.out_shape, U8)
        m = 256 * 56 * 56
        rec.update(ops=2 * m * 256 * 64 * 2, nbytes=m * (64 + 256 + 256 + 64) + 2 * 256 * 64,
                   ins=[(xd, rd)], out_shape=conv_b.out_shape, out_type=U8,
                   run=lambda i, o: conv_pair(conv_a, conv_b, rec["ins"][i][0], res=rec["ins"][i][1], out_a=ya,
                                              out_b=o))
    elif wl in ("vitl_fc1", "vitl_fc1_2of4", "gemm_int8_256"):
        sparse = wl == "vitl_fc1_2of4"   # weights magnitude-pruned to 2:4 along K, on the sparse MFMA
        g = synth.vitl_fc1(sparse_2of4=sparse) if wl.startswith("vitl") else synth.gemm_int8_256()
        m, n, k = g.shape
        if g.b_codes is not None:   # int8 codes drawn directly: their two's-complement bytes
            b_bytes = np.ascontiguousarray(g.b_codes.astype(np.int8)).view(np.uint8)
            a_dev = torch.from_numpy(np.ascontiguousarray(g.a_codes.astype(np.int8)).view(np.uint8)).cuda()
        else:
            b_bytes = quantize(torch.from_numpy(g.b).cuda(), g.s_b, 0, g.b_type, axis=0).cpu().numpy()
            a_dev = quantize(torch.from_numpy(g.a).cuda(), g.s_a, g.z_a, g.a_type)
        layer = QGemm(m, n, k, g.a_type, IB.INT8_2OF4 if sparse else g.b_type, g.c_type, g.epi, g.z_a, g.z_out,
                      b_bytes, g.bias, g.s_a, g.s_b, g.s_out)
        # ops: the dense problem's 2*M*N*K (with 2:4 weights half the products are with zero
        # codes and the kernel skips them); bytes: 2:4 weights move kept codes + positions
        rec.update(ops=2 * m * n * k, nbytes=m * k + (n * k // 2 + n * k // 8 if sparse else n * k) + m * n,
                   ins=[(a_dev, None)], out_shape=layer.out_shape, out_type=g.c_type,
                   run=lambda i, o: layer(rec["ins"][i][0], out=o, cfg=cfg))
        if not sparse:
            def oracle_out():
                O, OT, OE = oracle_names()
                ao = g.a_codes if g.a_codes is not None else O.quantize(g.a, g.s_a, g.z_a, OT[g.a_type])
                bo = g.b_codes if g.b_codes is not None else O.quantize(g.b, g.s_b, 0, OT[g.b_type], axis=0)
                t0 = time.perf_counter()
                y = O.qgemm(ao, g.z_a, g.s_a, bo, g.s_b, g.bias, g.s_out, g.z_out, OT[g.c_type], OE[g.epi])
                return O.pack(y, OT[g.c_type]), time.perf_counter() - t0
            rec["oracle"] = oracle_out
    else:
        raise SystemExit("unknown workload " + wl)
    return rec


def time_layer(torch, L, steps, cold=False):
    """Average seconds per launch of a single-layer workload (spin_time), warm (inputs
    reused) or cold (rotating enough input / output sets, at least 4 and over 256 MB in
    all, that every launch reads and writes HBM rather than the 256 MB Infinity Cache)."""
    from integer_quantized_nn_amd.layers import empty_codes
    n_sets = max(4, -(-(300 << 20) // L["nbytes"])) if cold else 1
    for _ in range(n_sets - 1):
        L["ins"].append(tuple(t.clone() if t is not None else None for t in L["ins"][0]))
    outs = [empty_codes(L["out_shape"], L["out_type"]) for _ in range(n_sets)]
    step_no = [0]

    def run():
        i = step_no[0] % n_sets
        step_no[0] += 1
        return L["run"](i, outs[i])

    return spin_time(torch, run, steps), outs[0], n_sets


def config_record(torch, wl, steps):
    """One workload of the configs block: timed on the GPU, its roofline, and the CPU
    oracle timed on its full output and compared with the GPU output byte for byte."""
    L = make_layer(torch, wl)
    avg, out, _ = time_layer(torch, L, steps)
    # the output of the timed launches (the same inputs every launch)
    got = out.cpu().numpy()
    r = {"ops": L["ops"], "algorithmic_bytes": L["nbytes"], "us_per_launch": avg * 1e6,
         "tops": L["ops"] / avg / 1e12, "pct_int8_mfma_peak": L["ops"] / avg / PEAK_INT8_OPS,
         "roofline": roofline(L["ops"], L["nbytes"], avg), "launch": "warm, back-to-back launches"}
    # the CPU baseline leg: the oracle on the same float data, its own quantization
    import oracle as O
    want, t_cpu = L["oracle"]()
    r["bit_exact_vs_oracle"] = bool(np.array_equal(got.reshape(-1), want.reshape(-1)))
    r["cpu_baseline"] = {"value": L["ops"] / t_cpu / 1e12, "unit": "TOPS", "cores": O.num_threads(), "kind": "oracle",
                         "sample": "the full output (%.2f s wall)" % t_cpu}
    return r


def bench_layer(args, torch, cal):
    cfg = (args.tile, args.xcd_groups) if (args.tile >= 0 or args.xcd_groups) else None
    L = make_layer(torch, args.workload, cfg)
    for _ in range(max(args.warmup, 1)):
        L["run"](0, None)
    torch.cuda.synchronize()
    avg, _, n_sets = time_layer(torch, L, args.steps, args.cold)
    roof = roofline(L["ops"], L["nbytes"], avg, L["peak_ops"])
    roof["traffic"] = measured_traffic(args.workload)
    roof["avg_launch_us"] = avg * 1e6
    roof["mfma_frac"] = L["ops"] / avg / L["peak_ops"]
    if cal:
        roof["frac_of_measured_mfma"] = L["ops"] / avg / (cal["mfma_int8_tops"] * 1e12)
    return {"metric": METRIC, "value": L["ops"] / avg / 1e12, "unit": "TOPS", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": avg * 1e3,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": L["dtype"],
            "data": "synthetic",
            "config": {"workload": args.workload, "ops": L["ops"], "algorithmic_bytes": L["nbytes"],
                       "cache": ("cold (%d rotating input/output sets, %.0f MB in all)" % (n_sets, n_sets * L["nbytes"] / 1e6)
                                 if args.cold else "warm (inputs reused)"),
                       **({"tile": args.tile} if args.tile >= 0 else {}),
                       **({"ops_note": "dense-equivalent 2*M*N*K; the 2:4 weights make half of the products "
                                       "zero, which the sparse MFMA skips"} if args.workload.endswith("2of4") else {})},
            "pct_int8_mfma_peak": L["ops"] / avg / PEAK_INT8_OPS, "roofline": roof, "calibration": cal,
            "cpu_baseline": None}


# ---------------------------------------------------------------- trunk


def cpu_baseline_trunk(tr, gpu_final_codes, budget_s):
    """Oracle chain on whole images until ~budget_s of wall time on all host cores, then
    one image on one core; returns the record."""
    import oracle as O
    w = {l.name: O.quantize(l.case.w, l.case.s_w, 0, O.INT8, axis=0) for l in tr.layers}
    per_img_ops = tr.ops() / tr.batch
    final = tr.layers[-1].out
    s_f, z_f = tr.qparams[final]

    def one_image(i):
        x = O.quantize(tr.x[i:i + 1], tr.s_in, tr.z_in, O.UINT8)
        acts = {"input": x}
        for layer in tr.layers:
            c = layer.case
            res = acts[layer.res_src] if layer.res_src is not None else None
            acts[layer.out] = O.qconv(acts[layer.src], c.z_in, c.s_in, w[layer.name], c.s_w, c.bias, c.s_out,
                                      c.z_out, O.UINT8, c.epi, c.stride, c.pad, res, c.s_res, c.z_res)
            if layer.name == "stem":
                acts["pool"] = O.maxpool2d(acts["stem"], 3, 2, 1)
        O.dequantize(acts[final], s_f, z_f)
        return np.array_equal(O.pack(acts[final], O.UINT8)[0], gpu_final_codes[i])

    cores = O.num_threads()
    t0 = time.perf_counter()
    n_img, exact = 0, True
    while n_img < tr.batch:
        exact = one_image(n_img) and exact
        n_img += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    O.set_num_threads(1)
    t1 = time.perf_counter()
    exact = one_image(tr.batch - 1) and exact
    dt1 = time.perf_counter() - t1
    O.set_num_threads(cores)
    return {"value": per_img_ops * n_img / dt / 1e12, "unit": "TOPS", "cores": cores, "kind": "oracle",
            "sample": "%d of %d images through the whole step (quantize, 53 convs, max pooling, dequantize) on "
                      "%d threads, %.1f s wall; image %d on 1 thread, %.1f s; weight quantization excluded"
                      % (n_img, tr.batch, cores, dt, tr.batch - 1, dt1),
            "value_1_thread": per_img_ops / dt1 / 1e12, "cpu_model": cpu_model(),
            "bit_exact_vs_gpu": bool(exact)}


def bench_trunk(args, torch, cal):
    from integer_quantized_nn_amd import synth
    from integer_quantized_nn_amd.resnet50 import QuantResNet50Trunk

    t0 = time.perf_counter()
    sparse = args.workload == "resnet50_trunk_2of4"   # 2:4-pruned weights after the stem
    tr = synth.resnet50_trunk(seed=0, batch=args.batch, sparse_2of4=sparse)
    log("synthetic trunk ready in %.1f s" % (time.perf_counter() - t0))
    # uint8 activation codes stored as int8 bytes q - 128 (zero points Z - 128): the same
    # trunk byte for byte up to the sign bit, with no per-fragment sign flip in the kernels
    net = QuantResNet50Trunk(tr, offset_codes=True, sparse_2of4=sparse)
    wl_name = ("resnet50_trunk_2of4_b%d" if sparse else "resnet50_trunk_b%d") % args.batch
    x = torch.from_numpy(tr.x).cuda()
    torch.cuda.synchronize()
    conv_launches = [l for l in net.launches() if l[0].startswith("qconv:")]
    n_conv = len(conv_launches)
    conv_ops = np.array([l[1] for l in conv_launches], np.float64)
    conv_bytes = np.array([l[2] for l in conv_launches], np.float64)
    step_ops = int(conv_ops.sum())
    log("prepacked %d convs; %.1f GOP per step" % (n_conv, step_ops / 1e9))

    for _ in range(args.warmup):
        net.step(x)
    torch.cuda.synchronize()
    g_quant, g_conv, g_deq = net.capture_parts(x)
    for _ in range(args.warmup):
        g_quant.replay()
        g_conv.replay()
        g_deq.replay()
    torch.cuda.synchronize()

    # ---- the timed region: exactly --steps steps, events around each step's conv graph
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(args.steps):
        g_quant.replay()
        ev[s][0].record()
        g_conv.replay()
        ev[s][1].record()
        g_deq.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps
    conv_s = np.array([a.elapsed_time(b) * 1e-3 for (a, b) in ev])   # conv graph seconds per step
    avg_launch = conv_s.mean() / n_conv

    roof = roofline(conv_ops.sum(), conv_bytes.sum(), conv_s.mean())
    roof["achieved"] = (conv_bytes.mean() / avg_launch / 1e9 if roof["bound"] == "hbm"
                        else conv_ops.mean() / avg_launch / 1e12)
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(wl_name)
    roof["kernel"] = ("qconv (qconv_stem_pool / qconv_direct3x3 / qconv_stream; %d launches per step, "
                      "one HIP graph)" % n_conv)
    roof["algorithmic_bytes_per_launch"] = conv_bytes.mean()
    roof["algorithmic_ops_per_launch"] = conv_ops.mean()
    roof["avg_launch_us"] = avg_launch * 1e6
    roof["duration_source"] = "HIP events around the conv graph of every timed step / launches per step"
    roof["mfma_frac"] = conv_ops.mean() / avg_launch / PEAK_INT8_OPS
    roof["frac_of_measured_mfma"] = conv_ops.mean() / avg_launch / (cal["mfma_int8_tops"] * 1e12)
    if roof["bound"] == "hbm":   # the same bytes against what a plain copy reaches on this GPU
        roof["frac_of_measured_copy"] = roof["achieved"] / cal["copy_gbs"]

    # ---- after the timed region: each conv alone, a graph of back-to-back launches
    reps = 8
    per_layer = np.zeros(n_conv)
    for i in range(n_conv):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                net.launch_unit(i)
        g.replay()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            best = min(best, a.elapsed_time(b) * 1e-3 / reps)
        per_layer[i] = best
        del g
    ai = conv_ops / conv_bytes
    classes = {"stem_pool": [0],
               "hbm_bound": [i for i in range(1, n_conv) if ai[i] < RIDGE],
               "mfma_bound": [i for i in range(1, n_conv) if ai[i] >= RIDGE]}
    layer_classes = {}
    for name, idx in classes.items():
        t, o, by = per_layer[idx].sum(), conv_ops[idx].sum(), conv_bytes[idx].sum()
        r = roofline(o, by, t)
        r.update(layers=len(idx), us_per_step=t * 1e6, tops=o / t / 1e12, gbs=by / t / 1e9,
                 frac_of_measured_mfma=o / t / (cal["mfma_int8_tops"] * 1e12),
                 frac_of_measured_copy=by / t / 1e9 / cal["copy_gbs"])
        layer_classes[name] = r

    value = step_ops / (ms_per_step * 1e-3) / 1e12
    rec = {
        "metric": METRIC, "value": value, "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": wl_name, "batch": args.batch, "image_hw": 224,
                   "convs": len(tr.layers), "conv_launches": n_conv, "ops_per_step": step_ops,
                   "activations": "uint8 asymmetric per-tensor, stored as int8 bytes q - 128 (zero points Z - 128)",
                   "weights": "int8 per-channel symmetric" + (
                       ", 2:4-pruned after the stem (sparse MFMA; ops counted as the dense 2*M*N*K)" if sparse else ""),
                   "step": "quantize fp32 input, %d fused convs + max pooling (fused with the stem) in %d "
                           "launches, dequantize output; three HIP graphs per step" % (len(tr.layers), n_conv)},
        "pct_int8_mfma_peak": value * 1e12 / PEAK_INT8_OPS,
        "pct_measured_mfma": value / cal["mfma_int8_tops"],
        "roofline": roof,
        "conv_time_share": float(conv_s.mean() / (ms_per_step * 1e-3)),
        "layer_classes": layer_classes,
        "per_layer_sum_over_conv_graph": float(per_layer.sum() / conv_s.mean()),
        "per_layer_us_tops": {net.unit_name(i): [round(per_layer[i] * 1e6, 1),
                                                 round(conv_ops[i] / per_layer[i] / 1e12, 1)]
                              for i in range(n_conv)},
        "calibration": cal,
    }
    if not args.no_cpu_baseline:
        # back to uint8 codes (the stored bytes are q - 128) for the comparison with the oracle
        g_quant.replay()
        g_conv.replay()
        torch.cuda.synchronize()
        final_codes = net.bufs[net.final].cpu().numpy() ^ np.uint8(0x80 if net.offset_codes else 0)
        rec["cpu_baseline"] = cpu_baseline_trunk(tr, final_codes, args.cpu_seconds)
    else:
        rec["cpu_baseline"] = None
    del g_quant, g_conv, g_deq, net, x
    torch.cuda.empty_cache()
    if not args.no_configs:
        rec["configs"] = {}
        for wl in CONFIG_WORKLOADS:
            t0 = time.perf_counter()
            rec["configs"][wl] = config_record(torch, wl, 50)
            log("config %s: %.1f us, bit-exact %s (%.1f s)" % (wl, rec["configs"][wl]["us_per_launch"],
                                                               rec["configs"][wl]["bit_exact_vs_oracle"],
                                                               time.perf_counter() - t0))
            torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batch", type=int, default=256)
    ap.add_argument("--workload", default="resnet50_trunk",
                    choices=["resnet50_trunk", "resnet50_trunk_2of4", "conv3x3_int8", "conv3x3_2of4", "conv3x3_4bit",
                             "conv3x3_4bit_fp6", "conv3x3_uint8w", "conv3x3_intrq", "resnet50_l3_conv3x3",
                             "resnet50_stem_pool", "conv1x1_int8", "conv1x1_intrq", "resnet50_l3_conv3x3_intrq",
                             "resnet50_l3_conv3x3_s8",
                             "resnet50_l1_pair", "vitl_fc1", "vitl_fc1_2of4", "gemm_int8_256"])
    ap.add_argument("--cold", action="store_true",
                    help="single-layer workloads: rotate input/output sets (> 256 MB) so every launch misses the caches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="trunk: leave out the four single-layer workloads of the configs block")
    ap.add_argument("--no-calibration", action="store_true",
                    help="single-layer workloads: leave out the calibration kernels (for profiling runs)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--tile", type=int, default=-1,
                    help="single-layer workloads: force this kernel configuration (iqnn_kernel_cfg.tile)")
    ap.add_argument("--xcd-groups", type=int, default=0,
                    help="single-layer workloads: force this many channel-tile groups across the XCDs")
    ap.add_argument("--traffic-db", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="print the TRAFFIC record of two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) made "
                         "with --calib-copy-mib and exit (no GPU needed)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one device-to-device copy of this many MiB before warm-up: a plain copy "
                         "kernel of known size that scales the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.traffic_db:
        t = traffic_from_dbs(args.traffic_db[0], args.traffic_db[1], args.workload)
        true_bytes = args.calib_copy_mib << 20
        f_fetch = true_bytes / (t["fetch"][0] * 1024.0)
        f_write = true_bytes / (t["write"][0] * 1024.0)
        per_launch = t["fetch"][1] * 1024.0 * f_fetch + t["write"][1] * 1024.0 * f_write
        wl = args.workload if args.workload != "resnet50_trunk" else "resnet50_trunk_b%d" % args.batch
        rec = {"workload": wl, "kernel_source": kernel_source_tag(), "bytes_per_launch": per_launch,
               "fetch_bytes_per_launch": t["fetch"][1] * 1024.0 * f_fetch,
               "write_bytes_per_launch": t["write"][1] * 1024.0 * f_write,
               "fetch_scale": f_fetch, "write_scale": f_write, "launches": t["fetch"][2]}
        print("TRAFFIC " + json.dumps(rec))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path (got --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    from integer_quantized_nn_amd import binding
    binding.lib()
    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: %d bytes read, %d bytes written" % (n, n))
        del src, dst
    trunk = args.workload.startswith("resnet50_trunk")
    cal = None if (args.no_calibration and not trunk) else calibrate(torch)
    rec = bench_trunk(args, torch, cal) if trunk else bench_layer(args, torch, cal)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
