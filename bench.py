"""Benchmark of the quantized conv / GEMM hot path on one MI355X.

Default workload: the ResNet-50 conv trunk at batch 256 (224x224x3 input), one
step = quantize the fp32 input (resident in HBM) -> 53 fused quantized convs
(Conv_Relu / Conv / Conv_Add_Relu) + one max pooling -> dequantize the output.
`value` is whole-step throughput in TOPS (2*M*N*K of every conv, K = KH*KW*C_in
without padding) over exactly --steps timed steps.

The JSON line also carries
  roofline      the implicit-GEMM conv kernel (all its launches in the timed
                steps, timed with HIP events on the launch stream): algorithmic
                bytes or ops per launch / average launch duration, against the
                MI355X peak that binds at the kernel's arithmetic intensity;
  cpu_baseline  the CPU oracle (plain C, OpenMP) timed on the host on a bounded
                sample of the same workload (whole images), scaled to TOPS; the
                GPU output of those images is compared with it byte for byte.

Other workloads (--workload) time a single layer for the kernel tables.
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "qconv_resnet50_trunk_b256_traffic.md")


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


# ---------------------------------------------------------------- trunk


def cpu_baseline_trunk(tr, gpu_final_codes, budget_s):
    """Oracle chain on whole images until ~budget_s of wall time; returns the record."""
    import oracle as O
    w = {l.name: O.quantize(l.case.w, l.case.s_w, 0, O.INT8, axis=0) for l in tr.layers}
    per_img_ops = tr.ops() / tr.batch
    final = tr.layers[-1].out
    s_f, z_f = tr.qparams[final]
    t0 = time.perf_counter()
    n_img, exact = 0, True
    while n_img < tr.batch:
        i = n_img
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
        n_img += 1
        exact = exact and np.array_equal(O.pack(acts[final], O.UINT8)[0], gpu_final_codes[i])
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": per_img_ops * n_img / dt / 1e12, "unit": "TOPS", "cores": O.num_threads(), "kind": "oracle",
            "sample": "%d of %d images through the whole step (quantize, 53 convs, max pooling, dequantize), "
                      "%.1f s wall; weight quantization excluded" % (n_img, tr.batch, dt),
            "bit_exact_vs_gpu": bool(exact)}


def bench_trunk(args):
    import torch
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
    launches = net.launches()
    conv_launches = [l for l in launches if l[0].startswith("qconv:")]
    step_ops = sum(l[1] for l in conv_launches)
    log("prepacked %d convs; %.1f GOP per step" % (len(conv_launches), step_ops / 1e9))

    for _ in range(args.warmup):
        net.step(x)
    torch.cuda.synchronize()

    # per-launch events around every conv of every timed step, on the launch stream
    stream = torch.cuda.current_stream()
    n_conv = len(tr.layers)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_conv)]
          for _ in range(args.steps)]

    def timed_step(evs):
        net.step(x, events=evs)

    # eager steps with per-conv events: the launch durations for the roofline
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(args.steps):
        timed_step(ev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step_eager = wall * 1e3 / args.steps
    ms_per_step = ms_per_step_eager
    if not args.no_graph:
        # the step as one HIP graph launch (the same kernels, without per-launch host gaps)
        graph = net.capture(x)
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for s in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        ms_per_step = wall * 1e3 / args.steps

    dur = np.array([[a.elapsed_time(b) * 1e-3 for (a, b) in row] for row in ev])   # seconds [steps][conv]
    conv_ops = np.array([l[1] for l in conv_launches], np.float64)
    conv_bytes = np.array([l[2] for l in conv_launches], np.float64)
    avg_dur = dur.mean()                                  # average launch duration
    ops_per_launch = conv_ops.mean()
    bytes_per_launch = conv_bytes.mean()
    ai = conv_ops.sum() / conv_bytes.sum()
    if ai < PEAK_INT8_OPS / PEAK_HBM:
        roof = {"bound": "hbm", "achieved": bytes_per_launch / avg_dur / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": ops_per_launch / avg_dur / 1e12, "peak": PEAK_INT8_OPS / 1e12,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    tr_bytes = measured_traffic(wl_name)
    roof["traffic"] = tr_bytes
    roof["kernel"] = "qconv (qconv_stem_pool / qconv_direct3x3 / qconv_stream; %d launches per step)" % n_conv
    roof["algorithmic_bytes_per_launch"] = bytes_per_launch
    roof["algorithmic_ops_per_launch"] = ops_per_launch
    roof["avg_launch_us"] = avg_dur * 1e6
    roof["mfma_frac"] = ops_per_launch / avg_dur / PEAK_INT8_OPS
    if roof["bound"] == "hbm":   # the same bytes against what a plain copy reaches on this GPU
        roof["measured_copy_gbs"] = measure_copy_gbs()
        roof["frac_of_measured_copy"] = roof["achieved"] / roof["measured_copy_gbs"]

    value = step_ops / (ms_per_step * 1e-3) / 1e12
    per_layer = {}
    for i, layer in enumerate(tr.layers):
        t = float(np.median(dur[:, i]))
        per_layer[layer.name] = [round(t * 1e6, 1), round(conv_ops[i] / t / 1e12, 1)]

    rec = {
        "metric": METRIC, "value": value, "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": wl_name, "batch": args.batch, "image_hw": 224,
                   "convs": n_conv, "ops_per_step": step_ops,
                   "activations": "uint8 asymmetric per-tensor, stored as int8 bytes q - 128 (zero points Z - 128)", "weights": "int8 per-channel symmetric" + (
                       ", 2:4-pruned after the stem (sparse MFMA; ops counted as the dense 2*M*N*K)" if sparse else ""),
                   "step": "quantize fp32 input, 53 fused convs + max pooling (fused with the stem), "
                           "dequantize output"},
        "pct_int8_mfma_peak": value * 1e12 / PEAK_INT8_OPS,
        "roofline": roof,
        "conv_time_share": float(dur.sum() / args.steps / (ms_per_step * 1e-3)),
        "launch": "one HIP graph per step" if not args.no_graph else "eager launches",
        "ms_per_step_eager": ms_per_step_eager,
        "per_layer_us_tops": per_layer,
    }
    if not args.no_cpu_baseline:
        # back to uint8 codes (the stored bytes are q - 128) for the comparison with the oracle
        final_codes = net.bufs[net.final].cpu().numpy() ^ np.uint8(0x80 if net.offset_codes else 0)
        rec["cpu_baseline"] = cpu_baseline_trunk(tr, final_codes, args.cpu_seconds)
    else:
        rec["cpu_baseline"] = None
    return rec


def measure_copy_gbs(mib=1024, reps=5):
    """Best rate of a device-to-device copy (bytes read + written per second, GB/s):
    the HBM rate a plain streaming kernel reaches on this GPU."""
    import torch
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


# --------------------------------------------------------- single layers


def bench_layer(args):
    import torch
    import oracle as O
    from integer_quantized_nn_amd import synth
    from integer_quantized_nn_amd.layers import QConv, QGemm, quantize

    wl = args.workload
    fp6 = wl == "conv3x3_4bit_fp6"   # the 4-bit layer on the FP6 MFMA (weights and activations as BF6)
    # kernel configuration of every timed call: the FP6 path, or --tile / --xcd-groups
    cfg = (19, 0) if fp6 else ((args.tile, args.xcd_groups) if (args.tile >= 0 or args.xcd_groups) else None)
    peak_ops = PEAK_FP6_OPS if fp6 else PEAK_INT8_OPS
    if wl in ("conv3x3_int8", "conv3x3_4bit", "conv3x3_4bit_fp6", "conv3x3_uint8w", "conv3x3_intrq", "conv3x3_2of4"):
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
        epi = c.epi | (16 if wl == "conv3x3_intrq" else 0)   # integer-only requantization flag
        if wl == "conv3x3_2of4":
            from integer_quantized_nn_amd import binding as IB
            w_type = IB.INT8_2OF4
        layer = QConv(n, h, w, ci, co, 3, c.stride, c.pad, c.x_type, w_type, c.y_type, epi, c.z_in, c.z_out,
                      wq, c.bias, c.s_in, s_w, c.s_out, res_type=c.res_type, z_res=c.z_res, s_res=c.s_res, z_w=z_w)
        xd = quantize(torch.from_numpy(c.x).cuda(), c.s_in, c.z_in, c.x_type)
        rd = quantize(torch.from_numpy(c.res).cuda(), c.s_res, c.z_res, c.res_type) if c.res is not None else None
        ops = c.ops(n, h, w)
        oh, ow = layer.out_shape[1:3]
        w_bytes = co * 9 * ci // (2 if c.w_type in (synth.UINT4, synth.INT4) else 1)
        if wl == "conv3x3_2of4":
            w_bytes = w_bytes * 5 // 8   # kept codes + positions
        y_bytes = n * oh * ow * co // (2 if c.y_type in (synth.UINT4, synth.INT4) else 1)
        nbytes = xd.numel() + w_bytes + y_bytes + (rd.numel() if rd is not None else 0)
        ins = [(xd, rd)]
        run_on = lambda i, o: layer(ins[i][0], res=ins[i][1], out=o, cfg=cfg)
        out_shape, out_type = layer.out_shape, c.y_type
    elif wl in ("vitl_fc1", "vitl_fc1_2of4", "gemm_int8_256"):
        sparse = wl == "vitl_fc1_2of4"   # weights magnitude-pruned to 2:4 along K, on the sparse MFMA
        g = synth.vitl_fc1(sparse_2of4=sparse) if wl.startswith("vitl") else synth.gemm_int8_256()
        m, n, k = g.shape
        if g.b_codes is not None:
            b_bytes = O.pack(g.b_codes, O.INT8)
            a_dev = torch.from_numpy(O.pack(g.a_codes, O.INT8)).cuda()
        else:
            b_bytes = quantize(torch.from_numpy(g.b).cuda(), g.s_b, 0, g.b_type, axis=0).cpu().numpy()
            a_dev = quantize(torch.from_numpy(g.a).cuda(), g.s_a, g.z_a, g.a_type)
        from integer_quantized_nn_amd import binding as IB
        layer = QGemm(m, n, k, g.a_type, IB.INT8_2OF4 if sparse else g.b_type, g.c_type, g.epi, g.z_a, g.z_out,
                      b_bytes, g.bias, g.s_a, g.s_b, g.s_out)
        # ops: the dense problem's 2*M*N*K (with 2:4 weights half the products are with zero
        # codes and the kernel skips them); bytes: 2:4 weights move kept codes + positions
        ops = 2 * m * n * k
        nbytes = m * k + (n * k // 2 + n * k // 8 if sparse else n * k) + m * n
        ins = [(a_dev, None)]
        run_on = lambda i, o: layer(ins[i][0], out=o, cfg=cfg)
        out_shape, out_type = layer.out_shape, g.c_type
    else:
        raise SystemExit("unknown workload " + wl)
    # --cold: rotate enough input / output sets (at least 4, over 256 MB in all) that
    # every launch reads and writes HBM rather than the 256 MB Infinity Cache
    from integer_quantized_nn_amd.layers import empty_codes
    set_bytes = nbytes
    n_sets = max(4, -(-(300 << 20) // set_bytes)) if args.cold else 1
    for _ in range(n_sets - 1):
        ins.append(tuple(t.clone() if t is not None else None for t in ins[0]))
    outs = [empty_codes(out_shape, out_type) for _ in range(n_sets)]
    step_no = [0]

    def run():
        i = step_no[0] % n_sets
        step_no[0] += 1
        return run_on(i, outs[i])

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(max(args.warmup, 1)):
        run()
    host_per_step = (time.perf_counter() - t0) / max(args.warmup, 1)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    # A launch here can take less GPU time than the host needs to issue it, so the
    # queue is first held by a spin kernel until every timed step is enqueued; the
    # steps then run back to back and one pair of HIP events on the launch stream
    # brackets them (an event between launches would add its own few microseconds).
    spin0, spin1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    spin0.record(stream)
    torch.cuda._sleep(1 << 20)
    spin1.record(stream)
    torch.cuda.synchronize()
    s_per_cycle = spin0.elapsed_time(spin1) * 1e-3 / (1 << 20)
    hold = 2.0 * args.steps * host_per_step + 2e-3
    t_begin, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    spin0.record(stream)
    torch.cuda._sleep(int(hold / s_per_cycle))
    t0 = time.perf_counter()
    t_begin.record(stream)
    for _ in range(args.steps):
        run()
    t_end.record(stream)
    enqueued = time.perf_counter() - t0
    torch.cuda.synchronize()
    span = t_begin.elapsed_time(t_end) * 1e-3
    avg = span / args.steps   # one launch per step: its duration plus the launch-to-launch gap
    if spin0.elapsed_time(t_begin) * 1e-3 < enqueued:
        print("warning: the spin kernel ended before every timed step was enqueued", file=sys.stderr)
    ai = ops / nbytes
    if ai < peak_ops / PEAK_HBM:
        roof = {"bound": "hbm", "achieved": nbytes / avg / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": ops / avg / 1e12, "peak": peak_ops / 1e12, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(wl)
    roof["avg_launch_us"] = avg * 1e6
    roof["mfma_frac"] = ops / avg / peak_ops
    return {"metric": METRIC, "value": ops * args.steps / span / 1e12, "unit": "TOPS", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": span * 1e3 / args.steps,
            "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf6" if fp6 else "int8", "data": "synthetic",
            "config": {"workload": wl, "ops": ops, "algorithmic_bytes": nbytes,
                       "cache": ("cold (%d rotating input/output sets, %.0f MB in all)" % (n_sets, n_sets * set_bytes / 1e6)
                                 if args.cold else "warm (inputs reused)"),
                       **({"ops_note": "dense-equivalent 2*M*N*K; the 2:4 weights make half of the products "
                                       "zero, which the sparse MFMA skips"} if wl.endswith("2of4") else {})},
            "pct_int8_mfma_peak": ops / avg / PEAK_INT8_OPS, "roofline": roof, "cpu_baseline": None}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batch", type=int, default=256)
    ap.add_argument("--workload", default="resnet50_trunk",
                    choices=["resnet50_trunk", "resnet50_trunk_2of4", "conv3x3_int8", "conv3x3_2of4", "conv3x3_4bit", "conv3x3_4bit_fp6", "conv3x3_uint8w", "conv3x3_intrq",
                             "vitl_fc1", "vitl_fc1_2of4", "gemm_int8_256"])
    ap.add_argument("--cold", action="store_true",
                    help="single-layer workloads: rotate input/output sets (> 256 MB) so every launch misses the caches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="trunk: time eager launches instead of one captured HIP graph per step")
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
    rec = bench_trunk(args) if args.workload.startswith("resnet50_trunk") else bench_layer(args)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
