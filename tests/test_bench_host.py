"""Host logic of bench.py (no GPU): the roofline's bound and fractions, the HBM traffic
reduction from rocprofv3 counter databases scaled by a copy of known size, the
traffic record's kernel-source check, and the one-GPU contract of the command line."""
import os
import sqlite3
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_roofline_bound_follows_the_ridge():
    ridge = bench.PEAK_INT8_OPS / bench.PEAK_HBM          # 625 ops per byte
    nbytes, secs = 1_000_000_000, 1e-3
    below = bench.roofline(ops=int(0.9 * ridge * nbytes), nbytes=nbytes, seconds=secs)
    assert below["bound"] == "hbm" and below["unit"] == "GB/s"
    assert below["achieved"] == pytest.approx(nbytes / secs / 1e9)
    assert below["frac"] == pytest.approx(below["achieved"] / below["peak"])
    above = bench.roofline(ops=int(1.1 * ridge * nbytes), nbytes=nbytes, seconds=secs)
    assert above["bound"] == "mfma" and above["unit"] == "TOPS"
    assert above["achieved"] == pytest.approx(1.1 * ridge * nbytes / secs / 1e12, rel=1e-6)
    assert above["peak"] == pytest.approx(bench.PEAK_INT8_OPS / 1e12)


def _counter_db(path, rows):
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (dispatch_id integer, kernel_name text, counter_name text, "
                "value real)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?)", rows)
    con.commit()
    con.close()


def test_traffic_from_counter_databases(tmp_path):
    # a 1 GiB copy whose FETCH_SIZE reads half its bytes (factor 2) and WRITE_SIZE all of
    # them (factor 1), then three conv dispatches
    fetch, write = str(tmp_path / "f.db"), str(tmp_path / "w.db")
    gib_kib = float(1 << 20)
    _counter_db(fetch, [(1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", gib_kib / 2),
                        (2, "void qconv_stream<A>(ConvParams)", "FETCH_SIZE", 1000.0),
                        (3, "void qconv_direct3x3<B>(ConvParams)", "FETCH_SIZE", 2000.0),
                        (4, "quantize_kernel(QuantParams)", "FETCH_SIZE", 9999.0),
                        (5, "void qconv_stream<A>(ConvParams)", "FETCH_SIZE", 3000.0)])
    _counter_db(write, [(1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", gib_kib),
                        (2, "void qconv_stream<A>(ConvParams)", "WRITE_SIZE", 400.0),
                        (3, "void qconv_direct3x3<B>(ConvParams)", "WRITE_SIZE", 500.0),
                        (5, "void qconv_stream<A>(ConvParams)", "WRITE_SIZE", 600.0)])
    t = bench.traffic_from_dbs(fetch, write, "resnet50_trunk")
    assert t["fetch"] == (gib_kib / 2, 2000.0, 3)      # calibration KiB, mean over qconv_*, count
    assert t["write"] == (gib_kib, 500.0, 3)
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--traffic-db", fetch, write,
                          "--calib-copy-mib", "1024"], capture_output=True, text=True, cwd=ROOT)
    assert out.returncode == 0, out.stderr
    line = [l for l in out.stdout.splitlines() if l.startswith("TRAFFIC ")][0]
    import json
    rec = json.loads(line[len("TRAFFIC "):])
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["bytes_per_launch"] == pytest.approx(2000.0 * 1024 * 2 + 500.0 * 1024)
    assert rec["kernel_source"] == bench.kernel_source_tag()


def test_traffic_record_only_for_the_built_kernel_source(monkeypatch):
    rec = bench.measured_traffic("resnet50_trunk_b256")
    if rec is not None:                                 # the committed record matches the source
        assert rec > 0
    monkeypatch.setattr(bench, "kernel_source_tag", lambda: "0000000000000000")
    assert bench.measured_traffic("resnet50_trunk_b256") is None
    assert bench.measured_traffic("no_such_workload") is None


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, cwd=ROOT, timeout=120)
    assert out.returncode == 2
    assert "one GPU" in out.stderr
