"""Host logic of bench.py that needs no GPU: the single-GPU refusal, the
algorithmic work and byte model the roofline divides by, and the ingestion
of rocprofv3 counter files (scaling by a plain copy, source hashing)."""
import csv
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_model_at_the_layer_shape():
    b = _bench()
    batch, dim, L, N = 4, 5120, 2048, 16
    elems = batch * dim * L * N
    # per element: Delta*A, exp (4 slots), Delta*x*B, state fma, readout fma = 8;
    # per (b, d, l): dt + bias 1, softplus 9, Delta*x 1, skip 1, silu 10, gate 1 = 23
    assert b.algorithmic_slots(batch, dim, L, N) == batch * dim * L * (8 * N + 23)
    assert b.algorithmic_slots(batch, dim, L, N) / elems == pytest.approx(9.4375)
    # x, dt, z bf16 in and y fp32 out per (b, d, l); Bm, Cm bf16; A, Dskip,
    # dt_bias fp32; hL fp32
    expect = (batch * dim * L * (3 * 2 + 4) + 2 * batch * N * L * 2 + dim * N * 4 + 2 * dim * 4
              + batch * dim * N * 4)
    assert b.algorithmic_bytes(batch, dim, L, N, 2, 4) == expect == 421_634_048


def _write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, c, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_counter_ingestion_scales_by_the_copy(tmp_path, monkeypatch):
    b = _bench()
    out = tmp_path / "counters.json"
    monkeypatch.setattr(b, "COUNTERS", str(out))
    kern = "void ssm::(anonymous namespace)::" + b.SCAN_KERNEL + "(ssm::ScanParams)"
    other = "void ssm::(anonymous namespace)::state_update_kernel<...>(...)"
    _write_counters(tmp_path / "fetch", [(kern, "FETCH_SIZE", 100.0), (kern, "FETCH_SIZE", 300.0),
                                         (other, "FETCH_SIZE", 1e9)])
    _write_counters(tmp_path / "write", [(kern, "WRITE_SIZE", 50.0), (other, "WRITE_SIZE", 7.0)])
    # a 1 MiB copy (1024 KiB each way) whose fetch counter reads half the bytes
    _write_counters(tmp_path / "copyf", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 512.0)])
    _write_counters(tmp_path / "copyw", [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 1024.0)])
    rec = b.ingest_counters(str(tmp_path / "fetch"), str(tmp_path / "write"), str(tmp_path / "copyf"),
                            str(tmp_path / "copyw"), copy_mib=1, workload="w")
    assert rec["copy_calibration"]["fetch_scale"] == 2.0
    assert rec["copy_calibration"]["write_scale"] == 1.0
    assert rec["fetch_size_kib_per_dispatch"] == {b.SCAN_KERNEL: 200.0}
    assert rec["traffic_bytes_per_launch"] == (200.0 * 2 + 50.0) * 1024
    assert json.loads(out.read_text()) == {"w": rec}
    # read back for the same sources and workload; another workload gets none
    assert b.counter_traffic("w") == rec["traffic_bytes_per_launch"]
    assert b.counter_traffic("another workload") is None
    # a changed kernel source (another hash) makes the stored traffic stale
    monkeypatch.setattr(b, "kernel_sources_sha256", lambda: "0" * 64)
    assert b.counter_traffic("w") is None


def test_counter_ingestion_sums_the_kernels_of_a_step(tmp_path, monkeypatch):
    """A split step is two launches (aggregate pass, main pass): its traffic
    is the sum of both kernels' per-dispatch means; records of several
    workloads live side by side in the one file."""
    b = _bench()
    out = tmp_path / "counters.json"
    monkeypatch.setattr(b, "COUNTERS", str(out))
    main, agg = b.scan_kernel_name("f32"), b.scan_kernel_name("f32", agg=True)
    assert main != agg and "true, true>" in agg
    _write_counters(tmp_path / "fetch", [(main, "FETCH_SIZE", 100.0), (agg, "FETCH_SIZE", 60.0),
                                         (agg, "FETCH_SIZE", 80.0)])
    _write_counters(tmp_path / "write", [(main, "WRITE_SIZE", 30.0), (agg, "WRITE_SIZE", 2.0)])
    _write_counters(tmp_path / "copyf", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 1024.0)])
    _write_counters(tmp_path / "copyw", [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 1024.0)])
    dirs = [str(tmp_path / d) for d in ("fetch", "write", "copyf", "copyw")]
    r1 = b.ingest_counters(*dirs, copy_mib=1, workload="long", kernels=(main, agg))
    assert r1["traffic_bytes_per_launch"] == (100.0 + 70.0 + 30.0 + 2.0) * 1024
    r2 = b.ingest_counters(*dirs, copy_mib=1, workload="layer", kernels=(main,))
    stored = json.loads(out.read_text())
    assert stored == {"long": r1, "layer": r2}
    assert b.counter_traffic("long") == r1["traffic_bytes_per_launch"]
    assert b.counter_traffic("layer") == (100.0 + 30.0) * 1024


def test_roofline_picks_the_binding_roof():
    b = _bench()
    # the 2.8B layer: ALU time (slots / 78.6 T) exceeds the HBM time (bytes / 8 TB/s)
    r = b.roofline(4, 5120, 2048, 16, 2, 200e-6)
    assert r["bound"] == "alu"
    assert r["hbm"]["min_seconds"] < b.algorithmic_slots(4, 5120, 2048, 16) / b.PEAK_SLOTS
    assert r["frac"] == pytest.approx(b.algorithmic_slots(4, 5120, 2048, 16) / 200e-6 / b.PEAK_SLOTS)
    # the fp32 2^20-step sequence: 16 bytes per (b, d, l) put HBM ahead
    r = b.roofline(1, 1536, 1 << 20, 16, 4, 15e-3)
    assert r["bound"] == "hbm"
    assert r["algorithmic_bytes"] == b.algorithmic_bytes(1, 1536, 1 << 20, 16, 4, 4)
    assert r["frac"] == pytest.approx(r["algorithmic_bytes"] / 15e-3 / b.PEAK_HBM)
    assert r["alu"]["min_seconds"] < r["algorithmic_bytes"] / b.PEAK_HBM


def test_ingestion_without_samples_fails_loudly(tmp_path, monkeypatch):
    b = _bench()
    monkeypatch.setattr(b, "COUNTERS", str(tmp_path / "counters.json"))
    for d in ("fetch", "write", "copyf", "copyw"):
        _write_counters(tmp_path / d, [])
    with pytest.raises(SystemExit):
        b.ingest_counters(*(str(tmp_path / d) for d in ("fetch", "write", "copyf", "copyw")))
    assert not (tmp_path / "counters.json").exists()
