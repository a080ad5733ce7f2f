"""Host logic of bench.py that needs no GPU: the HBM-traffic and MFMA-busy
summaries built from rocprofv3 counter CSVs, and their read-back guarded by
the source hash."""
import csv
import io
import json
import os
import sys
from contextlib import redirect_stdout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _write(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(["Kernel_Name", "Counter_Name", "Counter_Value"], r)))


def test_traffic_summary_scales_counters_by_the_copy(tmp_path):
    gib_kib = (1 << 30) // 1024
    _write(tmp_path / "copy_fetch", [("copy_kernel", "FETCH_SIZE", gib_kib // 2),
                                     ("copy_kernel", "FETCH_SIZE", 10)])
    _write(tmp_path / "copy_write", [("copy_kernel", "WRITE_SIZE", gib_kib)])
    _write(tmp_path / "attn_fetch", [("bi::k_decode_mfma<...>", "FETCH_SIZE", v)
                                     for v in (300, 301, 302)] + [("other", "FETCH_SIZE", 1e9)])
    _write(tmp_path / "attn_write", [("bi::k_decode_mfma<...>", "WRITE_SIZE", 10)] * 3)
    buf = io.StringIO()
    with redirect_stdout(buf):
        bench.traffic_summary(str(tmp_path))
    rec = json.loads([ln for ln in buf.getvalue().splitlines()
                      if ln.startswith("traffic-record: ")][0][len("traffic-record: "):])
    # fetch counts half the copy's bytes -> scale 2; write scale 1; medians of the kernel rows
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["fetch_bytes"] == 301 * 1024 * 2 and rec["write_bytes"] == 10 * 1024
    assert rec["hbm_bytes_per_launch"] == 301 * 2048 + 10 * 1024
    assert rec["source_sha256"] == bench.kernel_source_hash()


def test_measured_traffic_is_null_after_a_source_change(tmp_path, monkeypatch):
    good = {"kernel": "decode_attn", "hbm_bytes_per_launch": 123,
            "source_sha256": bench.kernel_source_hash()}
    p = tmp_path / "t.md"
    p.write_text("text\ntraffic-record: " + json.dumps(good) + "\n")
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(p))
    assert bench.measured_traffic()["hbm_bytes_per_launch"] == 123
    stale = dict(good, source_sha256="0" * 64)
    p.write_text("traffic-record: " + json.dumps(stale) + "\n")
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(tmp_path / "missing.md"))
    assert bench.measured_traffic() is None


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_mfma_summary_busy_fraction_and_clock(tmp_path):
    # two dispatches of 1 ms: MFMA busy on half / all of 1,024 SIMDs' cycles,
    # GUI-active 2e6 cycles per XCD (2 GHz), work equal to 2MNK
    d = tmp_path / "gemm_mfma"
    os.makedirs(d)
    M, N, K = 256, 256, 64
    mops = 2.0 * M * N * K / 512
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
              "Start_Timestamp", "End_Timestamp"]
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for disp, busy in ((1, 0.5), (2, 1.0)):
            for name, val in (("SQ_VALU_MFMA_BUSY_CYCLES", busy * 2e6 * 1024),
                              ("SQ_INSTS_VALU_MFMA_MOPS_BF16", mops),
                              ("GRBM_GUI_ACTIVE", 2e6 * 8)):
                w.writerow({"Dispatch_Id": disp, "Kernel_Name": "void bi::k_gemm_big<0>(...)",
                            "Counter_Name": name, "Counter_Value": val,
                            "Start_Timestamp": 1000, "End_Timestamp": 1000 + 1000000})
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": "other", "Counter_Name":
                        "GRBM_GUI_ACTIVE", "Counter_Value": 1, "Start_Timestamp": 0,
                        "End_Timestamp": 1})
    out = io.StringIO()
    with redirect_stdout(out):
        bench.mfma_summary(str(tmp_path), M=M, N=N, K=K)
    rec = json.loads([ln for ln in out.getvalue().splitlines()
                      if ln.startswith("mfma-record: ")][0][len("mfma-record: "):])
    assert rec["dispatches"] == 2
    assert rec["mfma_busy"] == 0.75 and rec["mfma_busy_range"] == [0.5, 1.0]
    assert rec["clock_ghz"] == 2.0 and rec["flops_counted_over_2mnk"] == 1.0
    assert rec["source_sha256"] == bench.kernel_source_hash(bench.MFMA_SOURCES)


def test_measured_mfma_is_null_after_a_source_change(tmp_path, monkeypatch):
    good = {"kernel": "k_gemm_big", "mfma_busy": 0.7, "mfma_busy_range": [0.6, 0.8],
            "clock_ghz": 1.8, "flops_counted_over_2mnk": 1.0,
            "source_sha256": bench.kernel_source_hash(bench.MFMA_SOURCES)}
    p = tmp_path / "m.md"
    p.write_text("mfma-record: " + json.dumps(good) + "\n")
    monkeypatch.setattr(bench, "MFMA_PROFILE", str(p))
    assert bench.measured_mfma()["mfma_busy"] == 0.7
    p.write_text("mfma-record: " + json.dumps(dict(good, source_sha256="0" * 64)) + "\n")
    assert bench.measured_mfma() is None
