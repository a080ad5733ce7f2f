"""Host logic of bench.py that needs no GPU: the HBM-traffic summary built
from rocprofv3 counter CSVs and its read-back guarded by the source hash."""
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
