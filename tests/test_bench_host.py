"""Host-side parts of bench.py (no GPU): the metric names, the one-GPU refusal and the keying of
the committed counter records to the kernel sources."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_default_workload_carries_the_headline_metric():
    headline = "TFLOP/s + % bf16 MFMA peak, GEMM+RS local share N=8192 (1 GPU)"
    sys_argv, sys.argv = sys.argv, ["bench.py"]
    try:
        args = bench.parse()
    finally:
        sys.argv = sys_argv
    assert args.workload == "rs_8192" and args.gpus == 1
    assert "TFLOP/s + % bf16 MFMA peak, " + bench.WORKLOAD_TITLES[args.workload] + " (1 GPU)" \
        == headline


def test_every_workload_has_a_title_and_a_kernel_family():
    for wl in ("rs_8192", "ag_8192", "ar_16384", "moe_dispatch", "moe_combine", "ring_attention",
               "rs_tiny"):
        assert wl in bench.WORKLOAD_TITLES
        assert len(bench.kernel_source_hash(bench.kernel_family(wl))) == 16


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_records_are_keyed_to_their_kernel_source(tmp_path, monkeypatch):
    rec = {"rs_8192/owner": {"source_hash": bench.kernel_source_hash("gemm"),
                             "bytes_per_launch": 123},
           "ring_attention/owner": {"source_hash": "0" * 16, "bytes_per_launch": 456}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("rs_8192", "owner") == 123
    assert bench.measured_traffic("ring_attention", "owner") is None   # stale source
    assert bench.measured_traffic("ag_8192", "owner") is None          # no record


def test_source_hash_ignores_comments_and_layout():
    a = "int f(int x) {  // doubles\n    return 2 * x; /* no overflow check */\n}\n"
    b = "int f(int x) {\n return 2 * x;\n}"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(a.replace("2 * x", "3 * x"))
