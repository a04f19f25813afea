"""bench.py's host-side contract, no GPU needed: it refuses more than one GPU with a
message, the kernel-source hash that keys the counter summaries ignores comments and
whitespace but not code, and its timing events use the HIP runtime torch loaded."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr or "one MI355X" in res.stderr
    assert res.stdout == ""


def test_source_hash_ignores_comments_only(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text("int f(int x) { return x + 1; } // one\n/* block */\n")
    b = tmp_path / "b.hip"
    b.write_text("int f(int x)  {\n  return x + 1;   // another comment\n}\n")
    c = tmp_path / "c.hip"
    c.write_text("int f(int x) { return x + 2; }\n")
    ha, hb, hc = (bench.kernel_source_hash([str(p)]) for p in (a, b, c))
    assert ha == hb
    assert ha != hc


def test_traffic_needs_matching_workload_and_source(tmp_path):
    import json
    p = tmp_path / "pmc.json"
    p.write_text(json.dumps({"workload": "headline", "kernel_source_sha256_16": bench.kernel_source_hash(),
                             "bwd": {"hbm_bytes_per_launch": 123}}))
    assert bench.measured_traffic("headline", path=str(p)) == 123
    assert bench.measured_traffic("mid", path=str(p)) is None
    p.write_text(json.dumps({"workload": "headline", "kernel_source_sha256_16": "0" * 16,
                             "bwd": {"hbm_bytes_per_launch": 123}}))
    assert bench.measured_traffic("headline", path=str(p)) is None


def test_timing_events_use_the_loaded_hip_runtime():
    """The bench's timing events go through the HIP runtime torch already mapped, found
    in this process's mappings, so no second runtime is ever loaded beside it."""
    import torch  # noqa: F401  (maps the HIP runtime)
    path = bench.TimingEvents._loaded_runtime()
    assert os.path.basename(path).startswith("libamdhip64.so") and os.path.exists(path)
