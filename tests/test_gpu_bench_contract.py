"""bench.py's JSON line on the GPU: a short run of the headline activation and of one MoE
op, each printing exactly one JSON line on stdout whose fields follow the bench contract
(metric, value, unit, step counts, dtype, config, roofline with its fraction, the CPU
oracle baseline, the streaming-probe ceilings)."""
import json
import os
import subprocess
import sys

import pytest

from parity import say

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run_bench(*args):
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), *args]
    say("[bench contract] " + " ".join(args))
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-3000:]
    lines = [ln for ln in res.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, f"expected one JSON line on stdout, got {len(lines)}"
    return json.loads(lines[0])


def _check_common(d, steps, warmup):
    assert d["unit"] == "GB/s" and d["value"] > 0 and d["ms_per_step"] > 0
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == warmup
    assert d["higher_is_better"] is True and d["scaling"] in ("weak", "strong")
    assert d["vs_baseline"] is None and d["dtype"] == "bf16" and d["data"] == "synthetic"
    assert isinstance(d["metric"], str) and isinstance(d["config"]["workload"], str)
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] > 0 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert r["traffic"] is None or r["traffic"] > 0
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["sample"]


def test_headline_line():
    d = _run_bench("--steps", "3", "--warmup", "2", "--cold-reps", "2", "--cpu-seconds", "0.1")
    _check_common(d, 3, 2)
    assert d["config"]["workload"] == "headline"
    assert d["config"]["rows"] == 53760 and d["config"]["inter"] == 2048
    assert d["roofline"]["kernel"] == "swiglu_probs_bwd"
    assert d["fwd"]["algorithmic_bytes"] == 660817920 and d["bwd"]["algorithmic_bytes"] == 1101434880
    assert abs(d["roofline"]["achieved"] - d["bwd"]["GB/s"]) < 0.2
    assert set(d["hbm_probe"]) == {"copy_1r1w", "fwd_like_2r1w", "bwd_like_3r2w", "read_only_3r",
                                   "write_only_2w", "torch_copy_1r1w", "torch_add_2r1w", "hip_memcpy_1r1w"}
    for name in ("fwd", "bwd"):
        k = d[name]
        # each launch's own start/end events: the durations are those of the kernel alone
        assert 0 < k["us_min"] <= k["us"] <= k["us_max"] and k["us_back_to_back"] > 0
        assert k["us_min"] <= k["us_median"] <= k["us_max"]
        assert 0 < k["frac_of_best_ceiling"] < 1.5
    assert d["device_ms_per_step"] > 0 and d["cold"]["reps"] == 2
    assert d["cpu_baseline"]["host_cores"] >= d["cpu_baseline"]["cores"]


def test_moe_op_line():
    d = _run_bench("--op", "unpermute", "--steps", "3", "--warmup", "2", "--cold-reps", "2",
                   "--cpu-seconds", "0.1")
    _check_common(d, 3, 2)
    assert d["config"]["workload"] == "moe_unpermute"
    k = d["kernels"]["unpermute"]
    assert k["algorithmic_bytes"] > 0 and k["GB/s"] > 0 and "cold_us_min" in k
    p = d["hbm_probe"]["unpermute"]
    assert p["mix"] == "2:1" and 0 < p["kernel_frac_of_probe"] < 2
