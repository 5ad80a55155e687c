"""The benchmark's output contract on a GPU: one JSON line with the metric,
the whole-step throughput, the dominant kernel's roofline and the oracle's
CPU rate, for both backward forms (run on the small workload, few steps)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("scores", ["stored", "recompute"])
def test_bench_prints_one_json_line(scores):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"[bench] contract, dkv scores {scores}", flush=True)
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny",
                          "--steps", "3", "--warmup", "1", "--cpu-seconds", "0.5", "--no-topk", "--no-configs",
                          "--dkv-scores", scores],
                         capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [ln for ln in res.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "nonfinite_check", "median", "host",
                "effective_gather"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["value"] > 0 and d["ms_per_step"] > 0
    assert d["config"]["dkv_scores"] == scores
    r = d["roofline"]
    assert r["bound"] == "mfma" and r["peak"] == 2516.6 and 0 < r["frac"] < 1
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1
    assert 1 <= c["cores"] <= c["affinity_cores"]
    kg = d["kv_groups"]
    assert kg["ms_per_step"] > 0 and kg["useful_tflops"] > 0 and kg["two_single_group_calls_ms"] > 0
    for part in ("warm", "cold_caches"):
        m = d["median"][part]
        assert 0 < m["fwd_ms"] < m["fwd_bwd_ms"] and 0 < m["bwd_ms"] < m["fwd_bwd_ms"]

