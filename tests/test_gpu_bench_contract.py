"""bench.py end to end: exactly one JSON line on stdout with the fields the
benchmark promises (metric, throughput, timing with cache eviction and
percentiles, the roofline object for the dominant call and the CPU-oracle
baseline), and a passing parity check -- eager launches on the small float32
workload, HIP-graph replay on a full-size decode workload."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CASES = [("tiny", ["--cpu-sample", "16"], "eager launches"),
         ("v2l_decode1", [], "hip graph replay")]


@pytest.mark.parametrize("workload,extra,launch", CASES, ids=[c[0] for c in CASES])
def test_bench_prints_one_json_line_with_roofline_and_cpu_baseline(workload, extra, launch):
    print(f"[bench-contract] {workload}", flush=True)
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", workload, "--steps", "5",
                          "--warmup", "1", *extra], capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-3000:]
    lines = [l for l in res.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, res.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline", "timing"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"] == workload
    t = d["timing"]
    assert t["launch"] == launch and t["cache"] == "evicted"
    st = t["step"]
    assert st["n"] == 5 and st["p10_ms"] <= st["median_ms"] <= st["p90_ms"]
    assert d["ms_per_step"] == pytest.approx(st["median_ms"], rel=1e-3)
    assert t["warm_cache_step"]["median_ms"] > 0
    r = d["roofline"]
    assert r["bound"] in ("hbm", "mfma") and r["unit"] in ("GB/s", "TFLOP/s")
    assert r["achieved"] > 0 and r["peak"] > 0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) <= 1e-3 * max(1.0, r["frac"])
    assert "traffic" in r and "frac_profile" in r
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["unit"] and c["sample"]
    assert c["cpu_model"] and c["blas"]
    p = d["parity"]
    assert p["pass"] is True
    assert p["routing"]["topk_bit_exact_on_gpu_logits"] and p["routing"]["logits_within_certified_bound"]
    assert p["oracle_routes_fed"]["scatter_bit_exact"] and p["oracle_routes_fed"]["tokens_compared"] >= 1
    assert p["own_routes"]["tokens_compared"] >= 1
