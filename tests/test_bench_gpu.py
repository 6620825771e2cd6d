"""bench.py's JSON line (GPU): a short run of the main step, of the decode step
and of the backward step through the command line, checked for the fields the
line must carry."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
QUICK = ["--steps", "5", "--warmup", "2", "--no-cpu-baseline", "--no-decode", "--no-backward",
         "--no-overlap", "--no-configs"]


def run_bench(*args):
    print("bench.py", " ".join(args), flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, lines                     # exactly one JSON line
    return json.loads(lines[0])


def check_line(d, steps, warmup):
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == warmup
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["value"] > 0 and d["ms_per_step"] > 0
    assert "workload" in d["config"]
    rf = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in rf, key
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["achieved"] > 0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    # the headline is the cold protocol; warm is reported beside it
    assert rf["frac_cold"] == rf["frac"] and rf["frac_warm"] > 0
    assert "cold" in d["protocol"] and d["warm"]["ms_per_step"] > 0
    assert len(d["us_per_step_p10_p50_p90"]) == 3
    for k in d["kernels"].values():
        assert k["us"] == k["us_cold"] > 0 and len(k["us_cold_p10_p50_p90"]) == 3
        assert k["us_warm"] > 0 and len(k["us_warm_p10_p50_p90"]) == 3


def test_bench_line_prefill():
    check_line(run_bench(*QUICK), 5, 2)


def test_bench_line_decode():
    d = run_bench("--workload", "decode", *QUICK)
    check_line(d, 5, 2)
    assert d["config"]["workload"].startswith("decode")


def test_bench_line_backward_step():
    d = run_bench("--step", "backward", *QUICK)
    check_line(d, 5, 2)
    assert set(d["kernels"]) == {"dispatch_bwd", "combine_bwd"}


def test_bench_line_per_call_at_both_sizes():
    """With the decode side measurement on, the line carries dispatch and
    combine us per call at 4096 and at 128 tokens, with their rates."""
    d = run_bench("--steps", "5", "--warmup", "2", "--no-cpu-baseline", "--no-backward", "--no-overlap",
                  "--no-configs")
    check_line(d, 5, 2)
    pc = d["per_call"]
    for size in ("4096_tokens", "128_tokens"):
        for n in ("dispatch", "combine"):
            e = pc[size][n]
            assert e["us"] > 0 and e["GB/s"] > 0 and 0 < e["pct_of_hbm_peak"] < 100, (size, n, e)
    assert pc["4096_tokens"]["dispatch"]["us"] == d["kernels"]["dispatch"]["us"]
    assert pc["128_tokens"]["combine"]["us"] == d["decode"]["us_per_call_graph"]["combine"]
