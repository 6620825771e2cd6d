"""Host logic of bench.py (CPU, no GPU): the single-GPU guard, and the
algorithmic byte counts the roofline divides by, recomputed here from the sizes
of the oracle's own outputs (every array the method must read or write, once)
on seeded workloads."""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "single GPU" in r.stderr
    assert r.stdout == ""                      # no JSON line


def _nbytes(*arrays):
    return sum(a.nbytes for a in arrays if a is not None)


@pytest.mark.parametrize("name,T", [("tiny", None), ("decode", None), ("prefill", 384), ("grouped", 384),
                                    ("skewed", 384)])
def test_algorithmic_bytes_match_the_oracle_outputs(name, T):
    d = W.make(name, T=T)
    c = d["cfg"]
    T, H, E, R, k = c["T"], c["H"], c["E"], c["R"], c["k"]
    ll = c["layout"] == W.LAYOUT_PADDED_LL
    idx, w = d["topk_idx"], d["topk_weights"]
    ref = oracle.dispatch(d["x"], idx, E, R, quant=c["quant"], max_tokens=c["max_tokens"] if ll else 0,
                          with_send=not ll)
    n_pairs, n_send = ref["n_pairs"], ref["n_send"]
    got = bench.algorithmic_bytes(c, T, n_send, n_pairs, T * k)

    # layout: the routing in; per-expert and per-rank counts and the token x rank flags out
    assert got["layout"] == _nbytes(idx, ref["num_tokens_per_expert"], ref["num_tokens_per_rank"],
                                    ref["is_token_in_rank"])
    # dispatch: x and the routing in; every payload row (and scale row) out once, plus the
    # handle: a position and a source index per routed slot, send sources, offsets and counts
    pos_valid = ref["pos"][ref["pos"] >= 0]
    handle = _nbytes(pos_valid, ref["recv_src_idx"], ref["expert_offsets"], ref["rank_offsets"],
                     ref["num_tokens_per_expert"])
    rows = _nbytes(ref["recv_rows"], ref["recv_scales"])
    if not ll:
        rows += _nbytes(ref["send_rows"], ref["send_scales"])
        handle += _nbytes(ref["send_src_idx"])
    assert got["dispatch"] == _nbytes(d["x"], idx) + rows + handle
    # combine: each routed expert-output row (bf16) once, weights and positions per slot, the output
    y_rows = 2 * H * n_pairs
    assert got["combine"] == y_rows + _nbytes(w, ref["pos"]) + 2 * T * H
    # backward: gradient rows mirror the forward's rows
    b = bench.backward_bytes(c, T, n_pairs)
    assert b["dispatch_bwd"] == y_rows + _nbytes(ref["pos"]) + 2 * T * H
    assert b["combine_bwd"] == 2 * T * H + _nbytes(w, ref["pos"]) + 2 * y_rows + _nbytes(w)


def test_percentiles_of_launch_durations():
    ms = [0.001 * v for v in range(1, 101)]   # 1..100 us
    p10, p50, p90 = bench.percentiles_us(ms)
    assert p10 == pytest.approx(10.9) and p50 == pytest.approx(50.5) and p90 == pytest.approx(90.1)


def test_kernel_table_reports_percentiles_and_cold_passes():
    kt = {"dispatch": {"total_ms": 0.3, "launches": 3, "ms": [0.1, 0.1, 0.1]},
          "combine": {"total_ms": 0.0, "launches": 0, "ms": []}}
    cold = {"cold": {"dispatch": {"total_ms": 0.6, "launches": 3, "ms": [0.2, 0.2, 0.2]},
                     "combine": {"total_ms": 0.0, "launches": 0, "ms": []}}}
    t = bench.kernel_table(kt, {"dispatch": 1_000_000, "combine": 5}, cold=cold)
    assert set(t) == {"dispatch"}                       # kernels with no launch are left out
    assert t["dispatch"]["us"] == 100.0 and t["dispatch"]["GB/s"] == 10.0
    assert t["dispatch"]["us_p10_p50_p90"] == [100.0, 100.0, 100.0]
    assert t["dispatch"]["us_cold_p10_p50_p90"] == [200.0, 200.0, 200.0]


def test_kernel_passes_reports_every_pass_and_the_primary():
    mk = lambda ms: {"total_ms": sum(ms), "launches": len(ms), "ms": ms}
    none = {"total_ms": 0.0, "launches": 0, "ms": []}
    passes = {"cold": {"dispatch": mk([0.2, 0.2, 0.2]), "combine": none},
              "warm": {"dispatch": mk([0.1, 0.1, 0.1]), "combine": none}}
    t = bench.kernel_passes(passes, {"dispatch": 1_000_000, "combine": 5}, "cold")
    assert set(t) == {"dispatch"}                       # kernels with no launch are left out
    k = t["dispatch"]
    assert k["us"] == k["us_cold"] == 200.0 and k["GB/s"] == k["GB/s_cold"] == 5.0
    assert k["us_warm"] == 100.0 and k["GB/s_warm"] == 10.0 and k["GB/s_cold_p50"] == 5.0
    assert k["us_cold_p10_p50_p90"] == [200.0, 200.0, 200.0]


def _tiny_state():
    import torch
    d = W.make("tiny")
    c = d["cfg"]
    ref = oracle.dispatch(d["x"], d["topk_idx"], c["E"], c["R"], quant=c["quant"])
    n = ref["n_pairs"]
    y = torch.from_numpy(W.expert_outputs(d, n).view(np.int16)).view(torch.bfloat16)
    return d, c, y, ref


def test_oracle_timing_runs_for_the_time_asked_and_splits_the_ops():
    """The oracle baseline repeats steps until the CPU time asked for is spent
    (at least three), timing layout, dispatch and combine each on its own, and
    reports their medians; pinned to one core and unpinned afterwards."""
    d, c, y, _ = _tiny_state()
    s = {"d": d, "c": c, "y": y}
    before = os.sched_getaffinity(0)
    o = bench.oracle_timing(s, seconds=0.0)
    assert o["runs"] == 3 and os.sched_getaffinity(0) == before
    for key in ("layout_ms", "dispatch_ms", "combine_ms", "step_ms"):
        assert o[key] > 0, key
    o = bench.oracle_timing(s, seconds=0.2)
    assert o["cpu_seconds"] >= 0.2 and o["runs"] > 3
    o = bench.oracle_timing(s, runs=7)
    assert o["runs"] == 7


def test_oracle_ops_are_the_oracle_step():
    """The three timed ops together compute what oracle.dispatch + combine
    compute (the timing splits the step, it does not change it)."""
    d, c, y, ref = _tiny_state()
    s = {"d": d, "c": c, "y": y}
    yb, kw = bench.oracle_inputs(s)
    combined = []
    real_combine = oracle.combine
    try:
        oracle.combine = lambda yy, w, pos: combined.append(real_combine(yy, w, pos))
        bench.oracle_ops(s, yb, kw)
    finally:
        oracle.combine = real_combine
    expect = real_combine(y.view(__import__("torch").int16).numpy().view(np.uint16), d["topk_weights"], ref["pos"])
    assert len(combined) == 1 and np.array_equal(combined[0], expect)


def test_host_time_per_call_is_the_median_call():
    """host_us_per_call times each call alone (no synchronization inside) and
    reports the median in microseconds."""
    import time
    import types
    syncs = []
    fake_torch = types.SimpleNamespace(cuda=types.SimpleNamespace(synchronize=lambda: syncs.append(1)))
    calls = []

    def fn():
        calls.append(1)
        time.sleep(0.002 if len(calls) % 10 == 0 else 0.0)   # a few slow outliers
    us = bench.host_us_per_call(fake_torch, fn, n=50)
    assert len(calls) == 50 and len(syncs) == 2
    assert 0 < us < 1000                       # the median ignores the 2 ms outliers


def test_oracle_inputs_in_both_receive_modes():
    """In the padded low-latency mode the oracle's combine reads the expert
    outputs at the oracle's own padded rows, gathered into its expert-major
    order: the same values as in the contiguous mode."""
    import torch
    d, c, y, ref = _tiny_state()
    y_c, kw = bench.oracle_inputs({"d": d, "c": c, "y": y})
    assert kw["with_send"] and kw["max_tokens"] == 0
    # the same tokens in the padded layout: expert outputs at e * cap + slot
    cl = dict(c, layout=1, max_tokens=c["T"])
    cap = cl["max_tokens"] * c["R"]
    ll = oracle.dispatch(d["x"], d["topk_idx"], c["E"], c["R"], quant=c["quant"], max_tokens=cl["max_tokens"],
                         with_send=False)
    valid = ll["pos"] >= 0
    y_pad = torch.zeros((c["E"] * cap, c["H"]), dtype=torch.bfloat16)
    y_pad[torch.from_numpy(ll["pos_ll"][valid].astype(np.int64))] = y[torch.from_numpy(
        ll["pos"][valid].astype(np.int64))]
    y_l, kw_l = bench.oracle_inputs({"d": d, "c": cl, "y": y_pad})
    assert not kw_l["with_send"] and kw_l["max_tokens"] == c["T"]
    assert np.array_equal(y_l, y_c)
    o = bench.oracle_timing({"d": d, "c": cl, "y": y_pad}, runs=2)
    assert o["runs"] == 2 and o["combine_ms"] > 0
