"""Benchmark: MoE dispatch layout + dispatch + combine on one MI355X.

One step = the whole hot path over one batch: moe_dispatch_layout, then
moe_dispatch reusing that layout, then moe_combine of the expert outputs
(low-latency workloads: moe_dispatch straight from topk_idx, then
moe_combine).  Side measurements: the 128-token decode step, and the backward
step (moe_dispatch_backward + moe_combine_backward) of the main workload.
Default workload: prefill, 4096 tokens x hidden 7168, 256 experts over 32
virtual ranks, top-8, bf16 dispatch into per-rank send buffers and the
expert-major receive layout, bf16 combine.  Inputs are resident in HBM before
the timed region; nothing is allocated inside it.

Headline protocol ("cold"): before every step, warm-up and timed alike, a
1 GiB buffer (4x the 256 MB Infinity Cache) is rewritten, untimed, so that
each step starts with the L2 and the Infinity Cache holding none of its data;
each timed step is bracketed by HIP events on the stream the library launches
on.  value = algorithmic HBM bytes of one step (x read once, every
destination row written once, expert outputs read once, outputs written once,
routing metadata) / mean cold step time, in GB/s.  The same steps back to back
with no flush ("warm") are reported beside it.  The per-kernel roofline uses
durations measured with HIP events the library records on its own launch
stream around each kernel (moe_timing_begin / moe_timing_end), cold.

Prints ONE JSON line.  --gpus N with N > 1 is refused: the library drives one GPU.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, vendor spec


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="prefill",
                   choices=["tiny", "decode", "prefill", "grouped", "skewed"])
    p.add_argument("--tokens", type=int, default=None,
                   help="override the workload's token count (same shapes and routing recipe otherwise)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-decode", action="store_true", help="skip the 128-token decode side measurement")
    p.add_argument("--no-backward", action="store_true", help="skip the backward side measurement")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the per-config table (all five workloads, warm step time)")
    p.add_argument("--no-overlap", action="store_true",
                   help="skip the GEMM-overlap side measurement (workgroup cap + hooks)")
    p.add_argument("--step", default="forward", choices=["forward", "backward"],
                   help="which step the main line times: forward (layout + dispatch + combine) or "
                        "backward (dispatch backward + combine backward)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="host CPU time the oracle baseline runs for (whole steps, at least 3)")
    p.add_argument("--profile-only", action="store_true",
                   help="run warmup + steps only (for rocprofv3), print the JSON line without baselines")
    p.add_argument("--protocol", default="cold", choices=["cold", "warm"],
                   help="cold (default, the headline): a 1 GiB write flush before every step; warm: no flush "
                        "(steps back to back, for profiling the kernels with warm caches)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run five 1 GiB device-to-device copies (known bytes) so that rocprofv3 "
                        "FETCH_SIZE / WRITE_SIZE counters can be scaled")
    return p.parse_args()


def algorithmic_bytes(c, T, n_send, n_pairs, n_slots):
    """Bytes the method must move per launch of each kernel (actual counts)."""
    H, k, E, R = c["H"], c["k"], c["E"], c["R"]
    fp8 = c["quant"] == 1
    B = (H + 4 * (H // 128)) if fp8 else 2 * H          # payload bytes per dispatched row
    ll = c["layout"] == 1
    layout = 8 * T * k + 4 * E + 4 * R + T * R
    if ll:
        dispatch = 2 * T * H + 8 * T * k + B * n_pairs + 8 * n_pairs + 4 * (2 * E + R + 2)
    else:
        dispatch = (2 * T * H + 8 * T * k + B * (n_send + n_pairs) + 4 * n_send + 8 * n_pairs
                    + 4 * (2 * E + R + 2))
    combine = 2 * n_pairs * H + 8 * n_slots + 2 * T * H
    return {"layout": layout, "dispatch": dispatch, "combine": combine}


def backward_bytes(c, T, n_pairs):
    """Algorithmic bytes of the backward kernels: dispatch backward reads the
    routed gradient rows and writes one row per token; combine backward reads
    the output gradient and the routed expert outputs and writes the routed
    gradient rows and grad_w (plus pos and weights per slot)."""
    H, k = c["H"], c["k"]
    return {"dispatch_bwd": 2 * n_pairs * H + 4 * T * k + 2 * T * H,
            "combine_bwd": 2 * T * H + 8 * T * k + 4 * n_pairs * H + 4 * T * k}


def setup_backward(torch, s):
    """Gradient buffers of the backward step, drawn on the GPU (seeded)."""
    c, y = s["c"], s["y"]
    dev = y.device
    g = torch.Generator(device=dev)
    g.manual_seed(4242 + c["index"])
    s["grad_recv"] = torch.randn(y.shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    s["grad_out"] = torch.randn((c["T"], c["H"]), generator=g, device=dev,
                                dtype=torch.float32).to(torch.bfloat16)
    s["grad_x"] = torch.empty((c["T"], c["H"]), dtype=torch.bfloat16, device=dev)
    s["grad_y"] = torch.empty_like(y)
    s["grad_w"] = torch.empty((c["T"], c["k"]), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()


def step_bwd(moe, s):
    """Backward of one step: dispatch backward (gradient rows -> tokens), then
    combine backward (output gradient -> expert-output gradient rows and grad_w)."""
    moe.moe_dispatch_backward(s["ctx"], s["grad_recv"], s["h"], grad_x=s["grad_x"])
    moe.moe_combine_backward(s["ctx"], s["grad_out"], s["w"], s["y"], s["h"],
                             grad_expert_out=s["grad_y"], grad_weights=s["grad_w"])


def percentiles_us(ms):
    """p10, p50 and p90 of per-launch durations (ms) in microseconds."""
    import numpy as np
    return [round(float(v), 2) for v in np.percentile(1e3 * np.asarray(ms, dtype=np.float64), [10, 50, 90])]


def kernel_table(kt, alg, cold=None):
    """Per kernel: mean event duration and algorithmic GB/s, p10/p50/p90 of the
    launches, and for each pass in `cold` ({label: timings}, passes with the
    caches flushed between steps) the same percentiles."""
    out = {}
    for name, b in alg.items():
        n = kt[name]["launches"]
        if n == 0 or b == 0:
            continue
        us = 1e3 * kt[name]["total_ms"] / n
        out[name] = {"us": round(us, 2), "alg_bytes": b, "GB/s": round(b / (us * 1e-6) / 1e9, 1),
                     "us_p10_p50_p90": percentiles_us(kt[name]["ms"])}
        for label, kc in (cold or {}).items():
            if kc[name]["launches"]:
                out[name]["us_%s_p10_p50_p90" % label] = percentiles_us(kc[name]["ms"])
    return out


def kernel_passes(passes, alg, primary):
    """Per kernel, for each pass ({label: timings}): mean event duration,
    algorithmic GB/s on it and on the median, p10/p50/p90 of the launches;
    "us" and "GB/s" repeat the primary pass's figures."""
    import numpy as np
    out = {}
    for name, b in alg.items():
        if b == 0 or passes[primary][name]["launches"] == 0:
            continue
        ent = {"alg_bytes": b}
        for lb, kt in passes.items():
            n = kt[name]["launches"]
            if n == 0:
                continue
            us = 1e3 * kt[name]["total_ms"] / n
            p50 = float(np.median(1e3 * np.asarray(kt[name]["ms"], dtype=np.float64)))
            ent["us_" + lb] = round(us, 2)
            ent["GB/s_" + lb] = round(b / (us * 1e-6) / 1e9, 1)
            ent["GB/s_%s_p50" % lb] = round(b / (p50 * 1e-6) / 1e9, 1)
            ent["us_%s_p10_p50_p90" % lb] = percentiles_us(kt[name]["ms"])
        ent["us"] = ent["us_" + primary]
        ent["GB/s"] = ent["GB/s_" + primary]
        out[name] = ent
    return out


def setup(moe, W, torch, name, T=None):
    d = W.make(name, T=T)
    c = d["cfg"]
    import numpy as np
    dev = torch.device("cuda", 0)
    cfg = moe.make_config(c["max_tokens"], c["H"], c["E"], c["R"], c["k"], 0, c["quant"], c["layout"])
    ctx = moe.Context(cfg)
    x = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).to(dev)
    idx = torch.from_numpy(d["topk_idx"]).to(dev)
    w = torch.from_numpy(d["topk_weights"]).to(dev)
    bufs = moe.DispatchBuffers(ctx)
    h = moe.Handle(ctx)
    cnt_e = torch.empty(c["E"], dtype=torch.int32, device=dev)
    cnt_r = torch.empty(c["R"], dtype=torch.int32, device=dev)
    in_rank = torch.empty((c["T"], c["R"]), dtype=torch.uint8, device=dev)
    out = torch.empty((c["T"], c["H"]), dtype=torch.bfloat16, device=dev)
    # expert outputs: N(0,1) bf16 in the receive layout, drawn on the GPU (seeded)
    n_rows = ctx.hint(moe.MOE_BUF_EXPERT_OUT) // (2 * c["H"])
    y = torch.empty((n_rows, c["H"]), dtype=torch.bfloat16, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(W.SEED_BASE + c["index"])
    if c["layout"] == 0:
        y.copy_(torch.randn((n_rows, c["H"]), generator=g, device=dev, dtype=torch.float32))
    # first pass to learn the routing counts (and fill low-latency slots of y)
    moe.moe_dispatch_layout(ctx, idx, cnt_e, cnt_r, in_rank)
    moe.moe_dispatch(ctx, x, idx, reuse_layout=True, bufs=bufs, handle=h)
    torch.cuda.synchronize()
    n_pairs = int(h.expert_offsets[-1].item())
    n_send = int(h.rank_offsets[-1].item())
    if c["layout"] == 1:
        pos = h.pos[:c["T"]].flatten()
        pos = pos[pos >= 0].long()
        y[pos] = torch.randn((pos.numel(), c["H"]), generator=g, device=dev,
                             dtype=torch.float32).to(torch.bfloat16)
    st, _ = moe.moe_poll_error(ctx)
    assert st == moe.MOE_OK, st
    return {"d": d, "c": c, "ctx": ctx, "x": x, "idx": idx, "w": w, "bufs": bufs, "h": h,
            "cnt_e": cnt_e, "cnt_r": cnt_r, "in_rank": in_rank, "out": out, "y": y,
            "n_pairs": n_pairs, "n_send": n_send}


def step(moe, s):
    """Layout, dispatch reusing that layout, combine (the normal-mode call
    sequence).  The layout call is given x, so that its launch also reads the
    token rows into the Infinity Cache for the dispatch
    (moe_dispatch_layout_prefetch)."""
    moe.moe_dispatch_layout(s["ctx"], s["idx"], s["cnt_e"], s["cnt_r"], s["in_rank"], x=s["x"])
    moe.moe_dispatch(s["ctx"], s["x"], s["idx"], reuse_layout=True, bufs=s["bufs"], handle=s["h"])
    moe.moe_combine(s["ctx"], s["y"], s["w"], s["h"], out=s["out"])


def step_ll(moe, s):
    """Low-latency call sequence: dispatch straight from topk_idx (the routing is
    computed inside the fused dispatch launch), then combine."""
    moe.moe_dispatch(s["ctx"], s["x"], s["idx"], reuse_layout=False, bufs=s["bufs"], handle=s["h"])
    moe.moe_combine(s["ctx"], s["y"], s["w"], s["h"], out=s["out"])


def timed(moe, torch, s, steps, warmup, fn=step):
    """Wall-clock time of `steps` back-to-back steps, nothing else on the stream."""
    for _ in range(warmup):
        fn(moe, s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn(moe, s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st, _ = moe.moe_poll_error(s["ctx"])
    assert st == moe.MOE_OK, st
    return wall


def timed_graph(moe, torch, s, fn, steps_per_graph=100, replays=10):
    """Per-step time of `steps_per_graph` steps captured in one HIP graph and
    replayed: the GPU-side time of a step without host launch overhead (the
    library's calls only launch kernels on the capturing stream)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            fn(moe, s)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(steps_per_graph):
            fn(moe, s)
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(replays):
        g.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st, _ = moe.moe_poll_error(s["ctx"])
    assert st == moe.MOE_OK, st
    del g
    return wall / (replays * steps_per_graph)


def timed_cold(moe, torch, s, steps, warmup, flush, fn=step):
    """The headline protocol: `warmup` then `steps` steps, each preceded by
    `flush` (untimed); each timed step is bracketed by events on the current
    stream, where the library launches.  Returns (per-step ms, wall seconds
    of the whole timed loop, flushes included)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for _ in range(warmup):
        flush()
        fn(moe, s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        flush()
        ev[i][0].record()
        fn(moe, s)
        ev[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st, _ = moe.moe_poll_error(s["ctx"])
    assert st == moe.MOE_OK, st
    return [e0.elapsed_time(e1) for e0, e1 in ev], wall


def make_flushes(torch):
    """Cache flushes run before a step: "cold" rewrites a 1 GiB buffer (the
    headline protocol; its dirty lines are written back while the step runs),
    "cold_read" only reads it (evicts without leaving dirty lines)."""
    fbuf = torch.zeros(1 << 28, dtype=torch.float32, device="cuda")
    return {"cold": lambda: fbuf.add_(1), "cold_read": lambda: fbuf.sum()}


def timed_kernels(moe, torch, s, steps, flush=None, fn=step):
    """Per-kernel durations from the HIP events the library records around
    each of its launches, on its launch stream, over `steps` more steps.  The
    events add a few microseconds per launch, so this pass is kept apart from
    the wall-clock pass above.  With `flush` (a function), it runs before each
    step, outside the kernel events, so that the caches start cold."""
    s["ctx"].timing_begin(3 * steps + 3)
    for _ in range(steps):
        if flush is not None:
            flush()
        fn(moe, s)
    torch.cuda.synchronize()
    per = s["ctx"].timing_launches()
    kt = s["ctx"].timing_end()
    for name in kt:
        kt[name]["ms"] = [ms for n, ms in per if n == name]
    st, _ = moe.moe_poll_error(s["ctx"])
    assert st == moe.MOE_OK, st
    return kt


def overlap(moe, torch, s, fn, caps, iters=40):
    """A bf16 GEMM [T, H] x [H, H] on the main stream while the step runs on a
    side stream (issued there, completed on the main stream by a hook), for
    each workgroup cap.  Reports the GEMM alone, the step alone, and per cap
    the step alone, the overlapped iteration and the GEMM's own duration
    inside it (events on the main stream)."""
    c, dev = s["c"], s["x"].device
    T, H = c["T"], c["H"]
    g = torch.Generator(device=dev)
    g.manual_seed(99)
    a = torch.randn((T, H), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    b = torch.randn((H, H), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16).contiguous()
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    hook = moe.Hook()

    def gemm():
        torch.matmul(a, b, out=out)

    def wall(f, n):
        for _ in range(5):
            f()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            f()
        torch.cuda.synchronize()
        return 1e6 * (time.perf_counter() - t0) / n

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]

    def median_us():
        return 1e3 * sorted(e0.elapsed_time(e1) for e0, e1 in ev)[iters // 2]

    for _ in range(5):
        gemm()
    for i in range(iters):   # the GEMM alone, timed the same way as inside the overlap
        ev[i][0].record(main)
        gemm()
        ev[i][1].record(main)
    torch.cuda.synchronize()
    gemm_us = median_us()
    res = {"gemm": "bf16 [%d, %d] x [%d, %d]" % (T, H, H, H),
           "gemm_tflops": round(2.0 * T * H * H / (gemm_us * 1e-6) / 1e12, 1),
           "us_gemm_alone": round(gemm_us, 1), "caps": []}
    for cap in caps:
        s["ctx"].set_max_workgroups(cap)
        step_us = wall(lambda: fn(moe, s), iters)

        def both(i=None):
            if i is not None:
                ev[i][0].record(main)
            gemm()
            if i is not None:
                ev[i][1].record(main)
            with torch.cuda.stream(side):
                fn(moe, s)
            hook.record(side)
            hook.wait(main)

        for _ in range(5):
            both()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(iters):
            both(i)
        torch.cuda.synchronize()
        both_us = 1e6 * (time.perf_counter() - t0) / iters
        g_us = median_us()
        res["caps"].append({"max_workgroups": cap, "us_step_alone": round(step_us, 1),
                            "us_overlapped_iteration": round(both_us, 1),
                            "us_gemm_in_overlap": round(g_us, 1),
                            "gemm_slowdown": round(g_us / gemm_us, 3),
                            "serial_us": round(gemm_us + step_us, 1)})
    s["ctx"].set_max_workgroups(0)
    st, _ = moe.moe_poll_error(s["ctx"])
    assert st == moe.MOE_OK, st
    hook.close()
    return res


def copy_reference(torch, nbytes=1 << 30, reps=20):
    """Achievable HBM rate of a plain 1 GiB device-to-device copy on this GPU
    (read + write bytes / time, HIP events on the current stream)."""
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / (us * 1e-6) / 1e9


def all_configs(moe, W, torch, flushes, with_oracle=True):
    """Per workload (the layout-reusing step for the contiguous layout, the
    fused low-latency step for the padded one): the step time and algorithmic
    GB/s cold (the headline protocol, a 1 GiB write flush before each step)
    and warm (back to back), the step replayed from a HIP graph (no host
    launch cost; warm), and per kernel the p10/p50/p90 event durations
    warm and cold: 10 warm-up steps, then 1000 timed steps for the two
    latency-bound workloads and 100 for the others.  With `with_oracle`, also
    the oracle on the same inputs on one host core, layout, dispatch and
    combine timed separately (medians of 101 steps for the two latency-bound
    workloads, 3 for the others): a reported baseline, not a target."""
    out = {}
    for name in ("tiny", "decode", "prefill", "grouped", "skewed"):
        steps = 1000 if name in ("tiny", "decode") else 100
        s = setup(moe, W, torch, name)
        c = s["c"]
        T = c["T"]
        alg = algorithmic_bytes(c, T, s["n_send"], s["n_pairs"], T * c["k"])
        fn = step
        if c["layout"] == 1:
            fn = step_ll
            alg["layout"] = 0
        us = 1e6 * timed(moe, torch, s, steps, 10, fn=fn) / steps
        us_graph = 1e6 * timed_graph(moe, torch, s, fn)
        cold_ms, _ = timed_cold(moe, torch, s, steps, 10, flushes["cold"], fn=fn)
        us_cold = 1e3 * sum(cold_ms) / len(cold_ms)
        kt = timed_kernels(moe, torch, s, steps, fn=fn)
        kt_cold = {lb: timed_kernels(moe, torch, s, steps, flush=f, fn=fn) for lb, f in flushes.items()}
        b = sum(alg.values())
        out[name] = {"T": T, "H": c["H"], "E": c["E"], "R": c["R"], "k": c["k"],
                     "mode": ("fp8 " if c["quant"] else "bf16 ") + ("padded-LL" if c["layout"] else "send+contiguous"),
                     "us_per_step_cold": round(us_cold, 2),
                     "us_per_step_cold_p10_p50_p90": percentiles_us(cold_ms),
                     "GB/s_cold": round(b / (us_cold * 1e-6) / 1e9, 1),
                     "pct_of_hbm_peak_cold": round(100 * b / (us_cold * 1e-6) / 1e9 / HBM_PEAK_GBS, 1),
                     "us_per_step": round(us, 2), "us_per_step_graph": round(us_graph, 2),
                     "alg_bytes": b, "GB/s": round(b / (us * 1e-6) / 1e9, 1),
                     "pct_of_hbm_peak": round(100 * b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1),
                     "steps": steps, "kernels": kernel_table(kt, alg, cold=kt_cold)}
        if with_oracle:
            runs = 101 if name in ("tiny", "decode") else 3
            out[name]["oracle_cpu"] = dict(oracle_timing(s, runs=runs), cores=1)
        s["ctx"].close()
        del s
        torch.cuda.empty_cache()
    return out


def host_cpu():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def host_us_per_call(torch, fn, n=200):
    """Host time for one call to return (argument checks, marshalling and the
    enqueue; nothing synchronizes inside), median over n calls, in us."""
    import numpy as np
    torch.cuda.synchronize()
    ts = []
    for _ in range(n):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    torch.cuda.synchronize()
    return round(1e6 * float(np.median(ts)), 2)


def oracle_inputs(s):
    """What the oracle's combine reads: the expert outputs the GPU step reads,
    in the oracle's expert-major order.  In the padded mode those outputs sit
    at the oracle's own padded rows (`pos_ll`), gathered once, untimed, into
    its expert-major order, so that the combine sums the same values."""
    import numpy as np
    import oracle
    import torch
    d, c = s["d"], s["c"]
    ll = c["layout"] == 1
    kw = dict(quant=c["quant"], max_tokens=c["max_tokens"] if ll else 0, with_send=not ll)
    ref = oracle.dispatch(d["x"], d["topk_idx"], c["E"], c["R"], **kw)
    pos = ref["pos"]
    if ll:
        valid = pos >= 0
        src = torch.from_numpy(ref["pos_ll"][valid].astype(np.int64)).to(s["y"].device)
        y = np.empty((ref["n_pairs"], c["H"]), np.uint16)
        y[pos[valid]] = s["y"][src].cpu().view(torch.int16).numpy().view(np.uint16)
    else:
        y = s["y"][:ref["n_pairs"]].cpu().view(torch.int16).numpy().view(np.uint16)
    return y, kw


def oracle_ops(s, y, kw):
    """One oracle step, each op timed on its own (seconds): layout; positions
    and payload rows (the dispatch); combine."""
    import oracle
    d, c = s["d"], s["c"]
    t0 = time.perf_counter()
    lay = oracle.layout(d["topk_idx"], c["E"], c["R"])
    t1 = time.perf_counter()
    pp = oracle.positions(d["topk_idx"], c["E"], c["R"], lay, kw["max_tokens"])
    oracle.rows(d["x"], pp, kw["quant"], kw["with_send"])
    t2 = time.perf_counter()
    oracle.combine(y, d["topk_weights"], pp["pos"])
    t3 = time.perf_counter()
    return t1 - t0, t2 - t1, t3 - t2


def oracle_timing(s, runs=None, seconds=None, min_runs=3, max_runs=100000):
    """The oracle (single-threaded scalar C) on one workload, pinned to one host
    core: layout, dispatch (positions + payload rows as the workload's mode
    writes them) and combine, each timed on its own, over `runs` steps or
    until about `seconds` of CPU time (at least min_runs).  Returns the medians
    in ms and the number of steps run."""
    import numpy as np
    y, kw = oracle_inputs(s)
    saved = os.sched_getaffinity(0)
    os.sched_setaffinity(0, {min(saved)})
    per = []
    try:
        while True:
            per.append(oracle_ops(s, y, kw))
            n = len(per)
            if runs is not None and n >= runs:
                break
            if runs is None and n >= min_runs and (sum(map(sum, per)) >= seconds or n >= max_runs):
                break
    finally:
        os.sched_setaffinity(0, saved)
    a = 1e3 * np.asarray(per)
    return {"layout_ms": round(float(np.median(a[:, 0])), 4), "dispatch_ms": round(float(np.median(a[:, 1])), 4),
            "combine_ms": round(float(np.median(a[:, 2])), 4),
            "step_ms": round(float(np.median(a.sum(axis=1))), 4), "runs": len(per),
            "cpu_seconds": round(float(a.sum()) / 1e3, 2)}


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py drives a single GPU: the library has no multi-GPU path "
              "(peer transport is replaced by a local copy); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    if a.copy_calibration:
        torch.cuda.set_device(0)
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": 1 << 30, "copy_calibration_bytes_written": 1 << 30,
                          "copies": 5}), flush=True)
        return
    import combine_moe_dispatch_layout_amd as moe
    import workloads as W
    moe.load_library()
    torch.cuda.set_device(0)

    s = setup(moe, W, torch, a.workload, T=a.tokens)
    c = s["c"]
    T = c["T"]
    if a.step == "backward":
        setup_backward(torch, s)
        alg = backward_bytes(c, T, s["n_pairs"])
        fn = step_bwd
        step_desc = "dispatch backward + combine backward"
    else:
        alg = algorithmic_bytes(c, T, s["n_send"], s["n_pairs"], T * c["k"])
        fn = step_ll if c["layout"] == 1 else step
        if fn is step_ll:
            alg["layout"] = 0                     # the routing is read inside the fused dispatch
        step_desc = ("dispatch from topk_idx (fused) + combine" if fn is step_ll
                     else "layout (reading x into the Infinity Cache meanwhile) + dispatch(reuse layout) + combine")
    step_bytes = sum(alg.values())
    # the headline: W + K steps, each after a 1 GiB write flush, K of them timed with events
    flushes = make_flushes(torch)
    head_flush = flushes["cold"] if a.protocol == "cold" else (lambda: None)
    cold_ms, cold_wall = timed_cold(moe, torch, s, a.steps, a.warmup, head_flush, fn=fn)
    ms_per_step = sum(cold_ms) / len(cold_ms)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    # per-kernel durations (library events), cold; warm (back to back) and after a read flush beside
    passes = {"cold": timed_kernels(moe, torch, s, a.steps, flush=head_flush, fn=fn)}
    warm = None
    if not a.profile_only:
        wall = timed(moe, torch, s, a.steps, a.warmup, fn=fn)
        warm = {"ms_per_step": round(1e3 * wall / a.steps, 4),
                "value": round(step_bytes / (wall / a.steps) / 1e9, 1),
                "pct_of_hbm_peak": round(100 * step_bytes / (wall / a.steps) / 1e9 / HBM_PEAK_GBS, 1),
                "what": "the same %d steps back to back, no flush, wall clock" % a.steps}
        passes["warm"] = timed_kernels(moe, torch, s, a.steps, fn=fn)
        passes["cold_read"] = timed_kernels(moe, torch, s, a.steps, flush=flushes["cold_read"], fn=fn)
    per_kernel = kernel_passes(passes, alg, "cold")
    dom = max(per_kernel, key=lambda n: per_kernel[n]["us"])
    achieved = per_kernel[dom]["GB/s"]
    cold_pass = lambda fn_, steps_: {lb: timed_kernels(moe, torch, s, steps_, flush=f, fn=fn_)
                                     for lb, f in flushes.items()}

    line = {
        "metric": "dispatch+combine us/call and HBM GB/s (% of peak), 128 & 4096 tok x 7168, top-8",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "protocol": ("cold: a 1 GiB buffer rewritten (untimed) before every warm-up and timed step; "
                     "per-step HIP events on the launch stream; value = bytes / mean step"
                     if a.protocol == "cold" else
                     "warm (profiling run): steps back to back with per-step HIP events; value = bytes / mean step"),
        "us_per_step_p10_p50_p90": percentiles_us(cold_ms),
        "timed_loop_s_with_flushes": round(cold_wall, 4),
        "warm": warm,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3/bf16" if c["quant"] else "bf16",
        "data": "synthetic (seeded N(0,1) tokens and expert outputs, routing per workload)",
        "config": {"workload": "%s: T=%d H=%d E=%d R=%d top-%d %s %s" % (
            a.workload, T, c["H"], c["E"], c["R"], c["k"], "fp8" if c["quant"] else "bf16",
            "padded-LL" if c["layout"] else "send+contiguous"),
            "step": step_desc,
            "alg_bytes_per_step": step_bytes, "n_send_rows": s["n_send"], "n_recv_rows": s["n_pairs"],
            "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1)},
        "kernels": per_kernel,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "frac_cold": round(achieved / HBM_PEAK_GBS, 4),
                     "achieved_cold_p50": per_kernel[dom]["GB/s_cold_p50"],
                     "frac_cold_p50": round(per_kernel[dom]["GB/s_cold_p50"] / HBM_PEAK_GBS, 4),
                     "achieved_warm": per_kernel[dom].get("GB/s_warm"),
                     "frac_warm": (round(per_kernel[dom]["GB/s_warm"] / HBM_PEAK_GBS, 4)
                                   if "GB/s_warm" in per_kernel[dom] else None),
                     "alg_bytes_per_launch": per_kernel[dom]["alg_bytes"],
                     "note": ("the layout launch before the dispatch reads x into the Infinity Cache "
                              "(moe_dispatch_layout_prefetch), so the dispatch's cold reads of x hit there; "
                              "the step value counts the layout's time for it" if fn is step else None),
                     "us_per_launch": per_kernel[dom]["us"],
                     "traffic": traffic_for(dom, a.workload + ("_backward" if a.step == "backward" else ""))},
    }

    if not a.profile_only and not a.no_backward and a.step == "forward":
        setup_backward(torch, s)
        alg_b = backward_bytes(c, T, s["n_pairs"])
        wall_b = timed(moe, torch, s, a.steps, a.warmup, fn=step_bwd)
        kt_b = timed_kernels(moe, torch, s, a.steps, fn=step_bwd)
        us_b = 1e6 * wall_b / a.steps
        line["backward"] = {
            "workload": line["config"]["workload"],
            "step": "dispatch backward + combine backward",
            "us_per_step": round(us_b, 2),
            "alg_bytes_per_step": sum(alg_b.values()),
            "GB/s": round(sum(alg_b.values()) / (us_b * 1e-6) / 1e9, 1),
            "kernels": kernel_table(kt_b, alg_b, cold=cold_pass(step_bwd, min(a.steps, 100))),
            "traffic_bytes_per_launch": {k_: traffic_for(k_, a.workload + "_backward") for k_ in alg_b}}
        for key in ("grad_recv", "grad_out", "grad_x", "grad_y", "grad_w"):
            del s[key]
        torch.cuda.empty_cache()

    if not a.profile_only and not a.no_overlap and a.step == "forward":
        line["overlap"] = overlap(moe, torch, s, fn, [0, 1024, 512, 256, 128, 64])
        torch.cuda.empty_cache()

    if not a.profile_only and not a.no_decode and a.workload != "decode":
        sd = setup(moe, W, torch, "decode")
        wall_d = timed(moe, torch, sd, 500, 50, fn=step_ll)
        kt_d = timed_kernels(moe, torch, sd, 100, flush=flushes["cold"], fn=step_ll)
        kt_dr = timed_kernels(moe, torch, sd, 100, flush=flushes["cold_read"], fn=step_ll)
        alg_d = algorithmic_bytes(sd["c"], 128, 0, sd["n_pairs"], 128 * 8)
        ll_bytes = alg_d["dispatch"] + alg_d["combine"]      # routing is read inside dispatch
        warm_us = 1e6 * wall_d / 500
        graph_us = 1e6 * timed_graph(moe, torch, sd, step_ll)
        # each call on its own, 100 of it captured in a graph: the GPU time of one
        # call with no host launch overhead (kernel plus the boundary to the next)
        graph_call_us = {
            "dispatch": 1e6 * timed_graph(moe, torch, sd, lambda moe_, s_: moe_.moe_dispatch(
                s_["ctx"], s_["x"], s_["idx"], reuse_layout=False, bufs=s_["bufs"], handle=s_["h"])),
            "combine": 1e6 * timed_graph(moe, torch, sd, lambda moe_, s_: moe_.moe_combine(
                s_["ctx"], s_["y"], s_["w"], s_["h"], out=s_["out"]))}
        # the same step through prepared calls (arguments marshalled once): what a
        # lean host loop sees, launch overhead included
        pd = moe.prepare_dispatch(sd["ctx"], sd["x"], sd["idx"], False, sd["bufs"], sd["h"])
        pc = moe.prepare_combine(sd["ctx"], sd["y"], sd["w"], sd["h"], sd["out"], sd["c"]["T"])

        def step_prepared(moe_, s_):
            pd()
            pc()
        prep_us = 1e6 * timed(moe, torch, sd, 500, 50, fn=step_prepared) / 500
        host_calls = {
            "dispatch": host_us_per_call(torch, lambda: moe.moe_dispatch(
                sd["ctx"], sd["x"], sd["idx"], reuse_layout=False, bufs=sd["bufs"], handle=sd["h"])),
            "combine": host_us_per_call(torch, lambda: moe.moe_combine(sd["ctx"], sd["y"], sd["w"], sd["h"],
                                                                         out=sd["out"])),
            "dispatch_prepared": host_us_per_call(torch, pd),
            "combine_prepared": host_us_per_call(torch, pc)}
        cold = {n: 1e3 * kt_d[n]["total_ms"] / kt_d[n]["launches"] for n in ("dispatch", "combine")}
        cold_pct = {n: percentiles_us(kt_d[n]["ms"]) for n in ("dispatch", "combine")}
        cold_read_pct = {n: percentiles_us(kt_dr[n]["ms"]) for n in ("dispatch", "combine")}
        line["decode"] = {
            "workload": "decode: T=128 H=7168 E=256 R=32 top-8 fp8 padded-LL",
            "step": "dispatch from topk_idx (one fused launch) + combine",
            "us_per_step_warm": round(warm_us, 2),
            "us_per_step_graph": round(graph_us, 2),
            "us_per_call_graph": {k_: round(v, 2) for k_, v in graph_call_us.items()},
            "us_per_step_prepared_calls": round(prep_us, 2),
            "host_us_per_call": host_calls,
            "us_per_kernel_cold": {k_: round(v, 2) for k_, v in cold.items()},
            "us_per_kernel_cold_p10_p50_p90": cold_pct,
            "us_per_kernel_cold_read_p10_p50_p90": cold_read_pct,
            "alg_bytes_per_step": ll_bytes,
            "alg_bytes_per_call": {n: alg_d[n] for n in ("dispatch", "combine")},
            "GB/s_warm": round(ll_bytes / (warm_us * 1e-6) / 1e9, 1)}
        sd["ctx"].close()
        del sd
        torch.cuda.empty_cache()

    if "decode" in line and a.workload == "prefill" and a.step == "forward":
        # the metric's two sizes side by side: dispatch and combine, us per call
        def call(us, nbytes):
            gbs = nbytes / (us * 1e-6) / 1e9
            return {"us": us, "GB/s": round(gbs, 1), "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1)}
        dd = line["decode"]
        line["per_call"] = {
            "what": ("us per call: 4096 tokens cold (a 1 GiB write before each step; the library's events "
                     "around each launch), 128 tokens as graph nodes (100 calls captured, replayed)"),
            "4096_tokens": {n: call(per_kernel[n]["us"], per_kernel[n]["alg_bytes"]) for n in ("dispatch", "combine")},
            "128_tokens": {n: call(dd["us_per_call_graph"][n], dd["alg_bytes_per_call"][n])
                           for n in ("dispatch", "combine")}}

    if not a.profile_only:
        cp = copy_reference(torch)
        line["copy_reference"] = {"GB/s": round(cp, 1), "what": "1 GiB device-to-device copy, read + write bytes",
                                  "step_frac_of_copy": round(value / cp, 3),
                                  "dominant_kernel_frac_of_copy": round(achieved / cp, 3)}

    if not a.profile_only and not a.no_configs and a.step == "forward":
        line["configs"] = all_configs(moe, W, torch, flushes, with_oracle=not a.no_cpu_baseline)

    if not a.profile_only and not a.no_cpu_baseline and a.step == "forward":
        model, ncpu = host_cpu()
        o = oracle_timing(s, seconds=a.cpu_seconds)
        sec = o["step_ms"] * 1e-3
        line["cpu_baseline"] = {"value": round(step_bytes / sec / 1e9, 3), "unit": "GB/s", "cores": 1,
                                "kind": "oracle",
                                "layout_ms": o["layout_ms"], "dispatch_ms": o["dispatch_ms"],
                                "combine_ms": o["combine_ms"], "step_ms": o["step_ms"],
                                "cpu_model": model, "host_cores_visible": ncpu,
                                "sample": "the full %s workload (%d tokens): layout, then positions and "
                                          "payload rows (dispatch), then combine, each timed on its own in "
                                          "the scalar C oracle; medians of %d steps (%.1f s of CPU in all), "
                                          "pinned to one of %d host cores (%s)"
                                          % (a.workload, T, o["runs"], o["cpu_seconds"], ncpu, model)}
    print(json.dumps(line), flush=True)
    s["ctx"].close()


def traffic_for(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    counters, only while the kernel source is unchanged since they were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    src = os.path.join(ROOT, "combine_moe_dispatch_layout_amd", "csrc", "moe_kernels.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    ent = rec.get(workload, {}).get(kernel)
    if ent is None or ent.get("kernel_source_sha256") != sha:
        return None
    return ent.get("bytes_per_launch")


if __name__ == "__main__":
    main()
