"""GPU parity of the backward pass: moe_dispatch_backward and
moe_combine_backward (through the C ABI) against the CPU oracle.

Bar: grad_x and grad_expert_out bit-exact (both sides take the same binary32
operations in the same order and round once to bf16); grad_weights within the
rigorous bound for any summation order of the H exact bf16 products:
|gpu - exact| <= gamma_H * sum_h |go[t, h] * y[pos, h]| + H * 2^-126, with
gamma_H = H u / (1 - H u), u = 2^-24 (the oracle's binary64 value is the exact
dot product to ~2^-53 relative).  Gradient buffers are poisoned first, and
expert-output rows no slot points at are NaN, so stray writes and wrong reads
show up.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

GPOISON = 0x5A5A          # bf16 bits left in rows the backward must not write


def log(*a):
    print(*a, flush=True)


def dev():
    return torch.device("cuda", 0)


def to_dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def bits_of(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double().numpy()


def grad_w_bound(go_bits, y_rows_bits, pos):
    """gamma_H * sum |go * y| per (t, j), plus an underflow allowance."""
    T, k = pos.shape
    H = go_bits.shape[1]
    u = 2.0 ** -24
    gamma = H * u / (1 - H * u)
    go = np.abs(bf16_f64(go_bits))
    y = np.abs(bf16_f64(y_rows_bits))
    b = np.zeros((T, k))
    for j in range(k):
        v = pos[:, j] >= 0
        b[v, j] = np.einsum("th,th->t", go[v], y[pos[v, j]])
    return gamma * b + H * 2.0 ** -126


def run_backward(gpu, c, x_bits, idx, w, max_tokens=None, tune=None, tag="", repeat=1, max_workgroups=0,
                 src_rank=0):
    T = idx.shape[0]
    H = c["H"]
    ll = c["layout"] == W.LAYOUT_PADDED_LL
    log("backward case %s: T=%d H=%d E=%d R=%d k=%d quant=%d layout=%d tune=%s" %
        (tag, T, H, c["E"], c["R"], c["k"], c["quant"], c["layout"], tune))
    M = max_tokens if max_tokens is not None else max(c["max_tokens"], T, 1)
    ctx = gpu.Context(gpu.make_config(M, H, c["E"], c["R"], c["k"], src_rank, c["quant"], c["layout"]))
    if tune is not None:
        ctx.tune(0, tune)
    if max_workgroups:
        ctx.set_max_workgroups(max_workgroups)
    ref = oracle.dispatch(x_bits, idx, c["E"], c["R"], quant=c["quant"], max_tokens=M if ll else 0,
                          src_rank=src_rank, with_send=not ll)
    n_pairs = ref["n_pairs"]
    dst_np = ref["pos_ll"] if ll else ref["pos"]         # row in the GPU receive layout
    # expert-major row of each slot that was placed (low latency: rows past a
    # slot window are not placed and take no part in the backward either)
    pos = np.where(dst_np >= 0, ref["pos"], -1).astype(np.int32)
    valid = pos >= 0

    x = to_dev_bf16(x_bits) if T else torch.empty((0, H), dtype=torch.bfloat16, device=dev())
    idx_d = torch.from_numpy(np.ascontiguousarray(idx)).to(dev())
    w_d = torch.from_numpy(np.ascontiguousarray(w)).to(dev())
    bufs = gpu.DispatchBuffers(ctx)
    h = gpu.Handle(ctx)
    gpu.moe_dispatch(ctx, x, idx_d, reuse_layout=False, bufs=bufs, handle=h)
    st, flags = gpu.moe_poll_error(ctx)
    assert st in (gpu.MOE_OK, gpu.MOE_ERR_BAD_TOPK, gpu.MOE_ERR_CAPACITY), (st, flags)
    assert np.array_equal(bits_of(h.pos[:T]), dst_np), "handle pos"
    del bufs

    n_cap = ctx.hint(gpu.MOE_BUF_EXPERT_OUT) // (2 * H)
    dst = torch.from_numpy(dst_np[valid].astype(np.int64)).to(dev())
    src = pos[valid]                                     # expert-major row of the same slots

    def receive_layout(rows_bits):
        """bf16 rows in expert-major order -> the GPU receive layout, NaN elsewhere."""
        buf = torch.empty((n_cap, H), dtype=torch.bfloat16, device=dev())
        buf.view(torch.int16).fill_(0x7FC0)
        if n_pairs:
            buf[dst] = to_dev_bf16(rows_bits[src])
        return buf

    # ---- dispatch backward
    g = W.grad_rows({"cfg": dict(c, extra_seed=3)}, max(n_pairs, 1))
    g_d = receive_layout(g)
    gx_ref = oracle.dispatch_backward(g, pos)
    for rep in range(repeat):
        gx = torch.empty((max(T, 1), H), dtype=torch.bfloat16, device=dev())
        gx.view(torch.int16).fill_(GPOISON)
        gpu.moe_dispatch_backward(ctx, g_d, h, grad_x=gx)
        st, flags = gpu.moe_poll_error(ctx)
        assert st == gpu.MOE_OK, (st, flags)
        got = bits_of(gx[:T])
        n_diff = int((got != gx_ref).sum())
        log("  dispatch backward (call %d): %d of %d elements differ" % (rep, n_diff, got.size))
        assert n_diff == 0, "dispatch backward expected bit-exact"
    del g_d

    # ---- combine backward
    yv = W.expert_outputs({"cfg": c}, max(n_pairs, 1))
    y_d = receive_layout(yv)
    go = W.grad_rows({"cfg": dict(c, extra_seed=5)}, T) if T else np.zeros((0, H), np.uint16)
    go_d = to_dev_bf16(go) if T else torch.empty((0, H), dtype=torch.bfloat16, device=dev())
    gy_ref, gw_ref = oracle.combine_backward(go, w, yv, pos)
    bound = grad_w_bound(go, yv, pos)
    first = None
    for rep in range(repeat):
        gy = torch.empty((n_cap, H), dtype=torch.bfloat16, device=dev())
        gy.view(torch.int16).fill_(GPOISON)
        gw = torch.full((max(T, 1), c["k"]), float("nan"), dtype=torch.float32, device=dev())
        gpu.moe_combine_backward(ctx, go_d, w_d, y_d, h, grad_expert_out=gy, grad_weights=gw)
        st, flags = gpu.moe_poll_error(ctx)
        assert st == gpu.MOE_OK, (st, flags)
        if n_pairs:
            got = bits_of(gy[dst])
            assert np.array_equal(got, gy_ref[src]), "grad_expert_out rows"
        # nothing else written: count rows that lost the poison
        touched = 0
        for r0 in range(0, n_cap, 1 << 16):
            blk = gy[r0:r0 + (1 << 16)].view(torch.int16)
            touched += int((blk[:, :8] != GPOISON).any(dim=1).sum())
        assert touched == int(valid.sum()), ("grad_expert_out rows written", touched, int(valid.sum()))
        gwh = bits_of(gw[:T]).astype(np.float64)
        err = np.abs(gwh - gw_ref)
        assert np.all(gwh[~valid] == 0.0), "empty slot -> grad_w = 0"
        ratio = float((err / bound)[valid].max(initial=0.0))
        log("  combine backward (call %d): grad_w max error %.3g of the bound" % (rep, ratio))
        assert np.all(err <= bound), "grad_w outside the summation bound"
        if first is None:
            first = (bits_of(gy[dst]) if n_pairs else None, bits_of(gw[:T]))
        else:
            assert np.array_equal(bits_of(gw[:T]), first[1]), "grad_w not deterministic"
        del gy, gw
    del y_d
    ctx.close()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def small_cfg(name, H=512):
    c = dict(W.WORKLOADS[name])
    c["H"] = H
    return c


# ---------------------------------------------------------------- workloads
@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "grouped", "skewed"])
def test_backward_workload_full_size(gpu, name):
    d = W.make(name)
    run_backward(gpu, d["cfg"], d["x"], d["topk_idx"], d["topk_weights"], tag=name, repeat=2)


# ---------------------------------------------------------------- ragged / edge cases
@pytest.mark.parametrize("T", [0, 1, 63, 65, 257, 1000])
@pytest.mark.parametrize("name", ["prefill", "decode"])
def test_backward_ragged_tokens(gpu, name, T):
    c = small_cfg(name)
    d = W.make(name, T=T)
    c["max_tokens"] = max(T, 1)
    run_backward(gpu, c, d["x"][:, :c["H"]].copy(), d["topk_idx"], d["topk_weights"],
                 max_tokens=max(T, 1), tag="ragged-%s" % name)


@pytest.mark.parametrize("H", [8, 136, 520, 1032, 7168, 32768])
def test_backward_hidden_sizes(gpu, H):
    """One 16-byte chunk, ragged chunk tails, one and many row slices, the
    largest supported row."""
    c = dict(W.WORKLOADS["prefill"], H=H)
    T = 96
    rng = np.random.Generator(np.random.PCG64(H))
    idx = W.route_uniform(rng, T, c["E"], c["k"])
    x = W.to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    w = W.softmax_weights(rng, T, c["k"])
    c["max_tokens"] = T
    run_backward(gpu, c, x, idx, w, max_tokens=T, tag="H%d" % H)


@pytest.mark.parametrize("chunks", [1, 2, 4, 8, 16])
def test_backward_row_split(gpu, chunks):
    """Every slice width: 14 wavefronts per token (7168-wide rows, 1 chunk per
    lane) down to a single wavefront at 16 chunks per lane."""
    c = small_cfg("prefill", H=7168)
    d = W.make("prefill", T=200)
    c["max_tokens"] = 200
    run_backward(gpu, c, d["x"], d["topk_idx"], d["topk_weights"], max_tokens=200, tune=chunks,
                 tag="chunks%d" % chunks, repeat=2)


@pytest.mark.parametrize("max_wg", [1, 7, 100])
def test_backward_max_workgroups(gpu, max_wg):
    """Capped grids: each combine-backward block loops over several tokens,
    reusing its LDS reduction buffer."""
    c = small_cfg("prefill", H=7168)
    d = W.make("prefill", T=300)
    c["max_tokens"] = 300
    run_backward(gpu, c, d["x"], d["topk_idx"], d["topk_weights"], max_tokens=300,
                 tag="maxwg%d" % max_wg, max_workgroups=max_wg)


@pytest.mark.parametrize("T,k,H", [(300, 1, 1024), (64, 32, 1024), (65, 17, 1024), (64, 32, 7168),
                                   (33, 17, 32768), (40, 9, 7168)])
def test_backward_topk_extremes(gpu, T, k, H):
    """k = 1 up to 32 (above 8 slots a token gets at most 4 wavefronts, so the
    slices are wide)."""
    c = dict(index=11, T=T, H=H, E=64, R=8, k=k, quant=W.QUANT_BF16,
             layout=W.LAYOUT_CONTIGUOUS, max_tokens=T)
    rng = np.random.Generator(np.random.PCG64(T + 31 * k))
    idx = W.route_uniform(rng, T, c["E"], k)
    x = W.to_bf16_bits(rng.standard_normal((T, c["H"]), dtype=np.float32))
    w = W.softmax_weights(rng, T, k)
    run_backward(gpu, c, x, idx, w, max_tokens=T, tag="k%d-H%d" % (k, H))


@pytest.mark.parametrize("name", ["prefill", "decode"])
def test_backward_empty_slots(gpu, name):
    c = small_cfg(name, H=1024)
    d = W.make(name, T=128)
    idx = W.with_empty_slots(d["topk_idx"], 0.3)
    idx[5, :] = -1                       # a token with no expert
    idx[9, :] = 3                        # one expert in every slot
    c["max_tokens"] = 128
    run_backward(gpu, c, d["x"][:, :c["H"]].copy(), idx, d["topk_weights"], max_tokens=128,
                 tag="empty-%s" % name)


def test_backward_consecutive_calls_shrinking(gpu):
    """Two calls in a row on one context, the second with fewer tokens: nothing
    carries over from the first."""
    c = small_cfg("prefill", H=7168)
    d = W.make("prefill", T=300)
    ctx = gpu.Context(gpu.make_config(300, c["H"], c["E"], c["R"], c["k"], 0, c["quant"], c["layout"]))
    ctx.tune(0, 1)                       # 14 wavefronts per token
    bufs = gpu.DispatchBuffers(ctx)
    h = gpu.Handle(ctx)
    n_cap = ctx.hint(gpu.MOE_BUF_EXPERT_OUT) // (2 * c["H"])
    for T in (300, 77):
        log("consecutive combine backward: T=%d" % T)
        idx = d["topk_idx"][:T].copy()
        w = d["topk_weights"][:T].copy()
        ref = oracle.dispatch(d["x"][:T], idx, c["E"], c["R"], quant=0)
        n = ref["n_pairs"]
        gpu.moe_dispatch(ctx, to_dev_bf16(d["x"][:T]), torch.from_numpy(idx).to(dev()), bufs=bufs, handle=h)
        yv = W.expert_outputs({"cfg": c}, n)
        y = torch.empty((n_cap, c["H"]), dtype=torch.bfloat16, device=dev())
        y[:n] = to_dev_bf16(yv)
        go = W.grad_rows({"cfg": dict(c, extra_seed=T)}, T)
        gy, gw = gpu.moe_combine_backward(ctx, to_dev_bf16(go), torch.from_numpy(w).to(dev()), y, h)
        st, _ = gpu.moe_poll_error(ctx)
        assert st == gpu.MOE_OK
        gy_ref, gw_ref = oracle.combine_backward(go, w, yv, ref["pos"])
        assert np.array_equal(bits_of(gy[:n]), gy_ref[:n])
        err = np.abs(bits_of(gw).astype(np.float64) - gw_ref)
        assert np.all(err <= grad_w_bound(go, yv, ref["pos"]))
    ctx.close()


@pytest.mark.parametrize("name", ["prefill", "decode"])
def test_two_live_handles(gpu, name):
    """Handles are caller-owned storage: two dispatches on one context leave two
    live handles, and the first one still drives combine and both backward
    calls correctly after the second dispatch (micro-batches whose backward
    runs in reverse order)."""
    c = small_cfg(name, H=1024)
    ll = c["layout"] == W.LAYOUT_PADDED_LL
    H, k, M = c["H"], c["k"], 128
    ctx = gpu.Context(gpu.make_config(M, H, c["E"], c["R"], k, 0, c["quant"], c["layout"]))
    n_cap = ctx.hint(gpu.MOE_BUF_EXPERT_OUT) // (2 * H)
    batches = []
    for b, T in enumerate((120, 57)):
        d = W.make(name, T=T, extra_seed=b + 1)
        x = np.ascontiguousarray(d["x"][:, :H])
        ref = oracle.dispatch(x, d["topk_idx"], c["E"], c["R"], quant=c["quant"], max_tokens=M if ll else 0,
                              with_send=not ll)
        bufs, h = gpu.DispatchBuffers(ctx), gpu.Handle(ctx)
        gpu.moe_dispatch(ctx, to_dev_bf16(x), torch.from_numpy(d["topk_idx"]).to(dev()), bufs=bufs, handle=h)
        dst_np = ref["pos_ll"] if ll else ref["pos"]
        valid = ref["pos"] >= 0
        cfg_b = dict(c, extra_seed=b + 1)
        batches.append(dict(T=T, w=d["topk_weights"], ref=ref, bufs=bufs, h=h, dst_np=dst_np, valid=valid,
                            dst=torch.from_numpy(dst_np[valid].astype(np.int64)).to(dev()),
                            yv=W.expert_outputs({"cfg": cfg_b}, ref["n_pairs"]),
                            go=W.grad_rows({"cfg": cfg_b}, T),
                            g=W.grad_rows({"cfg": dict(cfg_b, extra_seed=b + 11)}, ref["n_pairs"])))
    st, flags = gpu.moe_poll_error(ctx)
    assert st == gpu.MOE_OK, (st, flags)

    def receive_layout(bt, rows_bits):
        buf = torch.empty((n_cap, H), dtype=torch.bfloat16, device=dev())
        buf.view(torch.int16).fill_(0x7FC0)
        buf[bt["dst"]] = to_dev_bf16(rows_bits[bt["ref"]["pos"][bt["valid"]]])
        return buf

    for b, bt in enumerate(batches):              # forward, the older handle first
        log("two live handles (%s): forward of batch %d (T=%d)" % (name, b, bt["T"]))
        assert np.array_equal(bits_of(bt["h"].pos[:bt["T"]]), bt["dst_np"]), "handle pos"
        got = bits_of(bt["bufs"].recv_rows[bt["dst"]].view(torch.uint8))
        assert np.array_equal(got, bt["ref"]["recv_rows"][bt["ref"]["pos"][bt["valid"]]].view(np.uint8))
        out = gpu.moe_combine(ctx, receive_layout(bt, bt["yv"]), torch.from_numpy(bt["w"]).to(dev()), bt["h"])
        assert np.array_equal(bits_of(out), oracle.combine(bt["yv"], bt["w"], bt["ref"]["pos"])), "combine"
    for b in (1, 0):                              # backward, the newer handle first
        bt = batches[b]
        log("two live handles (%s): backward of batch %d" % (name, b))
        pos = bt["ref"]["pos"]
        gx = gpu.moe_dispatch_backward(ctx, receive_layout(bt, bt["g"]), bt["h"])
        assert np.array_equal(bits_of(gx), oracle.dispatch_backward(bt["g"], pos)), "dispatch backward"
        gy, gw = gpu.moe_combine_backward(ctx, to_dev_bf16(bt["go"]), torch.from_numpy(bt["w"]).to(dev()),
                                          receive_layout(bt, bt["yv"]), bt["h"])
        gy_ref, gw_ref = oracle.combine_backward(bt["go"], bt["w"], bt["yv"], pos)
        assert np.array_equal(bits_of(gy[bt["dst"]]), gy_ref[pos[bt["valid"]]]), "combine backward rows"
        err = np.abs(bits_of(gw).astype(np.float64) - gw_ref)
        assert np.all(err <= grad_w_bound(bt["go"], bt["yv"], pos)), "grad_w outside the summation bound"
    st, flags = gpu.moe_poll_error(ctx)
    assert st == gpu.MOE_OK, (st, flags)
    ctx.close()


def test_backward_api_errors(gpu):
    c = small_cfg("prefill")
    ctx = gpu.Context(gpu.make_config(64, c["H"], c["E"], c["R"], c["k"], 0, 0, 0))
    other = gpu.Context(gpu.make_config(65, c["H"], c["E"], c["R"], c["k"], 0, 0, 0))
    h = gpu.Handle(ctx)
    bufs = gpu.DispatchBuffers(ctx)
    d = W.make("prefill", T=64)
    gpu.moe_dispatch(ctx, to_dev_bf16(d["x"][:, :c["H"]].copy()), torch.from_numpy(d["topk_idx"]).to(dev()),
                     bufs=bufs, handle=h)
    n_cap = max(ctx.hint(gpu.MOE_BUF_EXPERT_OUT), other.hint(gpu.MOE_BUF_EXPERT_OUT)) // (2 * c["H"])
    y = torch.zeros((n_cap, c["H"]), dtype=torch.bfloat16, device=dev())
    go = torch.zeros((64, c["H"]), dtype=torch.bfloat16, device=dev())
    w = torch.zeros((64, c["k"]), dtype=torch.float32, device=dev())
    with pytest.raises(gpu.MoeError) as e:
        gpu.moe_combine_backward(other, go, w, y, h)      # handle from another context
    assert e.value.status == gpu.MOE_ERR_HANDLE
    with pytest.raises(gpu.MoeError) as e:
        gpu.moe_dispatch_backward(other, y, h)
    assert e.value.status == gpu.MOE_ERR_HANDLE
    lib = gpu.load_library()
    import ctypes
    # misaligned gradient pointer
    st = lib.moe_dispatch_backward(ctx.handle, ctypes.c_void_p(y.data_ptr() + 2), ctypes.byref(h.c),
                                   ctypes.c_void_p(go.data_ptr()), None)
    assert st == gpu.MOE_ERR_INVALID_ARG
    st = lib.moe_combine_backward(ctx.handle, ctypes.c_void_p(go.data_ptr()), ctypes.c_void_p(w.data_ptr()),
                                  ctypes.c_void_p(y.data_ptr()), ctypes.byref(h.c), None,
                                  ctypes.c_void_p(w.data_ptr()), None)
    assert st == gpu.MOE_ERR_INVALID_ARG
    torch.cuda.synchronize()
    ctx.close()
    other.close()


@pytest.mark.parametrize("name,T", [("prefill", 700), ("decode", 128)])
def test_backward_graph_capture(gpu, name, T):
    """The backward calls only enqueue kernels, so a backward step captures into
    a HIP graph: replay it several times, with eager work and a synchronisation
    between replays, and compare every replay with the eager step."""
    c = small_cfg(name)
    d = W.make(name, T=T)
    c["max_tokens"] = T
    ctx = gpu.Context(gpu.make_config(T, c["H"], c["E"], c["R"], c["k"], 0, c["quant"], c["layout"]))
    x = to_dev_bf16(np.ascontiguousarray(d["x"][:, :c["H"]]))
    idx = torch.from_numpy(d["topk_idx"]).to(dev())
    w = torch.from_numpy(d["topk_weights"]).to(dev())
    bufs, h = gpu.DispatchBuffers(ctx), gpu.Handle(ctx)
    gpu.moe_dispatch(ctx, x, idx, bufs=bufs, handle=h)
    n_cap = ctx.hint(gpu.MOE_BUF_EXPERT_OUT) // (2 * c["H"])
    g = torch.Generator(device=dev())
    g.manual_seed(11)
    grad_recv = torch.randn((n_cap, c["H"]), generator=g, device=dev()).to(torch.bfloat16)
    y = torch.randn((n_cap, c["H"]), generator=g, device=dev()).to(torch.bfloat16)
    grad_out = torch.randn((T, c["H"]), generator=g, device=dev()).to(torch.bfloat16)
    grad_x = torch.empty((T, c["H"]), dtype=torch.bfloat16, device=dev())
    grad_y = torch.empty_like(y)
    grad_w = torch.empty((T, c["k"]), dtype=torch.float32, device=dev())

    def step():
        gpu.moe_dispatch_backward(ctx, grad_recv, h, grad_x=grad_x)
        gpu.moe_combine_backward(ctx, grad_out, w, y, h, grad_expert_out=grad_y, grad_weights=grad_w)

    watch = [grad_x, grad_y, grad_w]
    for t in watch:
        t.view(torch.uint8).fill_(0x5A)
    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in watch]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        log("backward graph replay %d (%s)" % (rep, name))
        for t in watch:                       # eager work between replays
            t.view(torch.uint8).fill_(0x5A)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (t, e) in enumerate(zip(watch, eager)):
            assert torch.equal(t.view(torch.uint8), e.view(torch.uint8)), ("replay", rep, "tensor", i)
    st, _ = gpu.moe_poll_error(ctx)
    assert st == gpu.MOE_OK
    del graph
    ctx.close()
