"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bar: bit-exact for counts, offsets, positions, source indices, token->rank map,
payload rows (bf16 bytes, fp8 codes and fp32 scales); combine within one bf16
ulp (the kernel also uses separately rounded multiply and add, so it is
expected -- and checked separately -- to be bit-exact).  Output buffers are
poisoned first so stray or missing writes show up; combine inputs outside the
routed rows are NaN so a wrong read shows up.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import pins
import workloads as W

pytestmark = pytest.mark.gpu

POISON = 0xA5


def log(*a):
    print(*a, flush=True)


def dev():
    return torch.device("cuda", 0)


def to_dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def bits_of(t):
    """Device tensor -> host numpy array of raw bit patterns."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def make_ctx(gpu, c, T, max_tokens=None, src_rank=0):
    M = max_tokens if max_tokens is not None else max(c["max_tokens"], T, 1)
    cfg = gpu.make_config(M, c["H"], c["E"], c["R"], c["k"], src_rank, c["quant"], c["layout"])
    return gpu.Context(cfg)


def poison(bufs):
    for t in (bufs.send_rows, bufs.recv_rows, bufs.send_scales, bufs.recv_scales):
        if t is not None:
            t.view(torch.uint8).fill_(POISON)


def run_case(gpu, c, x_bits, idx, w, reuse=True, max_tokens=None, src_rank=0, check_poison=True,
             tag="", max_workgroups=0, side_stream=False, tune=None, ctx=None, prefetch=False):
    """Layout + dispatch + combine on the GPU and in the oracle; compare all.
    ctx: an existing context to run on (kept open), else a fresh one.
    prefetch: give the layout call x (moe_dispatch_layout_prefetch)."""
    T = idx.shape[0]
    ll = c["layout"] == W.LAYOUT_PADDED_LL
    fp8 = c["quant"] == W.QUANT_FP8
    log("case %s: T=%d H=%d E=%d R=%d k=%d quant=%d layout=%d reuse=%s s0=%d max_wg=%d side=%s prefetch=%s" %
        (tag, T, c["H"], c["E"], c["R"], c["k"], c["quant"], c["layout"], reuse, src_rank, max_workgroups,
         side_stream, prefetch))
    own_ctx = ctx is None
    if own_ctx:
        ctx = make_ctx(gpu, c, T, max_tokens, src_rank)
    if max_workgroups:
        ctx.set_max_workgroups(max_workgroups)
    if tune is not None:
        ctx.tune(*tune)                          # (dispatch, combine) chunks per lane
    M = ctx.cfg.max_tokens
    ref = oracle.dispatch(x_bits, idx, c["E"], c["R"], quant=c["quant"],
                          max_tokens=M if ll else 0, src_rank=src_rank, with_send=not ll)
    x = to_dev_bf16(x_bits) if T else torch.empty((0, c["H"]), dtype=torch.bfloat16, device=dev())
    idx_d = torch.from_numpy(np.ascontiguousarray(idx)).to(dev())
    w_d = torch.from_numpy(np.ascontiguousarray(w)).to(dev())
    bufs = gpu.DispatchBuffers(ctx)
    poison(bufs)
    h = gpu.Handle(ctx)
    h.pos.fill_(-7)

    # ---- layout
    cnt_e, cnt_r, in_rank = gpu.moe_dispatch_layout(ctx, idx_d, x=x if prefetch else None)
    # ---- dispatch (optionally issued on a side stream and completed by a hook)
    if side_stream:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        hook = gpu.Hook()
        with torch.cuda.stream(side):
            gpu.moe_dispatch(ctx, x, idx_d, reuse_layout=reuse, bufs=bufs, handle=h)
        hook.record(side)
        # unrelated work on the main stream while the dispatch runs
        a = torch.randn((2048, 2048), device=dev(), dtype=torch.float32)
        (a @ a).sum()
        hook.wait()
        hook.close()
    else:
        gpu.moe_dispatch(ctx, x, idx_d, reuse_layout=reuse, bufs=bufs, handle=h)
    st, flags = gpu.moe_poll_error(ctx)
    want = gpu.MOE_OK
    if ref["bad_ids"]:
        want = gpu.MOE_ERR_BAD_TOPK
    elif ll and ref["ll_overflow"]:
        want = gpu.MOE_ERR_CAPACITY          # rows past a slot window are not placed
    assert st == want, (st, flags)

    assert np.array_equal(bits_of(cnt_e), ref["num_tokens_per_expert"]), "num_tokens_per_expert"
    assert np.array_equal(bits_of(cnt_r), ref["num_tokens_per_rank"]), "num_tokens_per_rank"
    assert np.array_equal(bits_of(in_rank), ref["is_token_in_rank"]), "is_token_in_rank"
    n_send, n_pairs = ref["n_send"], ref["n_pairs"]
    assert np.array_equal(bits_of(h.expert_offsets), ref["expert_offsets"]), "expert_offsets"
    assert np.array_equal(bits_of(h.rank_offsets), ref["rank_offsets"]), "rank_offsets"
    assert np.array_equal(bits_of(h.recv_counts), ref["num_tokens_per_expert"]), "recv_counts"
    pos_ref = ref["pos_ll"] if ll else ref["pos"]
    assert np.array_equal(bits_of(h.pos[:T]), pos_ref), "handle pos"
    assert np.array_equal(bits_of(h.recv_src_idx[:n_pairs]), ref["recv_src_idx"]), "recv_src_idx"
    if not ll:
        assert np.array_equal(bits_of(h.send_src_idx[:n_send]), ref["send_src_idx"]), "send_src_idx"

    # ---- payload rows (low latency: the rows that were placed)
    valid = (pos_ref >= 0) & (ref["pos"] >= 0)
    pos_eff = np.where(valid, ref["pos"], -1).astype(np.int32)   # expert-major row of each placed slot
    n_placed = int(valid.sum())
    rowdt = np.uint8 if fp8 else np.uint16
    if ll:
        dst = torch.from_numpy(pos_ref[valid].astype(np.int64)).to(dev())
        got = bits_of(bufs.recv_rows[dst]).view(rowdt)
        assert np.array_equal(got, ref["recv_rows"][ref["pos"][valid]]), "LL receive rows"
        if fp8:
            assert np.array_equal(bits_of(bufs.recv_scales[dst]), ref["recv_scales"][ref["pos"][valid]])
        if check_poison:
            # exactly the routed slots were written
            r8 = bufs.recv_rows.view(torch.uint8)
            rows = r8.view(c["E"], -1, r8.shape[1])
            written = 0
            for e0 in range(0, c["E"], 16):
                blk = rows[e0:e0 + 16]
                written += int((blk[:, :, :64] != POISON).any(dim=2).sum())
            assert written == n_placed, ("LL slots written", written, n_placed)
    else:
        got = bits_of(bufs.recv_rows[:n_pairs]).view(rowdt)
        assert np.array_equal(got, ref["recv_rows"]), "expert-major receive rows"
        got = bits_of(bufs.send_rows[:n_send]).view(rowdt)
        assert np.array_equal(got, ref["send_rows"]), "send rows"
        if fp8:
            assert np.array_equal(bits_of(bufs.recv_scales[:n_pairs]), ref["recv_scales"])
            assert np.array_equal(bits_of(bufs.send_scales[:n_send]), ref["send_scales"])
        if check_poison:
            for t, n in ((bufs.recv_rows, n_pairs), (bufs.send_rows, n_send),
                         (bufs.recv_scales, n_pairs), (bufs.send_scales, n_send)):
                if t is not None and n < t.shape[0]:
                    assert bool((t[n:].view(torch.uint8) == POISON).all()), "stray write past the valid rows"

    # ---- combine: N(0,1) expert outputs at the routed rows, NaN elsewhere
    n_cap = ctx.hint(gpu.MOE_BUF_EXPERT_OUT) // (2 * c["H"])
    y = torch.empty((n_cap, c["H"]), dtype=torch.bfloat16, device=dev())
    y.view(torch.int16).fill_(0x7FC0)
    yv = W.expert_outputs({"cfg": c}, n_pairs)
    if n_pairs:
        if ll:
            y[dst] = to_dev_bf16(yv[ref["pos"][valid]])
        else:
            y[:n_pairs] = to_dev_bf16(yv)
    out = gpu.moe_combine(ctx, y, w_d, h)
    st, flags = gpu.moe_poll_error(ctx)
    assert st == gpu.MOE_OK, (st, flags)
    out_ref = oracle.combine(yv, w, pos_eff)
    got = bits_of(out)
    d = np.abs(pins.bf16_ordered(got) - pins.bf16_ordered(out_ref))
    n_diff = int((d != 0).sum())
    log("  combine: %d of %d elements differ from the oracle, max %d ulp" % (n_diff, d.size, d.max(initial=0)))
    assert d.max(initial=0) <= 1, "combine beyond 1 bf16 ulp"
    assert n_diff == 0, "combine expected bit-exact (separately rounded fp32 multiply and add)"
    del y
    if own_ctx:
        ctx.close()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return ref


# ---------------------------------------------------------------- workloads
@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "grouped", "skewed"])
def test_workload_full_size(gpu, name):
    d = W.make(name)
    run_case(gpu, d["cfg"], d["x"], d["topk_idx"], d["topk_weights"], reuse=True, tag=name)


@pytest.mark.parametrize("name", ["prefill", "grouped", "skewed", "tiny"])
def test_workload_layout_with_prefetch(gpu, name):
    """The layout launch that also reads x into the Infinity Cache gives the
    same layout (full size: the extra workgroups run; tiny: below the size at
    which they are launched)."""
    d = W.make(name)
    run_case(gpu, d["cfg"], d["x"], d["topk_idx"], d["topk_weights"], reuse=True, tag=name + "-prefetch",
             prefetch=True)


@pytest.mark.parametrize("T", [1, 300, 17000])
def test_layout_prefetch_ragged(gpu, T):
    """Ragged batches through the prefetching layout: one tile, per-tile sums,
    stored per-tile prefixes (x of 17000 tokens is larger than the part read)."""
    c = small_cfg("prefill", H=4096)
    d = W.make("prefill", T=T)
    run_case(gpu, c, d["x"][:, :4096].copy(), d["topk_idx"], d["topk_weights"], max_tokens=T,
             tag="prefetch-ragged", prefetch=True)


@pytest.mark.parametrize("name", ["tiny", "decode", "grouped"])
def test_workload_without_layout_reuse(gpu, name):
    d = W.make(name, T=min(W.WORKLOADS[name]["T"], 1024))
    run_case(gpu, d["cfg"], d["x"], d["topk_idx"], d["topk_weights"], reuse=False, tag=name)


# ---------------------------------------------------------------- ragged / edge cases
def small_cfg(name, H=512):
    c = dict(W.WORKLOADS[name])
    c["H"] = H
    return c


@pytest.mark.parametrize("T", [0, 1, 63, 64, 65, 255, 256, 257, 1000])
@pytest.mark.parametrize("name", ["prefill", "grouped", "decode"])
def test_ragged_token_counts(gpu, name, T):
    c = small_cfg(name)
    d = W.make(name, T=T)
    x = d["x"][:, :c["H"]].copy()
    M = max(T, 1) + 37 if c["layout"] == W.LAYOUT_CONTIGUOUS else max(T, 1)
    c["max_tokens"] = M
    run_case(gpu, c, x, d["topk_idx"], d["topk_weights"], max_tokens=M, tag="ragged-%s" % name)


@pytest.mark.parametrize("name", ["prefill", "decode"])
def test_empty_slots(gpu, name):
    c = small_cfg(name)
    d = W.make(name, T=300)
    idx = W.with_empty_slots(d["topk_idx"], 0.3)
    idx[5, :] = -1                       # a token with no expert at all
    run_case(gpu, c, d["x"][:, :c["H"]].copy(), idx, d["topk_weights"], max_tokens=300, tag="empty-slots")


def test_all_tokens_one_expert(gpu):
    c = small_cfg("skewed", H=256)
    T = 2000
    d = W.make("skewed", T=T)
    idx = np.full((T, c["k"]), -1, np.int64)
    idx[:, 0] = 7                        # every token to expert 7 (one huge segment)
    idx[::3, 1] = 63
    run_case(gpu, c, d["x"][:, :256].copy(), idx, d["topk_weights"], max_tokens=T, tag="one-expert")


def test_duplicate_experts_in_a_row(gpu):
    c = small_cfg("prefill", H=256)
    T = 700
    rng = np.random.Generator(np.random.PCG64(9))
    idx = rng.integers(0, 4, (T, c["k"])).astype(np.int64)    # many repeats within rows
    d = W.make("prefill", T=T)
    run_case(gpu, c, d["x"][:, :256].copy(), idx, d["topk_weights"], max_tokens=T, tag="duplicates")


def test_bad_expert_ids(gpu):
    c = small_cfg("grouped", H=256)
    T = 400
    d = W.make("grouped", T=T)
    idx = d["topk_idx"].copy()
    idx[3, 2] = c["E"]            # out of range -> error flag, slot treated as empty
    idx[10, 0] = -5
    idx[399, 7] = 1 << 40
    run_case(gpu, c, d["x"][:, :256].copy(), idx, d["topk_weights"], max_tokens=T, tag="bad-ids")


def test_low_latency_other_source_rank(gpu):
    c = small_cfg("decode")
    d = W.make("decode", T=100)
    run_case(gpu, c, d["x"][:, :c["H"]].copy(), d["topk_idx"], d["topk_weights"], max_tokens=128,
             src_rank=c["R"] - 3, tag="ll-s0")


def test_limits(gpu):
    """Largest supported expert count, rank count and top-k at once."""
    c = dict(index=9, T=3000, H=128, E=1024, R=64, k=32, quant=W.QUANT_FP8,
             layout=W.LAYOUT_CONTIGUOUS, max_tokens=3000)
    rng = np.random.Generator(np.random.PCG64(4))
    idx = W.route_uniform(rng, c["T"], c["E"], c["k"])
    x = W.to_bf16_bits(rng.standard_normal((c["T"], c["H"]), dtype=np.float32))
    w = W.softmax_weights(rng, c["T"], c["k"])
    run_case(gpu, c, x, idx, w, max_tokens=c["T"], tag="limits")


@pytest.mark.parametrize("quant,layout,T,k", [(W.QUANT_BF16, W.LAYOUT_CONTIGUOUS, 300, 8),
                                              (W.QUANT_FP8, W.LAYOUT_CONTIGUOUS, 300, 8),
                                              (W.QUANT_FP8, W.LAYOUT_PADDED_LL, 600, 4)])
def test_max_hidden(gpu, quant, layout, T, k):
    """The largest supported hidden size (32768: 4096 16-byte chunks per bf16
    row) on the send + contiguous path and on the two-launch low-latency path
    (T above the fused launch's limit)."""
    c = dict(index=11, T=T, H=32768, E=16, R=4, k=k, quant=quant, layout=layout, max_tokens=T)
    rng = np.random.Generator(np.random.PCG64(32768 + quant + 2 * layout))
    idx = W.route_uniform(rng, T, c["E"], k)
    x = W.to_bf16_bits(rng.standard_normal((T, c["H"]), dtype=np.float32))
    w = W.softmax_weights(rng, T, k)
    run_case(gpu, c, x, idx, w, reuse=(layout == W.LAYOUT_CONTIGUOUS), max_tokens=T, tag="max-hidden")


# ---------------------------------------------------------------- fp8 codec
def test_fp8_codec_exhaustive_bf16(gpu):
    """Blocks whose max is 448 quantise with scale exactly 1, so the GPU's
    E4M3 conversion is compared on every finite bf16 value of magnitude <= 448
    (ties, subnormal codes, signed zeros) -- and on a second scale (block max
    3.0, scale 448/3) that exercises full binary32 products."""
    v = pins.all_bf16_finite_f32()
    v = v[np.abs(v) <= 448]
    for amax in (448.0, 3.0):
        vv = v[np.abs(v) <= amax]
        per_row = 127 * 8               # 8 blocks of 128 (one slot per block holds amax)
        n = -(-vv.size // per_row)
        flat = np.zeros(n * per_row, np.float32)
        flat[:vv.size] = vv
        blocks = np.zeros((n * 8, 128), np.float32)
        blocks[:, :127] = flat.reshape(n * 8, 127)
        blocks[:, 127] = amax
        x = W.to_bf16_bits(blocks.reshape(n, 1024))
        c = dict(index=8, T=n, H=1024, E=8, R=2, k=1, quant=W.QUANT_FP8,
                 layout=W.LAYOUT_CONTIGUOUS, max_tokens=n)
        idx = np.zeros((n, 1), np.int64)
        idx[:, 0] = np.arange(n) % 8
        w = np.ones((n, 1), np.float32)
        ref = run_case(gpu, c, x, idx, w, max_tokens=n, tag="codec-amax%g" % amax)
        if amax == 448.0:
            q, _ = oracle.quant_rows(x)
            assert np.array_equal(q.reshape(-1, 128)[:, :127].ravel()[:vv.size], pins.brute_e4m3_encode(vv))
        del ref


# ---------------------------------------------------------------- round trip
@pytest.mark.parametrize("name", ["prefill", "skewed"])
def test_identity_expert_roundtrip(gpu, name):
    """Dispatch, identity expert (y = received rows), combine with weights
    summing to one: the output is x (the method's defining invariant)."""
    d = W.make(name, T=1024)
    c = d["cfg"]
    ctx = make_ctx(gpu, c, 1024)
    x = to_dev_bf16(d["x"])
    idx = torch.from_numpy(d["topk_idx"]).to(dev())
    w = torch.from_numpy(d["topk_weights"]).to(dev())
    bufs, h = gpu.moe_dispatch(ctx, x, idx)
    out = gpu.moe_combine(ctx, bufs.recv_rows, w, h)
    xb = d["x"].copy()
    xb[xb == 0x8000] = 0
    assert np.array_equal(bits_of(out), xb)
    ctx.close()


# ---------------------------------------------------------------- API errors
def test_api_errors(gpu):
    c = small_cfg("prefill", H=256)
    d = W.make("prefill", T=64)
    ctx = make_ctx(gpu, c, 64, max_tokens=64)
    x = to_dev_bf16(d["x"][:, :256].copy())
    idx = torch.from_numpy(d["topk_idx"]).to(dev())
    w = torch.from_numpy(d["topk_weights"]).to(dev())
    # reuse without a matching layout
    with pytest.raises(gpu.MoeError) as e:
        gpu.moe_dispatch(ctx, x, idx, reuse_layout=True)
    assert e.value.status == gpu.MOE_ERR_INVALID_ARG
    gpu.moe_dispatch_layout(ctx, idx)
    with pytest.raises(gpu.MoeError):
        gpu.moe_dispatch(ctx, x, idx.clone(), reuse_layout=True)   # another topk_idx buffer
    # capacity
    big = W.make("prefill", T=65)
    with pytest.raises(gpu.MoeError) as e:
        gpu.moe_dispatch(ctx, to_dev_bf16(big["x"][:, :256].copy()),
                         torch.from_numpy(big["topk_idx"]).to(dev()))
    assert e.value.status == gpu.MOE_ERR_CAPACITY
    # handle from another configuration is refused before anything is launched
    bufs, h = gpu.moe_dispatch(ctx, x, idx)
    c2 = dict(c)
    c2["k"] = 4
    ctx2 = make_ctx(gpu, c2, 64, max_tokens=64)
    y = torch.zeros((64 * 8, 256), dtype=torch.bfloat16, device=dev())
    lib = gpu.load_library()
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    assert lib.moe_combine(ctx2.handle, p(y), p(w), ctypes.byref(h.c), p(y), None) == gpu.MOE_ERR_HANDLE
    bad = gpu._binding.moe_handle.from_buffer_copy(h.c)
    bad.num_tokens = 65
    assert lib.moe_combine(ctx.handle, p(y), p(w), ctypes.byref(bad), p(y), None) == gpu.MOE_ERR_HANDLE
    st, _ = gpu.moe_poll_error(ctx)
    assert st == gpu.MOE_OK
    ctx.close()
    ctx2.close()


def test_binding_rejects_buffers_of_another_configuration(gpu):
    """The binding checks caller-supplied buffers, handles and outputs against
    the sizes the context's configuration needs before anything is launched
    (the C ABI takes raw pointers and cannot)."""
    c = small_cfg("prefill", H=256)
    d = W.make("prefill", T=64)
    small = make_ctx(gpu, c, 32, max_tokens=32)
    big = make_ctx(gpu, c, 64, max_tokens=64)
    x = to_dev_bf16(d["x"][:, :256].copy())
    idx = torch.from_numpy(d["topk_idx"]).to(dev())
    w = torch.from_numpy(d["topk_weights"]).to(dev())
    h_small, b_small = gpu.Handle(small), gpu.DispatchBuffers(small)
    h_big, b_big = gpu.Handle(big), gpu.DispatchBuffers(big)
    with pytest.raises(ValueError, match="handle"):
        gpu.moe_dispatch(big, x, idx, bufs=b_big, handle=h_small)
    with pytest.raises(ValueError, match="dispatch buffers"):
        gpu.moe_dispatch(big, x, idx, bufs=b_small, handle=h_big)
    with pytest.raises(ValueError, match="handle"):
        gpu.prepare_dispatch(big, x, idx, False, b_big, h_small)
    # a struct that no longer points at its tensors
    h_swapped = gpu.Handle(big)
    h_swapped.pos = torch.empty_like(h_swapped.pos)
    with pytest.raises(ValueError, match="no longer points"):
        gpu.moe_dispatch(big, x, idx, bufs=b_big, handle=h_swapped)
    # outputs too small or of the wrong type
    with pytest.raises(ValueError, match="is_token_in_rank"):
        gpu.moe_dispatch_layout(big, idx, is_token_in_rank=torch.empty((63, c["R"]), dtype=torch.uint8,
                                                                        device=dev()))
    with pytest.raises(TypeError, match="num_tokens_per_expert"):
        gpu.moe_dispatch_layout(big, idx, num_tokens_per_expert=torch.empty(c["E"], dtype=torch.int64,
                                                                             device=dev()))
    gpu.moe_dispatch(big, x, idx, bufs=b_big, handle=h_big)
    y = torch.zeros((big.hint(gpu.MOE_BUF_EXPERT_OUT) // 512, 256), dtype=torch.bfloat16, device=dev())
    with pytest.raises(ValueError, match="out"):
        gpu.moe_combine(big, y, w, h_big, out=torch.empty((63, 256), dtype=torch.bfloat16, device=dev()))
    # the same objects pass for a context of the same configuration, and the run is clean
    out = gpu.moe_combine(big, y, w, h_big)
    st, _ = gpu.moe_poll_error(big)
    assert st == gpu.MOE_OK and tuple(out.shape) == (64, 256)
    small.close()
    big.close()


def test_timing_api(gpu):
    d = W.make("tiny")
    c = d["cfg"]
    ctx = make_ctx(gpu, c, 16)
    x = to_dev_bf16(d["x"])
    idx = torch.from_numpy(d["topk_idx"]).to(dev())
    ctx.timing_begin(16)
    for _ in range(3):
        gpu.moe_dispatch_layout(ctx, idx)
        gpu.moe_dispatch(ctx, x, idx, reuse_layout=True)
    per = ctx.timing_launches()
    assert [n for n, _ in per] == ["layout", "dispatch"] * 3, per
    assert all(ms > 0 for _, ms in per)
    r = ctx.timing_end()
    assert r["layout"]["launches"] == 3 and r["dispatch"]["launches"] == 3
    assert r["combine"]["launches"] == 0
    assert r["dispatch"]["total_ms"] > 0
    for name in ("layout", "dispatch"):   # per-launch durations add up to the totals
        tot = sum(ms for n, ms in per if n == name)
        assert abs(tot - r[name]["total_ms"]) <= 1e-6 * max(1.0, tot), (name, tot, r[name])
    with pytest.raises(gpu.MoeError):     # no open timing window
        ctx.timing_launches()
    ctx.close()


def test_native_library_is_in_tree(gpu):
    import os
    lib = gpu.load_library()
    assert os.path.dirname(os.path.abspath(lib._name)) == os.path.dirname(os.path.abspath(gpu.LIB_PATH))


@pytest.mark.parametrize("E,R,k", [(1024, 1, 8), (64, 64, 8), (96, 3, 5), (1024, 64, 17)])
def test_expert_rank_extremes(gpu, E, R, k):
    """One rank holding every expert, one expert per rank, and odd sizes."""
    T = 777
    c = dict(index=10, T=T, H=128, E=E, R=R, k=k, quant=W.QUANT_BF16,
             layout=W.LAYOUT_CONTIGUOUS, max_tokens=T)
    rng = np.random.Generator(np.random.PCG64(E + R + k))
    idx = W.route_uniform(rng, T, E, k)
    x = W.to_bf16_bits(rng.standard_normal((T, 128), dtype=np.float32))
    w = W.softmax_weights(rng, T, k)
    run_case(gpu, c, x, idx, w, max_tokens=T, tag="extremes")


# ---------------------------------------------------------------- launch-geometry overrides
@pytest.mark.parametrize("chunks", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("name,H", [("prefill", 7168), ("prefill", 2176), ("grouped", 7168), ("decode", 2176)])
def test_row_split_overrides(gpu, name, H, chunks):
    """Every chunks-per-lane setting of moe_ctx_tune for the dispatch and the
    combine (1-16; the defaults use 1 and 2) gives the oracle's bytes, on full
    and ragged rows; the low-latency case runs layout + pack (T above the
    fused launch's limit)."""
    c = small_cfg(name, H=H)
    T = 600
    d = W.make(name, T=T)
    c["max_tokens"] = T
    run_case(gpu, c, np.ascontiguousarray(d["x"][:, :H]), d["topk_idx"], d["topk_weights"], max_tokens=T,
             reuse=(name != "decode"), tag="tune-%s-%d-%d" % (name, H, chunks), tune=(chunks, chunks))


# ---------------------------------------------------------------- resource control and hooks
@pytest.mark.parametrize("max_wg", [1, 3, 64, 1000])
@pytest.mark.parametrize("name,T", [("prefill", 700), ("grouped", 700), ("decode", 700), ("decode", 128)])
def test_max_workgroups_same_results(gpu, name, T, max_wg):
    """A capped grid (each workgroup loops over more rows) gives the same bytes.
    Low latency at 700 tokens runs layout + pack (capped); at 128 tokens the
    fused dispatch, which the cap does not apply to."""
    c = small_cfg(name, H=1024)
    d = W.make(name, T=T)
    c["max_tokens"] = T
    run_case(gpu, c, d["x"][:, :c["H"]].copy(), d["topk_idx"], d["topk_weights"], max_tokens=T,
             reuse=(name != "decode"), tag="maxwg-%s-%d" % (name, T), max_workgroups=max_wg)


def test_max_workgroups_full_prefill(gpu):
    d = W.make("prefill")
    run_case(gpu, d["cfg"], d["x"], d["topk_idx"], d["topk_weights"], tag="maxwg-prefill-full",
             max_workgroups=256)


@pytest.mark.parametrize("max_wg", [1, 3, 64])
def test_max_workgroups_with_prefetch(gpu, max_wg):
    """The layout that also reads x under a workgroup cap (its extra
    workgroups limited to the cap, none at a cap of 1): same results."""
    d = W.make("prefill")
    run_case(gpu, d["cfg"], d["x"], d["topk_idx"], d["topk_weights"], tag="maxwg-prefetch-%d" % max_wg,
             max_workgroups=max_wg, prefetch=True)


@pytest.mark.parametrize("name", ["prefill", "decode"])
def test_hook_issue_complete(gpu, name):
    """Dispatch issued on a side stream, completed on the main stream by a hook,
    with unrelated main-stream work in between; combine then runs on the main
    stream."""
    d = W.make(name, T=min(W.WORKLOADS[name]["T"], 1024))
    run_case(gpu, d["cfg"], d["x"], d["topk_idx"], d["topk_weights"], reuse=(name != "decode"),
             tag="hook-%s" % name, side_stream=True)


# ---------------------------------------------------------------- fused low-latency dispatch
# moe_dispatch without a reused layout in the padded low-latency mode runs the
# routing and the copy as one launch when T * k <= 2048 and T <= 512; above
# that it falls back to layout + pack.  Both must give the same results as the oracle.
@pytest.mark.parametrize("quant", [W.QUANT_FP8, W.QUANT_BF16])
@pytest.mark.parametrize("T", [0, 1, 63, 64, 65, 200, 255, 256, 257])
@pytest.mark.parametrize("H", [512, 7168])
def test_ll_fused_ragged(gpu, T, quant, H):
    """512-wide rows run 256-thread blocks, 7168-wide rows 1024-thread blocks
    (one 16-byte chunk per lane)."""
    c = small_cfg("decode", H=H)
    c["quant"] = quant
    d = W.make("decode", T=T)
    M = max(T, 1)
    c["max_tokens"] = M
    run_case(gpu, c, d["x"][:, :c["H"]].copy(), d["topk_idx"], d["topk_weights"], reuse=False,
             max_tokens=M, tag="ll-fused-%d" % quant)


@pytest.mark.parametrize("T,k,H", [(512, 4, 256), (513, 2, 256), (2048, 1, 256), (64, 32, 256), (65, 32, 256),
                                   (1000, 2, 256), (256, 8, 4096), (64, 32, 2176), (100, 3, 32768)])
def test_ll_fused_topk_extremes(gpu, T, k, H):
    c = dict(index=11, T=T, H=H, E=64, R=8, k=k, quant=W.QUANT_FP8,
             layout=W.LAYOUT_PADDED_LL, max_tokens=T)
    rng = np.random.Generator(np.random.PCG64(T + k))
    idx = W.route_uniform(rng, T, c["E"], k)
    x = W.to_bf16_bits(rng.standard_normal((T, c["H"]), dtype=np.float32))
    w = W.softmax_weights(rng, T, k)
    run_case(gpu, c, x, idx, w, reuse=False, max_tokens=T, tag="ll-fused-k%d-H%d" % (k, H))


def test_ll_fused_irregular_routing(gpu):
    """Empty slots, a token with no expert, repeated experts in a row, bad ids,
    a non-zero source rank."""
    c = small_cfg("decode")
    T = 128
    d = W.make("decode", T=T)
    idx = W.with_empty_slots(d["topk_idx"], 0.25)
    idx[7, :] = -1
    idx[9, :] = 17                     # one expert in every slot
    idx[11, 3] = c["E"] + 5            # bad ids: flagged, treated as empty
    idx[12, 0] = -9
    run_case(gpu, c, d["x"][:, :c["H"]].copy(), idx, d["topk_weights"], reuse=False, max_tokens=T,
             src_rank=5, tag="ll-fused-irregular")


# ---------------------------------------------------------------- HIP graph capture
@pytest.mark.parametrize("name,reuse,prefetch", [("decode", False, False), ("prefill", True, False),
                                                  ("prefill", True, True)])
def test_graph_capture_replays_match_eager(gpu, name, reuse, prefetch):
    """The calls only enqueue kernels (no allocation, no memset, no sync), so a
    step captures into a HIP graph.  Replay it several times, with eager work
    and a synchronisation between replays, and check every replay against the
    eager results.  prefetch: the layout call also reads x (2.7 MB of rows, so
    its extra workgroups run)."""
    c = small_cfg(name, H=2048 if prefetch else 512)
    T = 128 if name == "decode" else 700
    d = W.make(name, T=T)
    c["max_tokens"] = T
    ctx = make_ctx(gpu, c, T, max_tokens=T)
    x = to_dev_bf16(d["x"][:, :c["H"]].copy())
    idx = torch.from_numpy(d["topk_idx"]).to(dev())
    w = torch.from_numpy(d["topk_weights"]).to(dev())
    bufs = gpu.DispatchBuffers(ctx)
    h = gpu.Handle(ctx)
    n_cap = ctx.hint(gpu.MOE_BUF_EXPERT_OUT) // (2 * c["H"])
    y = torch.randn((n_cap, c["H"]), device=dev()).to(torch.bfloat16)
    out = torch.empty((T, c["H"]), dtype=torch.bfloat16, device=dev())
    cnt_e = torch.empty(c["E"], dtype=torch.int32, device=dev())
    cnt_r = torch.empty(c["R"], dtype=torch.int32, device=dev())
    in_rank = torch.empty((T, c["R"]), dtype=torch.uint8, device=dev())

    def step():
        if reuse:
            gpu.moe_dispatch_layout(ctx, idx, cnt_e, cnt_r, in_rank, x=x if prefetch else None)
        gpu.moe_dispatch(ctx, x, idx, reuse_layout=reuse, bufs=bufs, handle=h)
        gpu.moe_combine(ctx, y, w, h, out=out)

    watch = [out, h.pos, h.recv_src_idx, h.expert_offsets, h.recv_counts, bufs.recv_rows]
    if bufs.recv_scales is not None:
        watch.append(bufs.recv_scales)
    if reuse:
        watch += [cnt_e, cnt_r, in_rank, bufs.send_rows, h.send_src_idx, h.rank_offsets]
    for t in watch:                           # same fill as between replays (unwritten rows stay equal)
        t.view(torch.uint8).fill_(0x5A)
    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in watch]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in watch:                       # eager work between replays
            t.view(torch.uint8).fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, e) in enumerate(zip(watch, eager)):
            assert torch.equal(t.view(torch.uint8), e.view(torch.uint8)), ("replay", rep, "tensor", i)
    st, _ = gpu.moe_poll_error(ctx)
    assert st == gpu.MOE_OK
    del g
    ctx.close()


def test_launch_log(gpu, capfd, monkeypatch):
    """MOE_EP_LOG=1 at context creation logs each launch on stderr; results unchanged."""
    monkeypatch.setenv("MOE_EP_LOG", "1")
    d = W.make("tiny")
    run_case(gpu, d["cfg"], d["x"], d["topk_idx"], d["topk_weights"], tag="log")
    torch.cuda.synchronize()
    err = capfd.readouterr().err
    for name in ("layout on", "dispatch on", "combine on"):
        assert "[moe_ep]" in err and name in err, err[-2000:]


def test_contexts_on_concurrent_streams(gpu):
    """Three contexts (bf16 send + contiguous, fp8 send + contiguous, fp8 low
    latency) with their layout, dispatch and combine interleaved on three
    streams and no synchronisation in between: the contexts share no state, so
    each matches the oracle as if it had run alone."""
    cases = []
    for name, T in (("prefill", 700), ("grouped", 500), ("decode", 128)):
        d = W.make(name, T=T)
        c = d["cfg"]
        ll = c["layout"] == W.LAYOUT_PADDED_LL
        ctx = make_ctx(gpu, c, T)
        M = ctx.cfg.max_tokens
        ref = oracle.dispatch(d["x"], d["topk_idx"], c["E"], c["R"], quant=c["quant"],
                              max_tokens=M if ll else 0, with_send=not ll)
        pos_ref = ref["pos_ll"] if ll else ref["pos"]
        valid = ref["pos"] >= 0
        yv = W.expert_outputs({"cfg": c}, ref["n_pairs"])
        y = torch.empty((ctx.hint(gpu.MOE_BUF_EXPERT_OUT) // (2 * c["H"]), c["H"]), dtype=torch.bfloat16,
                        device=dev())
        y.view(torch.int16).fill_(0x7FC0)
        y[torch.from_numpy(pos_ref[valid].astype(np.int64)).to(dev())] = to_dev_bf16(yv[ref["pos"][valid]])
        cases.append(dict(name=name, c=c, ll=ll, ctx=ctx, ref=ref, pos_ref=pos_ref, yv=yv, y=y,
                          x=to_dev_bf16(d["x"]), idx=torch.from_numpy(d["topk_idx"]).to(dev()),
                          w=torch.from_numpy(d["topk_weights"]).to(dev()), w_np=d["topk_weights"],
                          bufs=gpu.DispatchBuffers(ctx), h=gpu.Handle(ctx), s=torch.cuda.Stream()))
    for cs in cases:
        cs["s"].wait_stream(torch.cuda.current_stream())   # inputs were copied on the default stream
    log("concurrent contexts: %s" % ", ".join(cs["name"] for cs in cases))
    # interleaved issue: layouts, then dispatches, then combines, each on its own stream
    for cs in cases:
        if not cs["ll"]:
            with torch.cuda.stream(cs["s"]):
                cs["layout"] = gpu.moe_dispatch_layout(cs["ctx"], cs["idx"])
    for cs in reversed(cases):
        with torch.cuda.stream(cs["s"]):
            gpu.moe_dispatch(cs["ctx"], cs["x"], cs["idx"], reuse_layout=not cs["ll"], bufs=cs["bufs"],
                             handle=cs["h"])
    for cs in cases:
        with torch.cuda.stream(cs["s"]):
            cs["out"] = gpu.moe_combine(cs["ctx"], cs["y"], cs["w"], cs["h"])
    torch.cuda.synchronize()
    for cs in cases:
        ref, c = cs["ref"], cs["c"]
        st, flags = gpu.moe_poll_error(cs["ctx"])
        assert st == gpu.MOE_OK, (cs["name"], st, flags)
        if not cs["ll"]:
            cnt_e, cnt_r, in_rank = cs["layout"]
            assert np.array_equal(bits_of(cnt_e), ref["num_tokens_per_expert"]), cs["name"]
            assert np.array_equal(bits_of(in_rank), ref["is_token_in_rank"]), cs["name"]
            assert np.array_equal(bits_of(cs["bufs"].send_rows[:ref["n_send"]]).view(ref["send_rows"].dtype),
                                  ref["send_rows"]), cs["name"]
        T = c["T"]
        assert np.array_equal(bits_of(cs["h"].pos[:T]), cs["pos_ref"]), cs["name"]
        valid = ref["pos"] >= 0
        dst = torch.from_numpy(cs["pos_ref"][valid].astype(np.int64)).to(dev())
        got = bits_of(cs["bufs"].recv_rows[dst]).view(ref["recv_rows"].dtype)
        assert np.array_equal(got, ref["recv_rows"][ref["pos"][valid]]), cs["name"]
        assert np.array_equal(bits_of(cs["out"]), oracle.combine(cs["yv"], cs["w_np"], ref["pos"])), cs["name"]
        cs["ctx"].close()
    del cases
    torch.cuda.empty_cache()


def test_current_stream_handle(gpu):
    """The binding's current-stream handle is torch's, on the default stream
    and inside a side-stream context."""
    from combine_moe_dispatch_layout_amd import _binding as B

    def handle(s):                       # an int; 0 is the null stream
        assert isinstance(s, int)
        return s
    assert handle(B._stream()) == torch.cuda.current_stream().cuda_stream
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        assert handle(B._stream()) == side.cuda_stream == torch.cuda.current_stream().cuda_stream
    assert handle(B._stream(side)) == side.cuda_stream


def test_prepared_calls_match(gpu):
    """prepare_dispatch / prepare_combine give the same bytes as the plain calls."""
    d = W.make("decode")
    c = d["cfg"]
    ctx = make_ctx(gpu, c, c["T"])
    x = to_dev_bf16(d["x"])
    idx = torch.from_numpy(d["topk_idx"]).to(dev())
    w = torch.from_numpy(d["topk_weights"]).to(dev())
    bufs, h = gpu.DispatchBuffers(ctx), gpu.Handle(ctx)
    n_cap = ctx.hint(gpu.MOE_BUF_EXPERT_OUT) // (2 * c["H"])
    y = torch.empty((n_cap, c["H"]), dtype=torch.bfloat16, device=dev())
    y.view(torch.int16).fill_(0x3F80)
    bufs.recv_rows.fill_(0)              # unrouted slots are never written: start both runs equal
    bufs.recv_scales.fill_(0)
    gpu.moe_dispatch(ctx, x, idx, bufs=bufs, handle=h)
    ref_rows = bufs.recv_rows.clone()
    ref_scales = bufs.recv_scales.clone()
    ref_pos = h.pos.clone()
    out_ref = gpu.moe_combine(ctx, y, w, h)
    bufs.recv_rows.fill_(0)
    bufs.recv_scales.fill_(0)
    h.pos.fill_(-5)
    out = torch.empty_like(out_ref)
    pd = gpu.prepare_dispatch(ctx, x, idx, False, bufs, h)
    pc = gpu.prepare_combine(ctx, y, w, h, out, c["T"])
    pd()
    pc()
    torch.cuda.synchronize()
    assert torch.equal(h.pos, ref_pos)
    assert torch.equal(bufs.recv_rows, ref_rows)
    assert torch.equal(bufs.recv_scales.view(torch.int32), ref_scales.view(torch.int32))
    assert torch.equal(out.view(torch.int16), out_ref.view(torch.int16))
    st, _ = gpu.moe_poll_error(ctx)
    assert st == gpu.MOE_OK
    ctx.close()


@pytest.mark.parametrize("quant", [W.QUANT_BF16, W.QUANT_FP8])
def test_many_tiles(gpu, quant):
    """65,536 tokens: 256 layout tiles (per-tile prefixes over many tiles, the
    arrival counter and the last block's scan), narrow rows to keep it quick."""
    T = 65536
    c = dict(index=21, T=T, H=128, E=256, R=32, k=8, quant=quant, layout=W.LAYOUT_CONTIGUOUS, max_tokens=T)
    rng = np.random.Generator(np.random.PCG64(65536 + quant))
    idx = W.with_empty_slots(W.route_uniform(rng, T, c["E"], c["k"]), 0.05, seed=9)
    x = W.to_bf16_bits(rng.standard_normal((T, c["H"]), dtype=np.float32))
    w = W.softmax_weights(rng, T, c["k"])
    run_case(gpu, c, x, idx, w, max_tokens=T, tag="many-tiles-q%d" % quant)


@pytest.mark.parametrize("T,layout,reuse", [(16384, W.LAYOUT_CONTIGUOUS, True), (16385, W.LAYOUT_CONTIGUOUS, True),
                                            (16385, W.LAYOUT_CONTIGUOUS, False), (20000, W.LAYOUT_PADDED_LL, True),
                                            (16384, W.LAYOUT_PADDED_LL, False)])
def test_tile_prefix_boundary(gpu, T, layout, reuse):
    """Both sides of the size where the layout stops leaving per-tile counts
    for the dispatch to sum (64 tiles, 16,384 tokens) and stores prefixes over
    the tiles instead; normal and low-latency layouts, layout reused or not,
    empty slots; then a smaller batch on the same context, which must not see
    the larger one's workspace contents."""
    c = dict(index=22, T=T, H=128, E=64, R=8, k=6, quant=W.QUANT_BF16, layout=layout, max_tokens=T)
    rng = np.random.Generator(np.random.PCG64(T + 7 * layout))
    idx = W.with_empty_slots(W.route_uniform(rng, T, c["E"], c["k"]), 0.05, seed=11)
    x = W.to_bf16_bits(rng.standard_normal((T, c["H"]), dtype=np.float32))
    w = W.softmax_weights(rng, T, c["k"])
    ctx = make_ctx(gpu, c, T, max_tokens=T)
    run_case(gpu, c, x, idx, w, reuse=reuse, max_tokens=T, tag="tile-boundary-%d" % T, ctx=ctx)
    T2 = 5000
    run_case(gpu, c, x[:T2].copy(), idx[:T2].copy(), w[:T2].copy(), reuse=reuse, max_tokens=T,
             tag="tile-boundary-then-%d" % T2, ctx=ctx)
    ctx.close()


@pytest.mark.parametrize("T,reuse,quant", [(128, False, W.QUANT_FP8), (128, True, W.QUANT_BF16),
                                           (600, False, W.QUANT_FP8), (600, True, W.QUANT_BF16)])
def test_ll_window_overflow(gpu, T, reuse, quant):
    """Every token repeats expert 0 in two slots, so expert 0 gets 2T rows from
    this source against a window of M = T slots: the rows past the window are
    not placed (pos -1), MOE_ERR_CAPACITY is reported, everything else matches
    the oracle -- fused path (T = 128) and layout + pack path (T = 600, or a
    reused layout)."""
    c = dict(index=31, T=T, H=512, E=64, R=8, k=8, quant=quant, layout=W.LAYOUT_PADDED_LL, max_tokens=T)
    rng = np.random.Generator(np.random.PCG64(T + quant))
    idx = pins.repeated_expert_routing(T, c["k"], c["E"], rng)
    x = W.to_bf16_bits(rng.standard_normal((T, c["H"]), dtype=np.float32))
    w = W.softmax_weights(rng, T, c["k"])
    ref = run_case(gpu, c, x, idx, w, reuse=reuse, max_tokens=T, src_rank=3, tag="ll-overflow")
    assert ref["ll_overflow"] >= T          # 2T repeated rows, plus any other slot on expert 0
