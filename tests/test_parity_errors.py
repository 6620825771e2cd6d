"""GPU: the data errors the kernels detect and report through moe_poll_error,
with every output they still produce checked against the oracle.

* A layout reused after topk_idx was rewritten in place: each token with a
  changed entry is dropped (pos -1, no rows), the others are placed exactly
  where the layout put them, MOE_ERR_STALE_LAYOUT.
* Inf / NaN in an fp8 dispatch: the blocks holding them are unspecified, every
  other block is exact, MOE_ERR_NONFINITE.
* is_token_in_rank at an address that is not 4-byte aligned: same flags as at
  an aligned one, and nothing written outside it.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

POISON = 0xA5


def log(*a):
    print(*a, flush=True)


def dev():
    return torch.device("cuda", 0)


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def host(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def setup(gpu, name, T, H):
    d = W.make(name, T=T)
    c = dict(d["cfg"])
    c["H"] = H
    x = np.ascontiguousarray(d["x"][:, :H])
    cfg = gpu.make_config(T, H, c["E"], c["R"], c["k"], 0, c["quant"], c["layout"])
    ctx = gpu.Context(cfg)
    bufs = gpu.DispatchBuffers(ctx)
    for t in (bufs.send_rows, bufs.recv_rows, bufs.send_scales, bufs.recv_scales):
        if t is not None:
            t.view(torch.uint8).fill_(POISON)
    h = gpu.Handle(ctx)
    h.pos.fill_(-7)
    return d, c, x, ctx, bufs, h


# ---------------------------------------------------------------- stale layout
@pytest.mark.parametrize("T", [700, 17000])   # per-tile sums; stored per-tile prefixes (> 64 tiles)
def test_reused_layout_after_topk_rewritten(gpu, T):
    d, c, x, ctx, bufs, h = setup(gpu, "prefill", T, 256)
    log("case stale-layout: T=%d E=%d R=%d k=%d" % (T, c["E"], c["R"], c["k"]))
    E, k = c["E"], c["k"]
    idx_old = d["topk_idx"].copy()
    idx_d = torch.from_numpy(idx_old).to(dev())
    gpu.moe_dispatch_layout(ctx, idx_d)
    # rewrite three tokens in place: a slot moved to the neighbouring expert
    # (usually on the same rank, so the token's rank set does not change), and
    # two emptied slots
    idx_new = idx_old.copy()
    changed = [5, T // 2, T - 1]
    idx_new[5, 2] = (idx_old[5, 2] + 1) % E
    idx_new[T // 2, 0] = -1
    idx_new[T - 1, k - 1] = -1
    torch.cuda.synchronize()
    idx_d.copy_(torch.from_numpy(idx_new))
    gpu.moe_dispatch(ctx, bf16_dev(x), idx_d, reuse_layout=True, bufs=bufs, handle=h)
    st, flags = gpu.moe_poll_error(ctx)
    assert st == gpu.MOE_ERR_STALE_LAYOUT and flags & gpu.ERR_FLAG_STALE, (st, flags)

    # the layout's routing is the old one: compare everything but the dropped tokens with it
    ref = oracle.dispatch(x, idx_old, c["E"], c["R"], quant=0)
    keep = np.ones(T, bool)
    keep[changed] = False
    pos = host(h.pos[:T])
    assert (pos[changed] == -1).all(), "dropped tokens keep no receive row"
    assert np.array_equal(pos[keep], ref["pos"][keep]), "untouched tokens' positions"
    assert np.array_equal(host(h.expert_offsets), ref["expert_offsets"])
    assert np.array_equal(host(h.rank_offsets), ref["rank_offsets"])
    n_pairs, n_send = ref["n_pairs"], ref["n_send"]
    recv = host(bufs.recv_rows[:n_pairs])
    send = host(bufs.send_rows[:n_send])
    rs, ss = ref["recv_src_idx"], ref["send_src_idx"]
    kept_r, kept_s = keep[rs], keep[ss]
    assert np.array_equal(recv[kept_r], ref["recv_rows"][kept_r]), "untouched tokens' receive rows"
    assert np.array_equal(send[kept_s], ref["send_rows"][kept_s]), "untouched tokens' send rows"
    assert (recv[~kept_r].view(np.uint8) == POISON).all(), "dropped tokens' receive rows not written"
    assert (send[~kept_s].view(np.uint8) == POISON).all(), "dropped tokens' send rows not written"
    assert np.array_equal(host(h.recv_src_idx[:n_pairs])[kept_r], rs[kept_r])
    assert np.array_equal(host(h.send_src_idx[:n_send])[kept_s], ss[kept_s])

    # a fresh layout of the rewritten routing makes the dispatch whole again
    gpu.moe_dispatch_layout(ctx, idx_d)
    gpu.moe_dispatch(ctx, bf16_dev(x), idx_d, reuse_layout=True, bufs=bufs, handle=h)
    st, flags = gpu.moe_poll_error(ctx)
    assert st == gpu.MOE_OK, (st, flags)
    ref = oracle.dispatch(x, idx_new, c["E"], c["R"], quant=0)
    assert np.array_equal(host(h.pos[:T]), ref["pos"])
    assert np.array_equal(host(bufs.recv_rows[:ref["n_pairs"]]), ref["recv_rows"])
    ctx.close()
    torch.cuda.empty_cache()


def test_reused_layout_unchanged_routing_is_clean(gpu):
    """The check passes silently when nothing changed, at the full prefill size."""
    d, c, x, ctx, bufs, h = setup(gpu, "prefill", 4096, 7168)
    idx_d = torch.from_numpy(d["topk_idx"]).to(dev())
    gpu.moe_dispatch_layout(ctx, idx_d)
    gpu.moe_dispatch(ctx, bf16_dev(x), idx_d, reuse_layout=True, bufs=bufs, handle=h)
    st, flags = gpu.moe_poll_error(ctx)
    assert st == gpu.MOE_OK and flags == 0, (st, flags)
    ctx.close()
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- non-finite fp8 input
@pytest.mark.parametrize("name,T", [("grouped", 300), ("decode", 128)])   # two-launch and fused paths
def test_fp8_nonfinite_blocks_flagged(gpu, name, T):
    H = 512
    d, c, x, ctx, bufs, h = setup(gpu, name, T, H)
    log("case fp8-nonfinite: %s T=%d H=%d" % (name, T, H))
    x = x.copy()
    bad = [(3, 5, 0x7F80), (7, 130, 0x7FC0), (T - 1, H - 1, 0xFF80)]   # +Inf, NaN, -Inf
    for t, ch, bits in bad:
        x[t, ch] = bits
    idx = d["topk_idx"]
    idx_d = torch.from_numpy(idx).to(dev())
    ll = c["layout"] == W.LAYOUT_PADDED_LL
    gpu.moe_dispatch(ctx, bf16_dev(x), idx_d, reuse_layout=False, bufs=bufs, handle=h)
    st, flags = gpu.moe_poll_error(ctx)
    assert st == gpu.MOE_ERR_NONFINITE and flags == gpu.ERR_FLAG_NONFINITE, (st, flags)

    ref = oracle.dispatch(x, idx, c["E"], c["R"], quant=1, max_tokens=T if ll else 0, with_send=not ll)
    pos_ref = ref["pos_ll"] if ll else ref["pos"]
    assert np.array_equal(host(h.pos[:T]), pos_ref)
    # every block except the three that hold a non-finite value is exact
    rs = ref["recv_src_idx"]
    valid = ref["pos"] >= 0
    if ll:
        dst = torch.from_numpy(pos_ref[valid].astype(np.int64)).to(dev())
        order = ref["pos"][valid]
        got_q = np.empty_like(ref["recv_rows"])
        got_s = np.empty_like(ref["recv_scales"])
        got_q[order] = host(bufs.recv_rows[dst])
        got_s[order] = host(bufs.recv_scales[dst])
    else:
        got_q = host(bufs.recv_rows[:ref["n_pairs"]])
        got_s = host(bufs.recv_scales[:ref["n_pairs"]])
    mask = np.ones(got_s.shape, bool)
    for t, ch, _ in bad:
        mask[rs == t, ch // 128] = False
    qmask = np.repeat(mask, 128, axis=1)
    assert (~mask).sum() > 0
    assert np.array_equal(got_q[qmask], ref["recv_rows"][qmask]), "finite blocks' codes"
    assert np.array_equal(got_s[mask], ref["recv_scales"][mask]), "finite blocks' scales"
    ctx.close()
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- unaligned token->rank map
@pytest.mark.parametrize("offset", [1, 2, 3])
def test_is_token_in_rank_unaligned(gpu, offset):
    d, c, x, ctx, bufs, h = setup(gpu, "prefill", 777, 256)    # R = 32: the 32-bit store path when aligned
    T, R = 777, c["R"]
    idx_d = torch.from_numpy(d["topk_idx"]).to(dev())
    raw = torch.full((T * R + 8,), 0x5A, dtype=torch.uint8, device=dev())
    in_rank = raw[offset:offset + T * R].view(T, R)
    assert in_rank.data_ptr() % 4 == offset
    gpu.moe_dispatch_layout(ctx, idx_d, is_token_in_rank=in_rank)
    st, flags = gpu.moe_poll_error(ctx)
    assert st == gpu.MOE_OK, (st, flags)
    ref = oracle.layout(d["topk_idx"], c["E"], R)
    assert np.array_equal(host(in_rank), ref["is_token_in_rank"])
    r = host(raw)
    assert (r[:offset] == 0x5A).all() and (r[offset + T * R:] == 0x5A).all(), "write outside is_token_in_rank"
    ctx.close()
    torch.cuda.empty_cache()
