"""GPU parity with special bf16 values in the routed rows: +-Inf, quiet,
signalling and negative NaNs, signed zeros, bf16 subnormals, and values near
the bf16 maximum whose weighted sum overflows; zero and NaN routing weights.

The readings these follow: combine accumulates in binary32 from +0 with a
separately rounded multiply and add per slot, and rounds once to bf16 (RNE, a
NaN stays a NaN with its quiet bit set); the backward takes the same binary32
operations.  IEEE 754 leaves the payload of a NaN produced from NaN operands to
the implementation, so NaNs are compared as a class: the NaN positions must be
the same, and every other element bit for bit.  grad_weights (a dot product,
summation order free) must be NaN or an infinity of the same sign where the
oracle's exact value is, and within the rigorous summation bound elsewhere.

The bf16 dispatch copies bits, so the special values must arrive unchanged in
the send and receive rows.  (FP8 of non-finite input is outside the method's
contract: the per-block scale is undefined there.)
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

NAN_CODES = np.array([0x7FC0, 0x7F81, 0xFFC1, 0x7FFF], np.uint16)   # quiet, signalling, negative, max payload
BF16_MAX = 0x7F7F


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


def bf16_isnan(b):
    return ((b & 0x7FFF) > 0x7F80)


def bf16_f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double().numpy()


def plant_specials(rows, rng, frac_rows=0.5, per_row=6, overflow_rows=()):
    """Copy of bf16 rows with special values planted in a fraction of them:
    NaNs of several payloads, +-Inf, +-0, subnormals and +-bf16 max."""
    r = rows.copy()
    n, H = r.shape
    pick = rng.choice(n, size=max(1, int(n * frac_rows)), replace=False)
    menu = np.concatenate([NAN_CODES, np.array([0x7F80, 0xFF80, 0x0000, 0x8000, 0x0001, 0x8001, 0x007F,
                                                0x80FF, BF16_MAX, 0xFF7F], np.uint16)])
    for i in pick:
        cols = rng.choice(H, size=per_row, replace=False)
        r[i, cols] = rng.choice(menu, size=per_row)
    for i in overflow_rows:                     # every element near the maximum: sums overflow
        r[i, :] = BF16_MAX
    return r


def assert_bf16_match(got, want, what):
    nan_g, nan_w = bf16_isnan(got), bf16_isnan(want)
    assert np.array_equal(nan_g, nan_w), "%s: NaN positions differ (%d against %d)" % (
        what, int(nan_g.sum()), int(nan_w.sum()))
    ok = nan_w | (got == want)
    assert ok.all(), "%s: %d non-NaN elements differ" % (what, int((~ok).sum()))
    return int(nan_w.sum())


def setup(gpu, T, H, E, R, k, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    idx = W.route_uniform(rng, T, E, k)
    idx = W.with_empty_slots(idx, 0.1, seed=seed)
    x = W.to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    x = plant_specials(x, rng)
    w = W.softmax_weights(rng, T, k)
    # weights 1 on a few tokens (their sums of near-maximum rows overflow), a
    # zero weight (times an infinity gives NaN), a NaN weight, a negative one
    w[1, :] = 1.0
    w[2, :] = 1.0
    w[3, 0] = 0.0
    w[4, 1] = np.float32(np.nan)
    w[5, 2] = -0.75
    ctx = gpu.Context(gpu.make_config(T, H, E, R, k, 0, W.QUANT_BF16, W.LAYOUT_CONTIGUOUS))
    ref = oracle.dispatch(x, idx, E, R, quant=W.QUANT_BF16, with_send=True)
    x_d = to_dev_bf16(x)
    idx_d = torch.from_numpy(np.ascontiguousarray(idx)).to(dev())
    w_d = torch.from_numpy(np.ascontiguousarray(w)).to(dev())
    bufs = gpu.DispatchBuffers(ctx)
    h = gpu.Handle(ctx)
    gpu.moe_dispatch_layout(ctx, idx_d)
    gpu.moe_dispatch(ctx, x_d, idx_d, reuse_layout=True, bufs=bufs, handle=h)
    st, flags = gpu.moe_poll_error(ctx)
    assert st == gpu.MOE_OK, (st, flags)
    assert np.array_equal(bits_of(h.pos[:T]), ref["pos"]), "handle pos"
    n_pairs, n_send = ref["n_pairs"], ref["n_send"]
    # bit copies: the planted values arrive unchanged
    assert np.array_equal(bits_of(bufs.recv_rows[:n_pairs]), ref["recv_rows"]), "receive rows"
    assert np.array_equal(bits_of(bufs.send_rows[:n_send]), ref["send_rows"]), "send rows"
    assert bf16_isnan(ref["recv_rows"]).any()
    del bufs
    # rows of the tokens with unit weights that every slot of them points at
    pos = ref["pos"]
    over = [int(p) for t in (1, 2) for p in pos[t] if p >= 0]
    return rng, ctx, h, ref, w, w_d, over


@pytest.mark.parametrize("H", [512, 7168])
def test_combine_special_values(gpu, H):
    T, E, R, k = 300, 256, 32, 8
    log("special values: combine and dispatch backward, T=%d H=%d" % (T, H))
    rng, ctx, h, ref, w, w_d, over = setup(gpu, T, H, E, R, k, seed=H)
    n_pairs, pos = ref["n_pairs"], ref["pos"]
    yv = plant_specials(W.to_bf16_bits(rng.standard_normal((n_pairs, H), dtype=np.float32)), rng,
                        overflow_rows=over)
    n_cap = ctx.hint(gpu.MOE_BUF_EXPERT_OUT) // (2 * H)
    y = torch.empty((n_cap, H), dtype=torch.bfloat16, device=dev())
    y.view(torch.int16).fill_(0x7FC0)
    y[:n_pairs] = to_dev_bf16(yv)

    out = gpu.moe_combine(ctx, y, w_d, h)
    st, flags = gpu.moe_poll_error(ctx)
    assert st == gpu.MOE_OK, (st, flags)
    want = oracle.combine(yv, w, pos)
    n_nan = assert_bf16_match(bits_of(out), want, "combine")
    n_inf = int(((want & 0x7FFF) == 0x7F80).sum())
    log("  combine: %d NaN and %d infinite outputs, all other elements bit-exact" % (n_nan, n_inf))
    assert n_inf > 0 and n_nan > 0
    # the tokens whose slots all hold near-maximum rows with weight 1 overflow
    assert np.all((want[1] & 0x7FFF) == 0x7F80) or bf16_isnan(want[1]).any()

    gx = gpu.moe_dispatch_backward(ctx, y, h)
    st, flags = gpu.moe_poll_error(ctx)
    assert st == gpu.MOE_OK, (st, flags)
    want = oracle.dispatch_backward(yv, pos)
    n_nan = assert_bf16_match(bits_of(gx[:T]), want, "dispatch backward")
    log("  dispatch backward: %d NaN outputs, all other elements bit-exact" % n_nan)
    del y
    ctx.close()
    torch.cuda.synchronize()


@pytest.mark.parametrize("H", [512, 7168])
def test_combine_backward_special_values(gpu, H):
    T, E, R, k = 300, 256, 32, 8
    log("special values: combine backward, T=%d H=%d" % (T, H))
    rng, ctx, h, ref, w, w_d, _ = setup(gpu, T, H, E, R, k, seed=H + 1)
    n_pairs, pos = ref["n_pairs"], ref["pos"]
    valid = pos >= 0
    # no near-maximum values here: the exact dot products would be finite where
    # binary32 sums overflow, which is not a difference in the method
    tame = dict(frac_rows=0.3, per_row=4)
    yv = W.to_bf16_bits(rng.standard_normal((n_pairs, H), dtype=np.float32))
    go = W.to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    yv = plant_specials(yv, rng, **tame)
    go = plant_specials(go, rng, **tame)
    yv[(yv & 0x7FFF) == BF16_MAX] = 0x4000
    go[(go & 0x7FFF) == BF16_MAX] = 0x4000

    n_cap = ctx.hint(gpu.MOE_BUF_EXPERT_OUT) // (2 * H)
    y = torch.empty((n_cap, H), dtype=torch.bfloat16, device=dev())
    y.view(torch.int16).fill_(0x7FC0)
    y[:n_pairs] = to_dev_bf16(yv)
    go_d = to_dev_bf16(go)
    gy = torch.empty((n_cap, H), dtype=torch.bfloat16, device=dev())
    gw = torch.full((T, k), 12345.0, dtype=torch.float32, device=dev())
    gpu.moe_combine_backward(ctx, go_d, w_d, y, h, grad_expert_out=gy, grad_weights=gw)
    st, flags = gpu.moe_poll_error(ctx)
    assert st == gpu.MOE_OK, (st, flags)
    gy_ref, gw_ref = oracle.combine_backward(go, w, yv, pos)
    n_nan = assert_bf16_match(bits_of(gy[:n_pairs]), gy_ref, "grad_expert_out")
    log("  grad_expert_out: %d NaN elements, all other elements bit-exact" % n_nan)

    g = bits_of(gw).astype(np.float64)
    assert np.all(g[~valid] == 0.0), "empty slot -> grad_w = 0"
    nan_w = np.isnan(gw_ref) & valid
    inf_w = np.isinf(gw_ref) & valid
    assert np.array_equal(np.isnan(g) & valid, nan_w), "grad_w NaN positions"
    assert np.array_equal(g[inf_w], gw_ref[inf_w]), "grad_w infinities"
    fin = valid & np.isfinite(gw_ref)
    u = 2.0 ** -24
    gamma = H * u / (1 - H * u)
    a_go, a_y = np.abs(bf16_f64(go)), np.abs(bf16_f64(yv))
    for t, j in zip(*np.nonzero(fin)):
        bound = gamma * float(np.dot(a_go[t], a_y[pos[t, j]])) + H * 2.0 ** -126
        assert abs(g[t, j] - gw_ref[t, j]) <= bound, ("grad_w", t, j, g[t, j], gw_ref[t, j], bound)
    log("  grad_w: %d NaN, %d infinite, %d finite within the bound" % (int(nan_w.sum()), int(inf_w.sum()),
                                                                      int(fin.sum())))
    assert nan_w.any() and inf_w.any()
    del y, gy
    ctx.close()
    torch.cuda.synchronize()
