"""CPU: the oracle against its pins (see pins.py for what each pin is)."""
import numpy as np
import pytest

import pins
import workloads as W


def test_e4m3_decode(orc):
    pins.check_e4m3_decode(orc)


def test_e4m3_encode(orc):
    pins.check_e4m3_encode(orc)


def test_bf16_codec(orc):
    pins.check_bf16_codec(orc)


@pytest.mark.parametrize("T,k,E,R", [(0, 2, 8, 2), (1, 1, 4, 1), (16, 2, 8, 2), (37, 3, 12, 3),
                                     (300, 8, 64, 8), (513, 6, 64, 8)])
def test_layout_positions_random(orc, T, k, E, R):
    rng = np.random.Generator(np.random.PCG64(T * 7 + k))
    idx = W.route_uniform(rng, T, E, k)
    pins.check_layout_and_positions(orc, idx, E, R)
    pins.check_layout_and_positions(orc, W.with_empty_slots(idx, 0.2), E, R)
    pins.check_layout_and_positions(orc, idx, E, R, M=max(T, 1), s0=0)
    pins.check_layout_and_positions(orc, idx, E, R, M=max(T, 1) + 5, s0=R - 1)


def test_ll_window_overflow(orc):
    """A token that repeats an expert can send one expert more rows than the
    window of M slots; the rows past it are not placed and are counted."""
    rng = np.random.Generator(np.random.PCG64(17))
    T, k, E, R = 40, 4, 8, 2
    idx = pins.repeated_expert_routing(T, k, E, rng)
    _, pp = pins.check_layout_and_positions(orc, idx, E, R, M=T, s0=1)
    assert pp["ll_overflow"] > 0
    # distinct experts per token and T <= M: never an overflow
    _, pp = pins.check_layout_and_positions(orc, pins.route_distinct(rng, T, E, k), E, R, M=T, s0=1)
    assert pp["ll_overflow"] == 0


def test_layout_degenerate(orc):
    # every slot to one expert; duplicates inside a row; bad ids; all empty
    T, k, E, R = 50, 4, 16, 4
    pins.check_layout_and_positions(orc, np.full((T, k), 5, np.int64), E, R)
    rng = np.random.Generator(np.random.PCG64(1))
    dup = rng.integers(0, 3, (T, k)).astype(np.int64)
    pins.check_layout_and_positions(orc, dup, E, R)
    bad = rng.integers(-3, E + 3, (T, k)).astype(np.int64)
    pins.check_layout_and_positions(orc, bad, E, R)
    pins.check_layout_and_positions(orc, np.full((T, k), -1, np.int64), E, R)


@pytest.mark.parametrize("seed", range(6))
def test_tiny_brute_force(orc, seed):
    d = W.make("tiny", extra_seed=seed)
    c = d["cfg"]
    idx = d["topk_idx"] if seed % 2 == 0 else W.with_empty_slots(d["topk_idx"], 0.3, seed)
    pins.check_tiny_brute(orc, idx, c["E"], c["R"])


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "grouped", "skewed"])
def test_workload_layout(orc, name):
    d = W.make(name)
    c = d["cfg"]
    M = c["max_tokens"] if c["layout"] == W.LAYOUT_PADDED_LL else 0
    pins.check_layout_and_positions(orc, d["topk_idx"], c["E"], c["R"], M=M)


def test_quant_invariants(orc):
    d = W.make("decode")
    x = d["x"][:64]
    pins.check_quant_invariants(orc, x)
    pins.check_quant_library(orc, x)
    # crafted blocks: all zero, one huge value, tiny values (subnormal codes),
    # a block whose max is exactly 448 (scale 1), negative zeros
    H = 1024
    f = np.zeros((6, H), np.float32)
    f[1, :] = 1e-3
    f[1, 5] = 100.0
    f[2, :] = np.linspace(-1e-6, 1e-6, H)
    f[3, :] = np.linspace(-448, 448, H)
    f[4, :] = -0.0
    f[5, :] = np.exp2(np.arange(H) % 40 - 30.0) * np.where(np.arange(H) % 2, 1, -1)
    xb = W.to_bf16_bits(f)
    pins.check_quant_invariants(orc, xb)
    pins.check_quant_library(orc, xb)
    q, s = orc.quant_rows(xb)
    assert np.all(q[0] == 0) and np.all(s[0] == np.float32(np.float32(1e-4) / np.float32(448)))
    assert np.all(q[4] == 0x80), "negative zero keeps its sign"


def test_quant_exhaustive_bf16(orc):
    """Scale exactly 1 (block max 448): every finite bf16 value of magnitude
    <= 448 is encoded as brute-force nearest-E4M3 says."""
    v = pins.all_bf16_finite_f32()
    v = v[np.abs(v) <= 448]
    n = -(-v.size // 127)
    blocks = np.zeros((n, 128), np.float32)
    flat = np.zeros(n * 127, np.float32)
    flat[:v.size] = v
    blocks[:, :127] = flat.reshape(n, 127)
    blocks[:, 127] = 448.0
    xb = W.to_bf16_bits(blocks)
    q, s = orc.quant_rows(xb)
    assert np.all(s == 1.0)
    assert np.array_equal(q[:, :127].ravel()[:v.size], pins.brute_e4m3_encode(v))


@pytest.mark.parametrize("name", ["tiny", "decode", "grouped", "skewed"])
def test_dispatch_rows(orc, name):
    d = W.make(name, T=min(W.WORKLOADS[name]["T"], 256))
    c = d["cfg"]
    pins.check_dispatch_rows(orc, d["x"], d["topk_idx"], c["E"], c["R"], c["quant"])


@pytest.mark.parametrize("name,T", [("tiny", 16), ("decode", 128), ("skewed", 300)])
def test_combine(orc, name, T):
    d = W.make(name, T=T)
    c = d["cfg"]
    lay = orc.layout(d["topk_idx"], c["E"], c["R"])
    pp = orc.positions(d["topk_idx"], c["E"], c["R"], lay)
    y = W.expert_outputs(d, pp["n_pairs"])
    pins.check_combine(orc, y, d["topk_weights"], pp["pos"])
    # empty slots contribute nothing
    idx2 = W.with_empty_slots(d["topk_idx"], 0.3)
    lay2 = orc.layout(idx2, c["E"], c["R"])
    pp2 = orc.positions(idx2, c["E"], c["R"], lay2)
    pins.check_combine(orc, y[:max(pp2["n_pairs"], 1)], d["topk_weights"], pp2["pos"])


@pytest.mark.parametrize("name", ["tiny", "decode", "skewed"])
def test_identity_roundtrip(orc, name):
    d = W.make(name, T=min(W.WORKLOADS[name]["T"], 512))
    c = d["cfg"]
    pins.check_identity_roundtrip(orc, d["x"], d["topk_idx"], d["topk_weights"], c["E"], c["R"])


def test_fp8_roundtrip_bound(orc):
    """Identity expert on dequantised fp8 rows, weights summing to one:
    |out - x| <= (2^-4 + 2^-8)|x| (E4M3 rounding plus the final bf16 rounding)."""
    d = W.make("grouped", T=256)
    c = d["cfg"]
    dd = orc.dispatch(d["x"], d["topk_idx"], c["E"], c["R"], quant=1)
    q = dd["recv_rows"]
    deq = orc.e4m3_to_f32(q).reshape(q.shape[0], -1, 128) * dd["recv_scales"][:, :, None]
    y = W.to_bf16_bits(deq.reshape(q.shape))
    out = orc.combine(y, d["topk_weights"], dd["pos"])
    xo = W.bf16_bits_to_f32(d["x"]).astype(np.float64)
    o = W.bf16_bits_to_f32(out).astype(np.float64)
    T, H = xo.shape
    amax = np.maximum(np.abs(xo).reshape(T, H // 128, 128).max(axis=2), 1e-4)
    # normal E4M3 range of the scaled value: |x| * 448 / amax >= 2^-6
    normal = (np.abs(xo).reshape(T, H // 128, 128) * 448.0 / amax[:, :, None] >= 2.0 ** -6).reshape(T, H)
    err = np.abs(o - xo)
    assert normal.mean() > 0.99
    assert np.all(err[normal] <= (2.0 ** -4 + 2.0 ** -8) * np.abs(xo[normal]) * (1 + 2.0 ** -10))


def test_pages_settings_fixture():
    """The decode workload carries the production setting the pages state."""
    vals = {}
    with open(pins.os.path.join(pins.GOLDEN, "pages_settings.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, val = line.split()[:2]
            vals[key] = val
    c = W.WORKLOADS["decode"]
    assert c["T"] == int(vals["production.tokens_per_batch"]) == int(vals["ampere.num_tokens"])
    assert c["H"] == int(vals["production.hidden"]) == int(vals["tutorial.hidden_size"])
    assert c["k"] == int(vals["production.topk"]) == int(vals["ampere.num_topk"])
    assert vals["production.dispatch_dtype"] == "fp8" and c["quant"] == W.QUANT_FP8
    assert vals["production.combine_dtype"] == "bf16"


# ---------------------------------------------------------------- backward
@pytest.mark.parametrize("name,T", [("tiny", 16), ("decode", 128), ("skewed", 300)])
def test_dispatch_backward(orc, name, T):
    d = W.make(name, T=T)
    c = d["cfg"]
    for idx in (d["topk_idx"], W.with_empty_slots(d["topk_idx"], 0.3)):
        pp = orc.positions(idx, c["E"], c["R"], orc.layout(idx, c["E"], c["R"]))
        g = W.grad_rows(d, max(pp["n_pairs"], 1))
        pins.check_dispatch_backward_bound(orc, g, pp["pos"])
        # unit weights: the same reduction as the (pinned) combine
        assert np.array_equal(orc.dispatch_backward(g, pp["pos"]),
                              orc.combine(g, np.ones(pp["pos"].shape, np.float32), pp["pos"]))


@pytest.mark.parametrize("T,k,E,R", [(1, 1, 4, 1), (40, 3, 12, 3), (200, 8, 64, 8)])
def test_dispatch_backward_adjoint(orc, T, k, E, R):
    rng = np.random.Generator(np.random.PCG64(100 + T))
    idx = W.route_uniform(rng, T, E, k)
    pins.check_dispatch_backward_adjoint(orc, idx, E, R, rng)
    pins.check_dispatch_backward_adjoint(orc, W.with_empty_slots(idx, 0.25), E, R, rng)


@pytest.mark.parametrize("name,T", [("tiny", 16), ("decode", 64), ("skewed", 200)])
def test_combine_backward(orc, name, T):
    d = W.make(name, T=T)
    c = d["cfg"]
    idx = W.with_empty_slots(d["topk_idx"], 0.2)
    pp = orc.positions(idx, c["E"], c["R"], orc.layout(idx, c["E"], c["R"]))
    y = W.expert_outputs(d, max(pp["n_pairs"], 1) + 3)   # 3 rows no slot points at
    go = W.grad_rows(d, T)
    pins.check_combine_backward_bounds(orc, go, d["topk_weights"], y, pp["pos"])


def test_combine_backward_adjoint(orc):
    """sum_{t,j} w[t,j] grad_w[t,j] = sum_t <go[t], sum_j w[t,j] y[pos]> =
    <grad_y, y> over the routed rows, exact on small-integer data."""
    rng = np.random.Generator(np.random.PCG64(41))
    T, k, E, R, H = 50, 4, 16, 4, 256
    idx = W.with_empty_slots(W.route_uniform(rng, T, E, k), 0.2)
    pp = orc.positions(idx, E, R, orc.layout(idx, E, R))
    n = pp["n_pairs"]
    y = pins.small_int_bf16(rng, (n, H))
    go = pins.small_int_bf16(rng, (T, H))
    w = (rng.integers(-8, 9, size=(T, k)) / 8).astype(np.float32)
    gy, gw = orc.combine_backward(go, w, y, pp["pos"])
    yf, gof = pins._bf16_f64(y), pins._bf16_f64(go)
    fwd = np.zeros((T, H))
    for j in range(k):
        v = pp["pos"][:, j] >= 0
        fwd[v] += w[v, j].astype(np.float64)[:, None] * yf[pp["pos"][v, j]]
    a = float((w.astype(np.float64) * gw).sum())
    b = float((gof * fwd).sum())
    cc = float((pins._bf16_f64(gy) * yf).sum())
    assert a == b == cc


def test_combine_backward_closed_form(orc):
    pins.check_combine_backward_closed_form(orc, np.random.Generator(np.random.PCG64(5)))


def test_backward_finite_differences(orc):
    pins.check_backward_finite_differences(orc, np.random.Generator(np.random.PCG64(6)))
