"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each check takes the oracle module (or a stand-in built from a planted-mistake
copy of its source, see test_oracle_mutants.py) and raises AssertionError when
the oracle disagrees with

  * a closed form or a specification table (tests/golden/),
  * an independent library routine (torch's float8_e4m3fn / bfloat16 casts,
    numpy's bincount, stable argsort, cumsum, float64 sums),
  * brute force (nearest-value search over every finite E4M3 code; pure-Python
    sorting and counting on tiny inputs),
  * an invariant the method must satisfy (counts sum to T*k, an identity expert
    with weights summing to one returns x, one-hot weights return the routed
    row, each quantised block reaches the E4M3 maximum).

None of them retypes the oracle's own formulas.
"""
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------
# helpers built on library routines (not on the oracle)
def torch_e4m3_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


def torch_e4m3_encode(v):
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return torch.clamp(t, -448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def brute_e4m3_encode(v):
    """Nearest finite E4M3 value by exhaustive search over all 254 finite
    codes; ties go to the even mantissa; zero keeps the input's sign; NaN
    gives 0x7F/0xFF.  Code values come from torch's decoder."""
    v = np.asarray(v, np.float32).astype(np.float64).ravel()
    vals = torch_e4m3_decode_all()
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    cv = vals[codes]
    out = np.empty(v.size, np.uint8)
    # float64 differences |v - c| are exact for |v| <= 2^12 (at most ~45
    # significant bits), so the search below decides ties exactly there.
    # Above that every finite code is smaller than |v|, so the distance
    # |v| - |c| is smallest for the largest magnitude, 448 (code 0x7E).
    big = np.abs(v) > 2.0 ** 12
    for s in range(0, v.size, 4096):
        blk = v[s:s + 4096]
        d = np.abs(blk[:, None] - cv[None, :])
        dmin = d.min(axis=1, keepdims=True)
        cand = d == dmin
        even = (codes & 1) == 0
        neg = np.signbit(blk)[:, None]
        cneg = (codes & 0x80) != 0
        # preference: among nearest, even mantissa first, then matching sign
        score = cand * (4 + 2 * even[None, :] + (neg == cneg[None, :]))
        out[s:s + 4096] = codes[np.argmax(score, axis=1)]
    out[big] = np.where(np.signbit(v[big]), 0xFE, 0x7E)
    nan = np.isnan(v)
    out[nan] = np.where(np.signbit(v[nan]), 0xFF, 0x7F)
    return out


def all_bf16_finite_f32():
    b = np.arange(65536, dtype=np.uint32)
    f = (b << 16).view(np.float32)
    return f[np.isfinite(f)]


def e4m3_midpoint_probes():
    """Every midpoint between adjacent finite E4M3 magnitudes, +-4 float32
    ulps around it, both signs, plus the 448/464 saturation edge."""
    vals = np.unique(np.abs(torch_e4m3_decode_all()[np.isfinite(torch_e4m3_decode_all())]))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    extra = np.array([448.0, 460.0, 463.9999, 464.0, 464.0001, 500.0, 1e6], np.float32)
    base = np.concatenate([mids, vals.astype(np.float32), extra])
    bits = base.view(np.uint32).astype(np.int64)
    probes = []
    for d in range(-4, 5):
        probes.append((bits + d).clip(0, 0x7F7FFFFF).astype(np.uint32).view(np.float32))
    p = np.concatenate(probes)
    return np.concatenate([p, -p])


def bf16_ordered(b):
    """Map bf16 bit patterns to integers whose difference counts ulps."""
    b = np.asarray(b, np.uint16).astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def f32_to_bf16_torch(v):
    t = torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------------------
# codecs
def check_e4m3_decode(orc):
    got = orc.e4m3_to_f32(np.arange(256, dtype=np.uint8)).astype(np.float64)
    ref = torch_e4m3_decode_all()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "NaN codes differ from torch's decoder"
    assert np.array_equal(got[~nan], ref[~nan]), "decoded values differ from torch's decoder"
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan])), "sign of zero"
    # specification table points
    with open(os.path.join(GOLDEN, "e4m3_spec_points.txt")) as f:
        for line in f:
            line = line.split("#")[0].split()
            if not line:
                continue
            code, val = int(line[0], 16), float(line[1])
            g = orc.e4m3_to_f32(np.array([code], np.uint8))[0]
            if math.isnan(val):
                assert math.isnan(g), hex(code)
            else:
                assert g == val and math.copysign(1, g) == math.copysign(1, val), (hex(code), g, val)
    # positive finite codes decode to strictly increasing values
    pos = got[:0x7F]
    assert np.all(np.diff(pos) > 0)


def check_e4m3_encode(orc):
    probes = np.concatenate([all_bf16_finite_f32(), e4m3_midpoint_probes(),
                             np.array([0.0, -0.0, 2.0 ** -10, -(2.0 ** -10), 1e-30, -1e-30,
                                       np.inf, -np.inf], np.float32)])
    got = orc.f32_to_e4m3(probes)
    brute = brute_e4m3_encode(probes)
    bad = np.flatnonzero(got != brute)
    assert bad.size == 0, ("vs brute force", probes[bad[:5]], got[bad[:5]], brute[bad[:5]])
    fin = np.isfinite(probes)
    ref = torch_e4m3_encode(probes[fin])
    bad = np.flatnonzero(got[fin] != ref)
    assert bad.size == 0, ("vs torch", probes[fin][bad[:5]], got[fin][bad[:5]], ref[bad[:5]])
    nan = orc.f32_to_e4m3(np.array([np.nan], np.float32))[0]
    assert nan & 0x7F == 0x7F
    # random float32 in the range the quantiser produces
    rng = np.random.Generator(np.random.PCG64(11))
    r = (rng.standard_normal(200000) * np.exp2(rng.integers(-12, 9, 200000))).astype(np.float32)
    assert np.array_equal(orc.f32_to_e4m3(r), torch_e4m3_encode(r))


def check_bf16_codec(orc):
    rng = np.random.Generator(np.random.PCG64(5))
    bits = rng.integers(0, 2 ** 32, 400000, dtype=np.uint64).astype(np.uint32)
    # exact ties: low half 0x8000, both parities of the kept half
    ties = (rng.integers(0, 2 ** 16, 4000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    near = np.concatenate([ties - 1, ties + 1])
    v = np.concatenate([bits, ties, near,
                        np.array([0x7F7FFFFF, 0xFF7FFFFF, 0x7F800000, 0x00000001,
                                  0x80000000, 0x7F7F8000, 0x3F808000, 0x3F818000], np.uint32)]).view(np.float32)
    got = orc.f32_to_bf16(v)
    ref = f32_to_bf16_torch(v)
    nan = np.isnan(v)
    assert np.array_equal(got[~nan], ref[~nan]), "fp32->bf16 differs from torch's RNE cast"
    gb = got[nan]
    assert np.all(((gb & 0x7F80) == 0x7F80) & ((gb & 0x7F) != 0)), "NaN must stay NaN"
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    dec = orc.bf16_to_f32(allb)
    tdec = torch.from_numpy(allb.view(np.int16)).view(torch.bfloat16).float().numpy()
    n = np.isnan(tdec)
    assert np.array_equal(dec.view(np.uint32)[~n], tdec.view(np.uint32)[~n])
    assert np.all(np.isnan(dec[n]))


# ----------------------------------------------------------------------------
# layout and positions
def np_layout(idx, E, R):
    El = E // R
    valid = (idx >= 0) & (idx < E)
    cnt_e = np.bincount(idx[valid], minlength=E).astype(np.int32)
    rk = np.where(valid, idx // El, -1)
    in_rank = (rk[:, :, None] == np.arange(R)[None, None, :]).any(axis=1).astype(np.uint8)
    return cnt_e, in_rank.sum(0).astype(np.int32), in_rank


def check_layout_and_positions(orc, idx, E, R, M=0, s0=0):
    T, k = idx.shape
    lay = orc.layout(idx, E, R)
    cnt_e, cnt_r, in_rank = np_layout(idx, E, R)
    assert np.array_equal(lay["num_tokens_per_expert"], cnt_e), "counts vs np.bincount"
    assert np.array_equal(lay["is_token_in_rank"], in_rank), "is_token_in_rank"
    assert np.array_equal(lay["num_tokens_per_rank"], cnt_r), "rank counts"
    n_bad = int(((idx < -1) | (idx >= E)).sum())
    assert lay["bad_ids"] == n_bad
    n_empty = int((idx == -1).sum())
    assert int(cnt_e.sum()) == T * k - n_empty - n_bad, "counts must sum to T*k"

    pp = orc.positions(idx, E, R, lay, M, s0)
    assert np.array_equal(pp["expert_offsets"], np.concatenate([[0], np.cumsum(cnt_e)]).astype(np.int32))
    assert np.array_equal(pp["rank_offsets"], np.concatenate([[0], np.cumsum(cnt_r)]).astype(np.int32))
    # expert-major order = stable sort of the flattened valid ids (token, then slot)
    flat = idx.ravel()
    valid = np.flatnonzero((flat >= 0) & (flat < E))
    order = valid[np.argsort(flat[valid], kind="stable")]
    pos_ref = np.full(T * k, -1, np.int64)
    pos_ref[order] = np.arange(order.size)
    assert np.array_equal(pp["pos"].ravel(), pos_ref), "pos vs stable argsort"
    assert np.array_equal(pp["recv_src_idx"], order // k if k else order), "recv_src_idx"
    # rank-major send order: for each rank, the tokens it receives, ascending
    send_ref = np.concatenate([np.flatnonzero(in_rank[:, r]) for r in range(R)] + [np.zeros(0, np.int64)])
    assert np.array_equal(pp["send_src_idx"], send_ref), "send_src_idx"
    spos_ref = np.full((T, R), -1, np.int64)
    for r in range(R):
        tk = np.flatnonzero(in_rank[:, r])
        spos_ref[tk, r] = pp["rank_offsets"][r] + np.arange(tk.size)
    assert np.array_equal(pp["spos"], spos_ref), "spos"
    assert pp["n_send"] == int(cnt_r.sum()) and pp["n_pairs"] == int(cnt_e.sum())
    if M > 0:
        cap = M * R
        pl = pp["pos_ll"].ravel()
        v = pos_ref >= 0
        assert np.all(pl[~v] == -1)
        # slots of one expert: this source's window [s0*M, s0*M + M), dense, in
        # (token, slot) order; rows past the window's M slots are not placed
        vi = np.flatnonzero(v)
        over = 0
        for ex in np.unique(flat[vi]):
            sel = vi[flat[vi] == ex]
            placed = min(sel.size, M)
            assert np.array_equal(pl[sel[:placed]] - ex * cap, s0 * M + np.arange(placed)), "LL slots"
            assert np.all(pl[sel[placed:]] == -1), "rows past the window must not be placed"
            over += sel.size - placed
        assert pp["ll_overflow"] == over, "LL overflow count"
    return lay, pp


def repeated_expert_routing(T, k, E, rng):
    """Every token repeats expert 0 in two of its slots: expert 0 then receives
    2T rows from one source, past a window of M = T slots."""
    idx = route_distinct(rng, T, E, k)
    idx[:, 1] = 0
    idx[:, 0] = 0
    return idx


def route_distinct(rng, T, E, k):
    return np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int64)


def brute_tiny(idx, E, R):
    """Pure-Python (lists, dicts, sorted) layout and positions."""
    El = E // R
    T = len(idx)
    pairs = [(e, t, j) for t in range(T) for j, e in enumerate(idx[t]) if 0 <= e < E]
    cnt_e = [0] * E
    for e, _, _ in pairs:
        cnt_e[e] += 1
    in_rank = [[0] * R for _ in range(T)]
    for e, t, _ in pairs:
        in_rank[t][e // El] = 1
    cnt_r = [sum(in_rank[t][r] for t in range(T)) for r in range(R)]
    recv = sorted(pairs)
    pos = {(t, j): i for i, (_, t, j) in enumerate(recv)}
    send = sorted((r, t) for t in range(T) for r in range(R) if in_rank[t][r])
    return cnt_e, cnt_r, in_rank, [t for _, t, _ in recv], [t for _, t in send], pos


def check_tiny_brute(orc, idx, E, R):
    d = brute_tiny(idx.tolist(), E, R)
    lay = orc.layout(idx, E, R)
    pp = orc.positions(idx, E, R, lay)
    assert lay["num_tokens_per_expert"].tolist() == d[0]
    assert lay["num_tokens_per_rank"].tolist() == d[1]
    assert lay["is_token_in_rank"].tolist() == d[2]
    assert pp["recv_src_idx"].tolist() == d[3]
    assert pp["send_src_idx"].tolist() == d[4]
    T, k = idx.shape
    for t in range(T):
        for j in range(k):
            assert pp["pos"][t, j] == d[5].get((t, j), -1)


# ----------------------------------------------------------------------------
# quantisation
def check_quant_invariants(orc, x_bits):
    q, s = orc.quant_rows(x_bits)
    n, H = x_bits.shape
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    xb = x.reshape(n, H // 128, 128)
    a = np.abs(xb).max(axis=2)
    ap = np.maximum(a, np.float32(1e-4))
    # stored scale is the dequant multiplier a'/448, within one float32 rounding
    rel = np.abs(s.astype(np.float64) * 448.0 - ap.astype(np.float64)) / ap
    assert np.all(rel <= 2.0 ** -24), "scale must be amax/448"
    qb = q.reshape(n, H // 128, 128)
    qmag = qb & 0x7F
    assert not np.any(qmag == 0x7F), "no NaN codes"
    hit = (qmag == 0x7E).any(axis=2)
    assert np.all(hit[a >= 1e-4]), "every non-tiny block must reach +-448"
    # sign agreement and error bound of dequantisation
    dq = torch.from_numpy(q.copy()).view(torch.float8_e4m3fn).float().numpy().reshape(n, H // 128, 128)
    y = dq * s[:, :, None]
    err = np.abs(y.astype(np.float64) - xb)
    xs = np.abs(xb) * (448.0 / ap[:, :, None])
    normal = xs >= 2.0 ** -6
    # E4M3 keeps 3 mantissa bits: half a unit in the last place is 2^-4 of the
    # value in the normal range and 2^-10 (in units of the scaled value) below
    # 2^-6; the float32 scale/product roundings add a few 2^-24 on top.
    bound_n = np.abs(xb) * (2.0 ** -4) * (1 + 2.0 ** -16)
    assert np.all(err[normal] <= bound_n[normal]), "relative error bound in the normal range"
    bound_s = (2.0 ** -10) * s[:, :, None].astype(np.float64) * (1 + 2.0 ** -16) + np.abs(xb) * 2.0 ** -22
    assert np.all(err[~normal] <= bound_s[~normal]), "subnormal bound"
    nz = xb != 0
    assert np.all((np.signbit(dq) == np.signbit(xb))[nz & (dq != 0)]), "sign"


def check_quant_library(orc, x_bits):
    """Same rows through numpy float32 arithmetic and torch's E4M3 cast."""
    q, s = orc.quant_rows(x_bits)
    n, H = x_bits.shape
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    xb = x.reshape(n, H // 128, 128)
    ap = np.maximum(np.abs(xb).max(axis=2), np.float32(1e-4)).astype(np.float32)
    sc = (np.float32(448.0) / ap).astype(np.float32)
    prod = (xb * sc[:, :, None]).astype(np.float32)
    assert np.array_equal(q.reshape(n, H // 128, 128), torch_e4m3_encode(prod))
    assert np.array_equal(s, (ap / np.float32(448.0)).astype(np.float32))


# ----------------------------------------------------------------------------
# combine
def check_combine(orc, y_bits, w, pos, x_bits=None):
    T, k = pos.shape
    H = y_bits.shape[1]
    out = orc.combine(y_bits, w, pos)
    y = torch.from_numpy(y_bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    exact = np.zeros((T, H))
    mag = np.zeros((T, H))
    for j in range(k):
        p = pos[:, j]
        v = p >= 0
        term = w[v, j].astype(np.float64)[:, None] * y[p[v]]
        exact[v] += term
        mag[v] += np.abs(term)
    # float64 products of a float32 and a bf16 are exact and the k-term float64
    # sum is exact to ~2^-50, so `exact` is the true weighted sum.  Summing k
    # binary32-rounded products in binary32 is off by at most
    # gamma * sum|terms|, gamma = (k + 1) 2^-24 (standard recursive-summation
    # bound), and the final bf16 rounding adds half a bf16 ulp (<= 2^-8 |acc|).
    gamma = (k + 1) * 2.0 ** -24 * (1 + 2.0 ** -20)
    o = torch.from_numpy(out.view(np.int16)).view(torch.bfloat16).double().numpy()
    bound = 2.0 ** -8 * (np.abs(exact) + gamma * mag) + gamma * mag + 2.0 ** -133
    assert np.all(np.abs(o - exact) <= bound), "combine outside the binary32 summation bound"
    # where the summation error is far below a bf16 ulp, the result is within
    # one bf16 ulp of the correctly rounded exact sum
    ref = f32_to_bf16_torch(exact.astype(np.float32))
    d = np.abs(bf16_ordered(out) - bf16_ordered(ref))
    clean = gamma * mag <= 2.0 ** -11 * np.abs(exact)
    assert clean.mean() > 0.99
    assert d[clean].max(initial=0) <= 1, "combine further than 1 bf16 ulp from the exact sum"
    # one-hot weights return the routed row bit-exactly
    rng = np.random.Generator(np.random.PCG64(3))
    if T:
        jstar = np.array([rng.choice(np.flatnonzero(pos[t] >= 0)) if (pos[t] >= 0).any() else 0
                          for t in range(T)])
        oh = np.zeros_like(w)
        oh[np.arange(T), jstar] = 1.0
        o1 = orc.combine(y_bits, oh, pos)
        has = (pos >= 0).any(axis=1)
        sel = pos[np.arange(T), jstar]
        assert np.array_equal(o1[has], y_bits[sel[has]]), "one-hot combine"
        assert np.all(o1[~has] == 0), "token without experts -> +0"
    # zero weights -> +0 everywhere
    z = orc.combine(y_bits, np.zeros_like(w), pos)
    assert np.all(z == 0)
    return out


def check_identity_roundtrip(orc, x_bits, idx, w, E, R):
    """Identity expert (y = dispatched row) and weights summing to one: combine
    returns x exactly."""
    d = orc.dispatch(x_bits, idx, E, R, quant=0)
    out = orc.combine(d["recv_rows"], w, d["pos"])
    has = (d["pos"] >= 0).any(axis=1)
    xb = x_bits.copy()
    xb[xb == 0x8000] = 0   # -0 comes back as +0
    assert np.array_equal(out[has], xb[has]), "identity round trip"


def check_dispatch_rows(orc, x_bits, idx, E, R, quant):
    d = orc.dispatch(x_bits, idx, E, R, quant=quant)
    if quant == 0:
        assert np.array_equal(d["send_rows"], x_bits[d["send_src_idx"]])
        assert np.array_equal(d["recv_rows"], x_bits[d["recv_src_idx"]])
    else:
        q, s = orc.quant_rows(x_bits)
        assert np.array_equal(d["send_rows"], q[d["send_src_idx"]])
        assert np.array_equal(d["recv_rows"], q[d["recv_src_idx"]])
        assert np.array_equal(d["send_scales"], s[d["send_src_idx"]])
        assert np.array_equal(d["recv_scales"], s[d["recv_src_idx"]])
    return d


# ----------------------------------------------------------------------------
# backward pass
def _bf16_f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double().numpy()


def small_int_bf16(rng, shape, lo=-4, hi=4):
    """bf16 bit patterns of small integers: every sum and product the backward
    pins form from them is exact in binary32 and binary64."""
    v = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    return f32_to_bf16_torch(v)


def check_dispatch_backward_bound(orc, g_bits, pos):
    """grad_x against the exact binary64 sum of the routed gradient rows: within
    the binary32 recursive-summation bound plus the final bf16 rounding, and
    within one bf16 ulp wherever the summation error is negligible."""
    T, k = pos.shape
    H = g_bits.shape[1]
    out = orc.dispatch_backward(g_bits, pos)
    g = _bf16_f64(g_bits)
    exact = np.zeros((T, H))
    mag = np.zeros((T, H))
    for j in range(k):
        p = pos[:, j]
        v = p >= 0
        exact[v] += g[p[v]]
        mag[v] += np.abs(g[p[v]])
    gamma = (k + 1) * 2.0 ** -24 * (1 + 2.0 ** -20)
    o = _bf16_f64(out)
    bound = 2.0 ** -8 * (np.abs(exact) + gamma * mag) + gamma * mag + 2.0 ** -133
    assert np.all(np.abs(o - exact) <= bound), "dispatch backward outside the summation bound"
    ref = f32_to_bf16_torch(exact.astype(np.float32))
    d = np.abs(bf16_ordered(out) - bf16_ordered(ref))
    clean = gamma * mag <= 2.0 ** -11 * np.abs(exact)
    assert clean.mean() > 0.95
    assert d[clean].max(initial=0) <= 1, "dispatch backward further than 1 bf16 ulp from the exact sum"
    has = (pos >= 0).any(axis=1)
    assert np.all(out[~has] == 0), "token without experts -> +0 gradient"
    return out


def check_dispatch_backward_adjoint(orc, idx, E, R, rng, H=256):
    """<dispatch(x), g> over the receive rows equals <x, dispatch_backward(g)>
    over the tokens (the defining property of an adjoint), on small-integer data
    where both sides are exact; with k = 1 the backward is a plain gather."""
    T, k = idx.shape
    x = small_int_bf16(rng, (T, H))
    d = orc.dispatch(x, idx, E, R, quant=0)
    n = d["n_pairs"]
    g = small_int_bf16(rng, (max(n, 1), H))
    gx = orc.dispatch_backward(g, d["pos"])
    lhs = float((_bf16_f64(d["recv_rows"]) * _bf16_f64(g[:n])).sum()) if n else 0.0
    rhs = float((_bf16_f64(x) * _bf16_f64(gx)).sum())
    assert lhs == rhs, "dispatch backward is not the adjoint of dispatch (%r vs %r)" % (lhs, rhs)
    one = d["pos"][:, :1].copy()
    g1 = orc.dispatch_backward(g, one)
    v = one[:, 0] >= 0
    assert np.array_equal(g1[v], g[one[v, 0]]), "single slot: backward is a gather"


def check_combine_backward_bounds(orc, go_bits, w, y_bits, pos):
    """grad_y: each routed row is w * grad_out rounded to binary32 then bf16
    (within 2^-8 relative plus binary32 rounding); w = 1 and w = -2 are exact
    (bit copy, sign flip and exponent step).  grad_w: within H * 2^-50 of the
    binary64 matrix product of grad_out and the routed rows.  Rows no slot
    points at are left alone; empty slots get grad_w = 0."""
    T, k = pos.shape
    rows, H = y_bits.shape
    sentinel = np.full((rows, H), 0x5A5A, np.uint16)
    gy, gw = orc.combine_backward(go_bits, w, y_bits, pos, grad_y=sentinel.copy())
    go = _bf16_f64(go_bits)
    y = _bf16_f64(y_bits)
    hit = np.zeros(rows, bool)
    for j in range(k):
        p = pos[:, j]
        v = p >= 0
        hit[p[v]] = True
        prod = w[v, j].astype(np.float64)[:, None] * go[v]
        err = np.abs(_bf16_f64(gy[p[v]]) - prod)
        # binary32 rounding (2^-24 relative), then bf16 rounding (unit roundoff 2^-8)
        assert np.all(err <= (2.0 ** -8 + 2.0 ** -23) * np.abs(prod) + 2.0 ** -133), \
            "grad_y is not the rounded weighted gradient"
        # binary64 matrix product (BLAS) of the token's gradient with its routed rows
        ref = np.einsum("th,th->t", go[v], y[p[v]])
        mag = np.einsum("th,th->t", np.abs(go[v]), np.abs(y[p[v]]))
        assert np.all(np.abs(gw[v, j] - ref) <= H * 2.0 ** -50 * mag + 1e-300), "grad_w is not the dot product"
        assert np.all(gw[~v, j] == 0.0), "empty slot -> grad_w = 0"
    assert np.all(gy[~hit] == 0x5A5A), "combine backward wrote a row no slot points at"
    # w = 3/4: the binary32 product is exact, so grad_y is torch's RNE cast of it
    gy34, _ = orc.combine_backward(go_bits, np.full_like(w, 0.75), y_bits, pos)
    for j in range(k):
        p = pos[:, j]
        v = p >= 0
        assert np.array_equal(gy34[p[v]], f32_to_bf16_torch((0.75 * go[v]).astype(np.float32))), \
            "grad_y with w = 3/4 is not the correctly rounded product"
    # exact special weights
    for wv in (1.0, -2.0):
        gy1, _ = orc.combine_backward(go_bits, np.full_like(w, wv), y_bits, pos)
        for j in range(k):
            p = pos[:, j]
            v = p >= 0
            assert np.array_equal(_bf16_f64(gy1[p[v]]), wv * go[v]), "grad_y with w = %g" % wv
    return gy, gw


def check_combine_backward_closed_form(orc, rng):
    """Constant rows: grad_out[t] = c_t, y row = d_r, so grad_w[t, j] = H c_t d_r."""
    T, k, H = 6, 3, 384
    rows = T * k
    pos = np.arange(rows, dtype=np.int32).reshape(T, k)[:, ::-1].copy()
    pos[2, 1] = -1
    c = rng.integers(-3, 4, size=T).astype(np.float32) / 4
    d = rng.integers(-5, 6, size=rows).astype(np.float32) / 8
    go = f32_to_bf16_torch(np.repeat(c[:, None], H, axis=1))
    y = f32_to_bf16_torch(np.repeat(d[:, None], H, axis=1))
    w = rng.standard_normal((T, k)).astype(np.float32)
    _, gw = orc.combine_backward(go, w, y, pos)
    for t in range(T):
        for j in range(k):
            p = pos[t, j]
            want = 0.0 if p < 0 else H * float(c[t]) * float(d[p])
            assert gw[t, j] == want, "grad_w closed form at (%d, %d)" % (t, j)


def check_backward_finite_differences(orc, rng):
    """Brute force on a tiny case: the loss L(w, y) = sum_t <go[t], sum_j
    w[t, j] y[pos[t, j]]> in binary64, differentiated by central differences
    in every weight and every expert-output entry (exact here: L is linear in
    each, the data are small integers), must equal grad_w and, for w = 1,
    grad_y.  Dispatch backward against the differences of <dispatch(x), g> in
    every x entry."""
    T, k, H, rows = 4, 2, 8, 9
    pos = np.array([[3, 0], [5, -1], [8, 1], [2, 7]], np.int32)
    go = small_int_bf16(rng, (T, H))
    y = small_int_bf16(rng, (rows, H))
    w = (rng.integers(-4, 5, size=(T, k)) / 4).astype(np.float32)

    def loss(wv, yv):
        s = 0.0
        for t in range(T):
            for j in range(k):
                if pos[t, j] >= 0:
                    for h in range(H):
                        s += float(go_f[t, h]) * float(wv[t, j]) * float(yv[pos[t, j], h])
        return s

    go_f, y_f = _bf16_f64(go), _bf16_f64(y)
    _, gw = orc.combine_backward(go, w, y, pos)
    w_f = w.astype(np.float64)
    for t in range(T):
        for j in range(k):
            wp, wm = w_f.copy(), w_f.copy()
            wp[t, j] += 1.0
            wm[t, j] -= 1.0
            assert gw[t, j] == (loss(wp, y_f) - loss(wm, y_f)) / 2, "grad_w finite difference (%d, %d)" % (t, j)
    gy, _ = orc.combine_backward(go, np.ones_like(w), y, pos)
    ones = np.ones((T, k))
    for r in set(pos[pos >= 0].tolist()):
        for h in range(H):
            yp, ym = y_f.copy(), y_f.copy()
            yp[r, h] += 1.0
            ym[r, h] -= 1.0
            assert _bf16_f64(gy[r:r + 1, h:h + 1])[0, 0] == (loss(ones, yp) - loss(ones, ym)) / 2, \
                "grad_y finite difference (%d, %d)" % (r, h)
    # dispatch: L(x) = <dispatch(x) receive rows, g>, through the forward oracle
    idx = np.array([[3, 0], [5, -1], [7, 1], [2, 3]], np.int64)
    x = small_int_bf16(rng, (T, H))
    fwd = orc.dispatch(x, idx, 8, 2, quant=0)
    g = small_int_bf16(rng, (fwd["n_pairs"], H))
    g_f = _bf16_f64(g)

    def dloss(xb):
        return float((_bf16_f64(orc.dispatch(xb, idx, 8, 2, quant=0)["recv_rows"]) * g_f).sum())

    gx = _bf16_f64(orc.dispatch_backward(g, fwd["pos"]))
    x_f = _bf16_f64(x)
    for t in range(T):
        for h in range(H):
            xp, xm = x_f.copy(), x_f.copy()
            xp[t, h] += 1.0
            xm[t, h] -= 1.0
            fd = (dloss(f32_to_bf16_torch(xp.astype(np.float32))) -
                  dloss(f32_to_bf16_torch(xm.astype(np.float32)))) / 2
            assert gx[t, h] == fd, "dispatch backward finite difference (%d, %d)" % (t, h)
