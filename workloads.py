"""Seeded synthetic inputs for MoE dispatch / combine.

Shared by the oracle tests, the GPU parity tests and the benchmark.  This module
holds none of the method's arithmetic: it only draws random numbers and builds
routing decisions the way an upstream router would.  Floating-point values are
rounded to bf16 with torch's own CPU cast (a library routine, not the codec
under test).

The five workloads stand in for the settings the pages name: the DeepSeek-V3/R1
"production" decode batch (128 tokens, hidden 7168, top-8, FP8 dispatch, BF16
combine -- "DeepEP cross-node optimisation guide", "Core advantages /
low-latency kernels") and the "pretraining" prefill setting of the normal
kernels (DeepTech release article on DeepEP, performance paragraph), plus the
group-limited gating the normal kernels are built around (same article,
paragraph on group-limited gating).  No public dataset is named or needed.

Recipe: numpy PCG64 under SeedSequence(20261202 + c) for workload c (1..5),
spawned into four child streams in the order [x, routing, weights, expert_out].
"""
import numpy as np
import torch

QUANT_BF16 = 0
QUANT_FP8 = 1
LAYOUT_CONTIGUOUS = 0
LAYOUT_PADDED_LL = 1

SEED_BASE = 20261202

WORKLOADS = {
    # c1: tiny, bf16, contiguous
    "tiny": dict(index=1, T=16, H=256, E=8, R=2, k=2, routing="uniform",
                 weights="softmax", quant=QUANT_BF16, layout=LAYOUT_CONTIGUOUS, max_tokens=16),
    # c2: low-latency decode, fp8, padded [8 local experts, 128*32 slots, 7168]
    "decode": dict(index=2, T=128, H=7168, E=256, R=32, k=8, routing="uniform",
                   weights="softmax", quant=QUANT_FP8, layout=LAYOUT_PADDED_LL, max_tokens=128),
    # c3: prefill / training, bf16, send buffers + contiguous expert-major
    "prefill": dict(index=3, T=4096, H=7168, E=256, R=32, k=8, routing="uniform",
                    weights="softmax", quant=QUANT_BF16, layout=LAYOUT_CONTIGUOUS, max_tokens=4096),
    # c4: group-limited gating, fp8, send + contiguous
    "grouped": dict(index=4, T=4096, H=7168, E=256, R=8, k=8, routing="group_limited",
                    groups=8, topk_groups=4, weights="sigmoid", quant=QUANT_FP8,
                    layout=LAYOUT_CONTIGUOUS, max_tokens=4096),
    # c5: skewed (Zipf s = 1.2 popularity, hot experts = low ids), bf16
    "skewed": dict(index=5, T=8192, H=4096, E=64, R=8, k=6, routing="zipf", zipf_s=1.2,
                   weights="softmax", quant=QUANT_BF16, layout=LAYOUT_CONTIGUOUS, max_tokens=8192),
}


def streams(index, extra=0):
    """Five independent generators [x, routing, weights, expert_out, grads].
    (Children of one SeedSequence: the first four do not depend on how many
    are spawned.)"""
    ss = np.random.SeedSequence(SEED_BASE + index + 1000 * extra)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(5)]


def to_bf16_bits(a):
    """float32 numpy array -> bf16 bit patterns (uint16) via torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b):
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).float().numpy()


# ---------------------------------------------------------------- routing
def route_uniform(rng, T, E, k):
    """Each token: k distinct experts, a uniformly random ordered k-subset."""
    if T == 0:
        return np.zeros((0, k), np.int64)
    keys = rng.random((T, E))
    return np.argsort(keys, axis=1, kind="stable")[:, :k].astype(np.int64)


def route_group_limited(rng, T, E, k, groups, topk_groups):
    """Group-limited gating: keep the topk_groups groups with the largest
    per-group max score, then the k best experts inside them.  Ties go to the
    lower index; slots are ordered by score, descending.  Returns (idx, scores)."""
    scores = rng.standard_normal((T, E)).astype(np.float32)
    if T == 0:
        return np.zeros((0, k), np.int64), scores
    gsize = E // groups
    gmax = scores.reshape(T, groups, gsize).max(axis=2)
    keep_g = np.argsort(-gmax, axis=1, kind="stable")[:, :topk_groups]
    mask = np.zeros((T, groups), bool)
    np.put_along_axis(mask, keep_g, True, axis=1)
    masked = np.where(np.repeat(mask, gsize, axis=1), scores, -np.inf)
    idx = np.argsort(-masked, axis=1, kind="stable")[:, :k].astype(np.int64)
    return idx, scores


def route_zipf(rng, T, E, k, s):
    """k distinct experts per token, Plackett-Luce draws with popularity
    p(e) ~ (e+1)^-s (low ids are hot), via Gumbel-top-k; slot order = draw order."""
    if T == 0:
        return np.zeros((0, k), np.int64)
    logp = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    g = -np.log(-np.log(rng.random((T, E))))
    keys = logp[None, :] + g
    return np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int64)


# ---------------------------------------------------------------- weights
def softmax_weights(rng, T, k):
    logits = rng.standard_normal((T, k))
    z = np.exp(logits - logits.max(axis=1, keepdims=True)) if T else logits
    return (z / z.sum(axis=1, keepdims=True)).astype(np.float32) if T else np.zeros((0, k), np.float32)


def sigmoid_weights(scores, idx):
    if idx.shape[0] == 0:
        return np.zeros(idx.shape, np.float32)
    s = np.take_along_axis(scores.astype(np.float64), idx, axis=1)
    sg = 1.0 / (1.0 + np.exp(-s))
    return (sg / sg.sum(axis=1, keepdims=True)).astype(np.float32)


# ---------------------------------------------------------------- workloads
def make(name, T=None, extra_seed=0):
    """Inputs of one workload: bf16 x bits [T,H], topk_idx int64 [T,k], fp32
    topk_weights [T,k], plus the config and the expert-output generator."""
    cfg = dict(WORKLOADS[name])
    if T is not None:
        cfg["T"] = T
        cfg["max_tokens"] = max(cfg["max_tokens"], T)
    T, H, E, k = cfg["T"], cfg["H"], cfg["E"], cfg["k"]
    rx, rr, rw = streams(cfg["index"], extra_seed)[:3]
    x = to_bf16_bits(rx.standard_normal((T, H), dtype=np.float32))
    if cfg["routing"] == "uniform":
        idx = route_uniform(rr, T, E, k)
        w = softmax_weights(rw, T, k)
    elif cfg["routing"] == "group_limited":
        idx, scores = route_group_limited(rr, T, E, k, cfg["groups"], cfg["topk_groups"])
        w = sigmoid_weights(scores, idx)
    elif cfg["routing"] == "zipf":
        idx = route_zipf(rr, T, E, k, cfg["zipf_s"])
        w = softmax_weights(rw, T, k)
    else:
        raise ValueError(cfg["routing"])
    cfg["extra_seed"] = extra_seed
    return {"cfg": cfg, "x": x, "topk_idx": idx, "topk_weights": w}


def expert_outputs(inputs, n_rows):
    """Independent N(0,1) bf16 expert outputs, n_rows x H, from the expert_out
    stream (same values for the same workload and row count)."""
    cfg = inputs["cfg"]
    rng = streams(cfg["index"], cfg.get("extra_seed", 0))[3]
    H = cfg["H"]
    return to_bf16_bits(rng.standard_normal((n_rows, H), dtype=np.float32))


def grad_rows(inputs, n_rows):
    """Independent N(0,1) bf16 gradient rows, n_rows x H (the gradient of the
    combine output, or of the dispatched receive rows), from their own stream."""
    cfg = inputs["cfg"]
    rng = streams(cfg["index"], cfg.get("extra_seed", 0))[4]
    return to_bf16_bits(rng.standard_normal((n_rows, cfg["H"]), dtype=np.float32))


def with_empty_slots(idx, frac, seed=7):
    """Copy of idx with a random fraction of slots set to -1 (empty)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = idx.copy()
    out[rng.random(idx.shape) < frac] = -1
    return out
