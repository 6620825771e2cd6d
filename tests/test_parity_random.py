"""GPU parity over seeded random configurations: expert and rank counts,
top-k, hidden size, token count, quantisation, layout, layout reuse, source
rank and workgroup cap drawn together, with empty slots, repeated experts in
a row and bad expert ids, forward (layout, in every other case reading x as
well, dispatch, combine) and backward (dispatch backward, combine backward)
against the oracle.  Same bar as the targeted tests."""
import numpy as np
import pytest

import workloads as W
from test_parity import run_case
from test_parity_backward import run_backward

pytestmark = pytest.mark.gpu

N_CASES = 40
_MAX_EXPERT_OUT_BYTES = 4 << 30      # keeps every case's buffers small on the device


def _cases():
    rng = np.random.Generator(np.random.PCG64(20261202))
    out = []
    while len(out) < N_CASES:
        R = int(rng.choice([1, 2, 3, 4, 8, 16, 32, 64]))
        El = int(rng.choice([1, 2, 3, 4, 8, 16, 32]))
        E = R * El
        if E > 1024:
            continue
        k = int(rng.integers(1, min(32, E) + 1))
        quant = int(rng.integers(0, 2))
        layout = int(rng.integers(0, 2))
        H = int(rng.choice([128, 384, 1024, 2176, 4096] if quant else [8, 64, 200, 520, 2176, 4096]))
        T = int(rng.choice([0, 1, 5, 63, 64, 65, 130, 257, 600]))
        M = max(T, 1) + (0 if layout else int(rng.integers(0, 40)))
        rows = E * M * R if layout else M * k
        if rows * 2 * H > _MAX_EXPERT_OUT_BYTES:
            continue
        out.append(dict(index=100 + len(out), T=T, H=H, E=E, R=R, k=k, quant=quant, layout=layout,
                        max_tokens=M, reuse=bool(rng.integers(0, 2)), s0=int(rng.integers(0, R)),
                        max_wg=int(rng.choice([0, 0, 0, 3, 50])), empty=float(rng.choice([0.0, 0.1, 0.4])),
                        dup=float(rng.choice([0.0, 0.2])), bad=bool(rng.random() < 0.25)))
    return out


CASES = _cases()


def _inputs(c):
    rng = np.random.Generator(np.random.PCG64(c["index"]))
    T, H, E, k = c["T"], c["H"], c["E"], c["k"]
    idx = W.route_uniform(rng, T, E, k)
    if c["empty"]:
        idx = W.with_empty_slots(idx, c["empty"], seed=c["index"])
    if c["dup"] and k > 1 and T:
        rows = rng.random(T) < c["dup"]
        idx[rows, 1] = idx[rows, 0]                     # the same expert in two slots of a row
    if c["bad"] and idx.size:                         # ids outside [-1, E): flagged, treated as empty
        flat = idx.reshape(-1)
        for v in (E + 5, -7, E):
            flat[int(rng.integers(0, flat.size))] = v
    x = W.to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    w = W.softmax_weights(rng, T, k)
    return x, idx, w


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_config(gpu, case):
    c = CASES[case]
    x, idx, w = _inputs(c)
    tag = "random-%d (E=%d R=%d k=%d H=%d T=%d q=%d ll=%d)" % (case, c["E"], c["R"], c["k"], c["H"], c["T"],
                                                               c["quant"], c["layout"])
    # every other case gives the layout call x too (its launch then also reads the rows)
    run_case(gpu, c, x, idx, w, reuse=c["reuse"], max_tokens=c["max_tokens"], src_rank=c["s0"], tag=tag,
             max_workgroups=c["max_wg"], prefetch=case % 2 == 1)
    run_backward(gpu, c, x, idx, w, max_tokens=c["max_tokens"], tag=tag, max_workgroups=c["max_wg"],
                 src_rank=c["s0"])
