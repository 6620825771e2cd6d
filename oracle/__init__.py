"""CPU oracle for MoE dispatch-layout / dispatch / combine.

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by
the cpu_baseline leg of bench.py, never by the product package.  The arithmetic
lives in moe_oracle.c (plain scalar C); this module only marshals numpy arrays
through ctypes.  bf16 tensors travel as uint16 bit patterns, fp8 as uint8 codes.

Pages followed (cited per function in moe_oracle.c): "DeepEP cross-node
optimisation guide" (cyqw.cn) -- opening paragraph, "Core API example",
"Core advantages / low-latency kernels", "Performance tuning" -- and the
DeepTech release article on DeepEP (010bt.com), feature list and EP paragraph.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None

_i64 = ctypes.c_int64
_i32 = ctypes.c_int
_vp = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    _lib = _bind(_LIB_PATH)
    return _lib


def _bind(path):
    """Open a build of moe_oracle.c and declare its C signatures."""
    lib = ctypes.CDLL(path)
    lib.orc_layout.restype = _i64
    lib.orc_layout.argtypes = [_vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp]
    lib.orc_positions.restype = _i64
    lib.orc_positions.argtypes = [_vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp,
                                  _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _vp, _vp, _vp]
    lib.orc_quant_rows.restype = None
    lib.orc_quant_rows.argtypes = [_vp, _i64, _i32, _vp, _vp]
    lib.orc_dispatch_rows.restype = None
    lib.orc_dispatch_rows.argtypes = [_vp, _i32, _i32, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp]
    lib.orc_combine.restype = None
    lib.orc_combine.argtypes = [_vp, _i32, _vp, _vp, _i64, _i32, _vp]
    lib.orc_dispatch_backward.restype = None
    lib.orc_dispatch_backward.argtypes = [_vp, _i32, _vp, _i64, _i32, _vp]
    lib.orc_combine_backward.restype = None
    lib.orc_combine_backward.argtypes = [_vp, _vp, _vp, _vp, _i64, _i32, _i32, _vp, _vp]
    for name in ("orc_f32_to_e4m3_n", "orc_e4m3_to_f32_n", "orc_f32_to_bf16_n", "orc_bf16_to_f32_n"):
        f = getattr(lib, name)
        f.restype = None
        f.argtypes = [_vp, _i64, _vp]
    return lib


def _p(a):
    return a.ctypes.data if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- codecs
def f32_to_e4m3(v):
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    _load().orc_f32_to_e4m3_n(_p(v), v.size, _p(out))
    return out


def e4m3_to_f32(q):
    q = _c(q, np.uint8)
    out = np.empty(q.shape, np.float32)
    _load().orc_e4m3_to_f32_n(_p(q), q.size, _p(out))
    return out


def f32_to_bf16(v):
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint16)
    _load().orc_f32_to_bf16_n(_p(v), v.size, _p(out))
    return out


def bf16_to_f32(b):
    b = _c(b, np.uint16)
    out = np.empty(b.shape, np.float32)
    _load().orc_bf16_to_f32_n(_p(b), b.size, _p(out))
    return out


# ---------------------------------------------------------------- the method
def layout(topk_idx, num_experts, num_ranks):
    """Step 1: counts per expert and per virtual rank, token->rank map."""
    idx = _c(topk_idx, np.int64)
    T, k = idx.shape
    cnt_e = np.empty(num_experts, np.int32)
    cnt_r = np.empty(num_ranks, np.int32)
    in_rank = np.empty((T, num_ranks), np.uint8)
    bad = _load().orc_layout(_p(idx), T, k, num_experts, num_ranks,
                             _p(cnt_e), _p(cnt_r), _p(in_rank))
    return {"num_tokens_per_expert": cnt_e, "num_tokens_per_rank": cnt_r,
            "is_token_in_rank": in_rank, "bad_ids": int(bad)}


def positions(topk_idx, num_experts, num_ranks, lay, max_tokens=0, src_rank=0):
    """Step 2: offsets, stable positions, inverse (source index) maps."""
    idx = _c(topk_idx, np.int64)
    T, k = idx.shape
    E, R = num_experts, num_ranks
    eoff = np.empty(E + 1, np.int32)
    roff = np.empty(R + 1, np.int32)
    pos = np.empty((T, k), np.int32)
    spos = np.empty((T, R), np.int32)
    send_src = np.empty(max(T * min(k, R), 1), np.int32)
    recv_src = np.empty(max(T * k, 1), np.int32)
    pos_ll = np.empty((T, k), np.int32) if max_tokens > 0 else None
    n_pairs = ctypes.c_int64(0)
    overflow = ctypes.c_int64(0)
    n_send = _load().orc_positions(
        _p(idx), T, k, E, R, _p(lay["num_tokens_per_expert"]), _p(lay["num_tokens_per_rank"]),
        _p(lay["is_token_in_rank"]), _p(eoff), _p(roff), _p(pos), _p(spos),
        _p(send_src), _p(recv_src), max_tokens, src_rank, _p(pos_ll), ctypes.byref(n_pairs),
        ctypes.byref(overflow))
    if n_send < 0:
        raise MemoryError("oracle positions: out of host memory")
    n_pairs = n_pairs.value
    return {"expert_offsets": eoff, "rank_offsets": roff, "pos": pos, "spos": spos,
            "send_src_idx": send_src[:n_send].copy(), "recv_src_idx": recv_src[:n_pairs].copy(),
            "pos_ll": pos_ll, "n_send": int(n_send), "n_pairs": int(n_pairs),
            "ll_overflow": int(overflow.value)}


def quant_rows(x_bf16):
    """FP8 E4M3 codes and per-128-channel fp32 dequant scales of bf16 rows."""
    x = _c(x_bf16, np.uint16)
    n, H = x.shape
    assert H % 128 == 0
    q = np.empty((n, H), np.uint8)
    s = np.empty((n, H // 128), np.float32)
    _load().orc_quant_rows(_p(x), n, H, _p(q), _p(s))
    return q, s


def rows(x_bf16, pp, quant=0, with_send=True):
    """Step 3 (payload): the packed send rows and the expert-major receive rows
    of `pp` (the result of positions()), bf16 copies or E4M3 codes + scales."""
    x = _c(x_bf16, np.uint16)
    T, H = x.shape
    n_send, n_pairs = pp["n_send"], pp["n_pairs"]
    if quant == 0:
        send = np.empty((n_send, H), np.uint16) if with_send else None
        recv = np.empty((n_pairs, H), np.uint16)
        send_s = recv_s = None
    else:
        send = np.empty((n_send, H), np.uint8) if with_send else None
        recv = np.empty((n_pairs, H), np.uint8)
        send_s = np.empty((n_send, H // 128), np.float32) if with_send else None
        recv_s = np.empty((n_pairs, H // 128), np.float32)
    _load().orc_dispatch_rows(_p(x), H, quant, _p(pp["send_src_idx"]), n_send,
                              _p(pp["recv_src_idx"]), n_pairs, _p(send), _p(send_s),
                              _p(recv), _p(recv_s))
    return {"send_rows": send, "send_scales": send_s, "recv_rows": recv, "recv_scales": recv_s}


def dispatch(x_bf16, topk_idx, num_experts, num_ranks, quant=0, max_tokens=0,
             src_rank=0, with_send=True):
    """Layout + positions + payload rows.

    Returns a dict with every layout/handle array, the packed send rows
    (rank-major, N_send rows) and the expert-major receive rows (N_pairs rows,
    row i = token recv_src_idx[i]).  For the low-latency padded layout the
    receive rows are the same; their padded addresses are pos_ll.
    """
    lay = layout(topk_idx, num_experts, num_ranks)
    pp = positions(topk_idx, num_experts, num_ranks, lay, max_tokens, src_rank)
    out = dict(lay)
    out.update(pp)
    out.update(rows(x_bf16, pp, quant, with_send))
    return out


def combine(y_bf16, topk_weights, pos):
    """Step 4: out[t] = bf16(sum_j w[t,j] * y[pos[t,j]]), fp32, j ascending."""
    y = _c(y_bf16, np.uint16)
    w = _c(topk_weights, np.float32)
    pos = _c(pos, np.int32)
    T, k = pos.shape
    H = y.shape[1]
    if T:
        valid = pos[pos >= 0]
        if valid.size and valid.max() >= y.shape[0]:
            raise IndexError("oracle combine: pos beyond expert-output rows")
    out = np.empty((T, H), np.uint16)
    _load().orc_combine(_p(y), H, _p(w), _p(pos), T, k, _p(out))
    return out


# ---------------------------------------------------------------- backward
def _check_pos(pos, rows):
    if pos.size:
        valid = pos[pos >= 0]
        if valid.size and valid.max() >= rows:
            raise IndexError("oracle: pos beyond the receive rows")


def dispatch_backward(grad_recv_bf16, pos):
    """grad_x[t] = bf16(sum over valid j, ascending, of grad_recv[pos[t, j]]),
    binary32 from +0 (the adjoint of dispatch's copy into the receive rows)."""
    g = _c(grad_recv_bf16, np.uint16)
    pos = _c(pos, np.int32)
    T, k = pos.shape
    H = g.shape[1]
    _check_pos(pos, g.shape[0])
    out = np.empty((T, H), np.uint16)
    _load().orc_dispatch_backward(_p(g), H, _p(pos), T, k, _p(out))
    return out


def combine_backward(grad_out_bf16, topk_weights, y_bf16, pos, grad_y=None):
    """Gradients of combine: grad_y rows at pos = bf16(w * grad_out) (binary32
    product), grad_w[t, j] = <grad_out[t], y[pos[t, j]]> (binary64, float64
    result).  grad_y: optional uint16 [rows, H] array updated in place (rows no
    slot points at keep their contents); by default a zero array the size of y."""
    go = _c(grad_out_bf16, np.uint16)
    w = _c(topk_weights, np.float32)
    y = _c(y_bf16, np.uint16)
    pos = _c(pos, np.int32)
    T, k = pos.shape
    H = go.shape[1]
    assert y.shape[1] == H and go.shape[0] == T
    _check_pos(pos, y.shape[0])
    if grad_y is None:
        grad_y = np.zeros(y.shape, np.uint16)
    assert grad_y.dtype == np.uint16 and grad_y.flags.c_contiguous and grad_y.shape == y.shape
    grad_w = np.empty((T, k), np.float64)
    _load().orc_combine_backward(_p(go), _p(w), _p(y), _p(pos), T, k, H, _p(grad_y), _p(grad_w))
    return grad_y, grad_w
