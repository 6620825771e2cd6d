"""GPU: moe_dispatch_noalloc (no context, no allocation; the layout lives in
the library's static per-GPU scratch) against moe_dispatch(reuse_layout=0) on
a context of the same configuration, through the C ABI.  Bit-exact on every
output: rows, scales, handle arrays.  Several calls in a row share the
scratch: a large batch, then a smaller one of the same configuration, then
other configurations (the scratch is laid out per configuration)."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

POISON = 0xA5


def log(*a):
    print(*a, flush=True)


def dev():
    return torch.device("cuda", 0)


def to_dev(d):
    x = torch.from_numpy(np.ascontiguousarray(d["x"]).view(np.int16)).view(torch.bfloat16).to(dev())
    idx = torch.from_numpy(np.ascontiguousarray(d["topk_idx"])).to(dev())
    return x, idx


def poisoned(gpu, sizer):
    bufs = gpu.DispatchBuffers(sizer)
    for t in (bufs.send_rows, bufs.recv_rows, bufs.send_scales, bufs.recv_scales):
        if t is not None:
            t.view(torch.uint8).fill_(POISON)
    h = gpu.Handle(sizer)
    for t in (h.pos, h.expert_offsets, h.rank_offsets, h.send_src_idx, h.recv_src_idx, h.recv_counts):
        t.fill_(-7)
    return bufs, h


def same(a, b, what):
    if a is None or b is None:
        assert a is None and b is None, what
        return
    assert torch.equal(a.view(torch.uint8) if a.dtype != torch.int32 else a,
                       b.view(torch.uint8) if b.dtype != torch.int32 else b), what


def compare(gpu, name, T, M):
    """One call of each entry point on the same inputs; every output equal."""
    d = W.make(name, T=T)
    c = d["cfg"]
    log("noalloc case %s: T=%d max_tokens=%d H=%d E=%d R=%d k=%d quant=%d layout=%d" %
        (name, T, M, c["H"], c["E"], c["R"], c["k"], c["quant"], c["layout"]))
    cfg = gpu.make_config(M, c["H"], c["E"], c["R"], c["k"], 0, c["quant"], c["layout"])
    x, idx = to_dev(d)
    ctx = gpu.Context(cfg)
    b_ref, h_ref = poisoned(gpu, ctx)
    gpu.moe_dispatch(ctx, x, idx, reuse_layout=False, bufs=b_ref, handle=h_ref)
    st, flags = gpu.moe_poll_error(ctx)
    assert st == gpu.MOE_OK, (st, flags)

    scfg = gpu.StaticConfig(cfg)
    b, h = poisoned(gpu, scfg)
    err = torch.zeros(1, dtype=torch.int32, device=dev())
    gpu.moe_dispatch_noalloc(scfg, x, idx, b, h, error_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for part in ("send_rows", "send_scales", "recv_rows", "recv_scales"):
        same(getattr(b, part), getattr(b_ref, part), part)
    for part in ("pos", "expert_offsets", "rank_offsets", "send_src_idx", "recv_src_idx", "recv_counts"):
        same(getattr(h, part), getattr(h_ref, part), part)
    assert h.num_tokens == h_ref.num_tokens == T
    assert h.c.tag == h_ref.c.tag
    # the handle is accepted by combine on the context
    n_rows = ctx.hint(gpu.MOE_BUF_EXPERT_OUT) // (2 * c["H"])
    y = torch.zeros((n_rows, c["H"]), dtype=torch.bfloat16, device=dev())
    w = torch.from_numpy(d["topk_weights"]).to(dev())
    out = gpu.moe_combine(ctx, y, w, h)
    out_ref = gpu.moe_combine(ctx, y, w, h_ref)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_ref.view(torch.int16))
    ctx.close()
    del b, h, b_ref, h_ref, y
    torch.cuda.empty_cache()


def test_noalloc_matches_dispatch_then_smaller(gpu):
    # prefill shape (many tiles, stored tile sums), then a smaller batch of the same configuration
    compare(gpu, "prefill", 4096, 4096)
    compare(gpu, "prefill", 300, 4096)


def test_noalloc_other_configurations(gpu):
    compare(gpu, "grouped", 1024, 1024)   # fp8, R = 8
    compare(gpu, "skewed", 8192, 8192)    # k = 6, E = 64: another workspace layout
    compare(gpu, "decode", 128, 128)      # padded low-latency: the fused launch
    compare(gpu, "tiny", 16, 16)          # one tile
    compare(gpu, "tiny", 0, 16)           # no tokens: offsets and counts only


def test_noalloc_beyond_scratch_rejected(gpu):
    # a workspace larger than the static scratch: refused on the host, nothing launched
    cfg = gpu.make_config(1 << 17, 256, 256, 64, 16, 0, 0, 0)
    assert gpu.moe_size_hint(cfg, gpu.MOE_BUF_WORKSPACE) > (8 << 20)
    import ctypes
    from combine_moe_dispatch_layout_amd import _binding as B
    lib = gpu.load_library()
    bufs = B.moe_dispatch_buffers(0, 0, 16, 0)
    h = B.moe_handle(16, 16, 16, 16, 16, 16, 0, 0)
    st = lib.moe_dispatch_noalloc(ctypes.byref(cfg), None, None, 0, ctypes.byref(bufs), ctypes.byref(h), None, None)
    assert st == gpu.MOE_ERR_CAPACITY
