"""CPU: the C-ABI library loads, exports every symbol include/moe_ep.h
declares, and its host-side logic (sizes, configuration checks, status names)
behaves as documented.  No GPU call is made."""
import ctypes
import os
import re
import subprocess

import pytest

import combine_moe_dispatch_layout_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ep.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        from combine_moe_dispatch_layout_amd import _build
        _build.build()
    return moe.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 19
    assert set(names) == set(moe.EXPORTS)
    nm = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)$", nm, flags=re.M))
    for n in names:
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_status_strings(lib):
    for code, name in [(0, "MOE_OK"), (1, "MOE_ERR_INVALID_ARG"), (2, "MOE_ERR_UNSUPPORTED"),
                       (3, "MOE_ERR_CAPACITY"), (4, "MOE_ERR_HANDLE"), (5, "MOE_ERR_HIP"),
                       (6, "MOE_ERR_BAD_TOPK"), (7, "MOE_ERR_DEVICE_BOUNDS"), (8, "MOE_ERR_STALE_LAYOUT"),
                       (9, "MOE_ERR_NONFINITE")]:
        assert moe.status_str(code) == name
    assert moe.status_str(99) == "MOE_ERR_UNKNOWN"


@pytest.mark.parametrize("M,H,E,R,k,q,l", [(16, 256, 8, 2, 2, 0, 0), (128, 7168, 256, 32, 8, 1, 1),
                                           (4096, 7168, 256, 32, 8, 0, 0), (4096, 7168, 256, 8, 8, 1, 0),
                                           (8192, 4096, 64, 8, 6, 0, 0)])
def test_size_hints(lib, M, H, E, R, k, q, l):
    cfg = moe.make_config(M, H, E, R, k, 0, q, l)
    row = H if q else 2 * H
    ks = min(k, R)
    recv_rows = E * M * R if l else M * k
    send_rows = 0 if l else M * ks
    want = {
        moe.MOE_BUF_SEND_ROWS: send_rows * row,
        moe.MOE_BUF_SEND_SCALES: send_rows * (H // 128) * 4 if q else 0,
        moe.MOE_BUF_RECV_ROWS: recv_rows * row,
        moe.MOE_BUF_RECV_SCALES: recv_rows * (H // 128) * 4 if q else 0,
        moe.MOE_BUF_EXPERT_OUT: recv_rows * 2 * H,
        moe.MOE_BUF_COMBINE_OUT: M * 2 * H,
        moe.MOE_BUF_HANDLE_POS: M * k * 4,
        moe.MOE_BUF_HANDLE_EXPERT_OFFSETS: (E + 1) * 4,
        moe.MOE_BUF_HANDLE_RANK_OFFSETS: (R + 1) * 4,
        moe.MOE_BUF_HANDLE_SEND_SRC: M * ks * 4,
        moe.MOE_BUF_HANDLE_RECV_SRC: M * k * 4,
        moe.MOE_BUF_HANDLE_RECV_COUNTS: E * 4,
        moe.MOE_BUF_LAYOUT_EXPERT_COUNTS: E * 4,
        moe.MOE_BUF_LAYOUT_RANK_COUNTS: R * 4,
        moe.MOE_BUF_LAYOUT_TOKEN_IN_RANK: M * R,
    }
    for kind, v in want.items():
        assert moe.moe_size_hint(cfg, kind) == v, kind
    ws = moe.moe_size_hint(cfg, moe.MOE_BUF_WORKSPACE)
    assert 0 < ws < 64 << 20
    with pytest.raises(moe.MoeError):
        moe.moe_size_hint(cfg, 16)


@pytest.mark.parametrize("bad,code", [
    (dict(max_tokens=0), moe.MOE_ERR_INVALID_ARG),
    (dict(hidden=0), moe.MOE_ERR_INVALID_ARG),
    (dict(topk=0), moe.MOE_ERR_INVALID_ARG),
    (dict(src_rank=8), moe.MOE_ERR_INVALID_ARG),
    (dict(src_rank=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(quant=7), moe.MOE_ERR_INVALID_ARG),
    (dict(layout=3), moe.MOE_ERR_INVALID_ARG),
    (dict(num_experts=250), moe.MOE_ERR_UNSUPPORTED),      # not a multiple of R
    (dict(num_experts=2048), moe.MOE_ERR_UNSUPPORTED),
    (dict(num_ranks=128, num_experts=256), moe.MOE_ERR_UNSUPPORTED),
    (dict(topk=33), moe.MOE_ERR_UNSUPPORTED),
    (dict(hidden=7172), moe.MOE_ERR_UNSUPPORTED),           # not a multiple of 8
    (dict(hidden=7168 + 64, quant=1), moe.MOE_ERR_UNSUPPORTED),  # fp8 needs whole 128-blocks
    (dict(max_tokens=1 << 20, layout=1, num_experts=1024, num_ranks=64), moe.MOE_ERR_UNSUPPORTED),
])
def test_config_rejected_without_gpu(lib, bad, code):
    base = dict(max_tokens=4096, hidden=7168, num_experts=256, num_ranks=8, topk=8,
                src_rank=0, quant=0, layout=0)
    base.update(bad)
    cfg = moe.make_config(**base)
    n = ctypes.c_size_t(0)
    assert lib.moe_size_hint(ctypes.byref(cfg), 0, ctypes.byref(n)) == code
    h = ctypes.c_void_p(0)
    # moe_ctx_create validates on the host before touching the device
    assert lib.moe_ctx_create(ctypes.byref(cfg), ctypes.byref(h)) == code
    assert not h.value


def test_null_arguments_rejected(lib):
    assert lib.moe_ctx_create(None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_size_hint(None, 0, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_ctx_destroy(None) == moe.MOE_OK
    assert lib.moe_dispatch_layout(None, None, 0, None, None, None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch_layout_prefetch(None, None, 0, None, None, None, None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch(None, None, None, 0, 0, None, None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(None, None, None, None, None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch_backward(None, None, None, None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_combine_backward(None, None, None, None, None, None, None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_ctx_set_max_workgroups(None, 4) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_hook_create(None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_hook_destroy(None) == moe.MOE_OK
    assert lib.moe_hook_record(None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_hook_wait(None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_poll_error(None, None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_timing_begin(None, 4) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_timing_end(None, None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_timing_launches(None, None, None, 0, None) == moe.MOE_ERR_INVALID_ARG


def test_noalloc_host_checks_without_gpu(lib):
    """moe_dispatch_noalloc checks its configuration, the scratch bound and its
    arguments on the host before any HIP call."""
    null = (None, None, 0, None, None, None, None)
    assert lib.moe_dispatch_noalloc(None, *null) == moe.MOE_ERR_INVALID_ARG
    big = moe.make_config(1 << 17, 256, 256, 64, 16, 0, 0, 0)    # workspace above the static scratch
    assert moe.moe_size_hint(big, moe.MOE_BUF_WORKSPACE) > 8 << 20
    assert lib.moe_dispatch_noalloc(ctypes.byref(big), *null) == moe.MOE_ERR_CAPACITY
    ok = moe.make_config(4096, 7168, 256, 32, 8, 0, 0, 0)
    assert moe.moe_size_hint(ok, moe.MOE_BUF_WORKSPACE) <= 8 << 20
    assert lib.moe_dispatch_noalloc(ctypes.byref(ok), *null) == moe.MOE_ERR_INVALID_ARG
    bad = moe.make_config(4096, 7168, 250, 32, 8, 0, 0, 0)
    assert lib.moe_dispatch_noalloc(ctypes.byref(bad), *null) == moe.MOE_ERR_UNSUPPORTED


def test_product_does_not_reference_oracle():
    """The product package never imports, loads or links the oracle."""
    pkg = os.path.join(ROOT, "combine_moe_dispatch_layout_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f
                assert "orc_" not in text, f
    nm = subprocess.run(["nm", "-D", moe.LIB_PATH], capture_output=True, text=True, check=True).stdout
    assert "orc_" not in nm


@pytest.mark.gpu
def test_c_consumer_runs():
    """tests/c_abi_check (built by __graft_entry__.build()) drives layout,
    dispatch, combine, both backward calls, a hook and the per-launch timing
    through the C ABI with no Python in between and checks closed-form
    properties (counts, receive rows, identity round trip, gradients of
    small-integer inputs)."""
    exe = os.path.join(ROOT, "tests", "c_abi_check")
    if not os.path.exists(exe):
        pytest.fail("tests/c_abi_check is not built (run __graft_entry__.build())")
    print("running", exe, flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "result ok" in r.stdout


def test_missing_library_fails_loudly(tmp_path):
    """No fallback: a missing libmoe_ep.so is an error, never a silent CPU path."""
    from combine_moe_dispatch_layout_amd import _binding as B
    saved = B._lib
    B._lib = None
    try:
        with pytest.raises(RuntimeError, match="not built"):
            B.load_library(str(tmp_path / "libmoe_ep.so"))
    finally:
        B._lib = saved
