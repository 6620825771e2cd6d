"""ctypes binding of libmoe_ep.so (include/moe_ep.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  torch provides device memory (torch.empty on the current device) and
the stream (torch.cuda.current_stream()).  There is no fallback: if the library
is missing or a call fails, an exception is raised.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_ep.so")

# ---------------------------------------------------------------- constants
MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_CAPACITY = 3
MOE_ERR_HANDLE = 4
MOE_ERR_HIP = 5
MOE_ERR_BAD_TOPK = 6
MOE_ERR_DEVICE_BOUNDS = 7
MOE_ERR_STALE_LAYOUT = 8
MOE_ERR_NONFINITE = 9
# moe_poll_error's raw bits
ERR_FLAG_BAD_TOPK, ERR_FLAG_BOUNDS, ERR_FLAG_CAPACITY, ERR_FLAG_STALE, ERR_FLAG_NONFINITE = 1, 2, 4, 8, 16
_POLL_STATUSES = (MOE_OK, MOE_ERR_BAD_TOPK, MOE_ERR_CAPACITY, MOE_ERR_DEVICE_BOUNDS, MOE_ERR_STALE_LAYOUT,
                  MOE_ERR_NONFINITE)

MOE_QUANT_BF16 = 0
MOE_QUANT_FP8_E4M3 = 1
MOE_LAYOUT_CONTIGUOUS = 0
MOE_LAYOUT_PADDED_LL = 1

(MOE_BUF_SEND_ROWS, MOE_BUF_SEND_SCALES, MOE_BUF_RECV_ROWS, MOE_BUF_RECV_SCALES, MOE_BUF_EXPERT_OUT,
 MOE_BUF_COMBINE_OUT, MOE_BUF_HANDLE_POS, MOE_BUF_HANDLE_EXPERT_OFFSETS, MOE_BUF_HANDLE_RANK_OFFSETS,
 MOE_BUF_HANDLE_SEND_SRC, MOE_BUF_HANDLE_RECV_SRC, MOE_BUF_HANDLE_RECV_COUNTS,
 MOE_BUF_LAYOUT_EXPERT_COUNTS, MOE_BUF_LAYOUT_RANK_COUNTS, MOE_BUF_LAYOUT_TOKEN_IN_RANK,
 MOE_BUF_WORKSPACE) = range(16)

(MOE_KERNEL_LAYOUT, MOE_KERNEL_DISPATCH, MOE_KERNEL_COMBINE, MOE_KERNEL_DISPATCH_BWD,
 MOE_KERNEL_COMBINE_BWD) = range(5)
KERNEL_NAMES = ("layout", "dispatch", "combine", "dispatch_bwd", "combine_bwd")


class MoeError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s failed: %s" % (what, status_str(status)))


# ---------------------------------------------------------------- C structs
class moe_config(ctypes.Structure):
    _fields_ = [("max_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("num_ranks", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("src_rank", ctypes.c_int32),
                ("quant", ctypes.c_int32), ("layout", ctypes.c_int32)]


class moe_dispatch_buffers(ctypes.Structure):
    _fields_ = [("send_rows", ctypes.c_void_p), ("send_scales", ctypes.c_void_p),
                ("recv_rows", ctypes.c_void_p), ("recv_scales", ctypes.c_void_p)]


class moe_handle(ctypes.Structure):
    _fields_ = [("pos", ctypes.c_void_p), ("expert_offsets", ctypes.c_void_p),
                ("rank_offsets", ctypes.c_void_p), ("send_src_idx", ctypes.c_void_p),
                ("recv_src_idx", ctypes.c_void_p), ("recv_counts", ctypes.c_void_p),
                ("num_tokens", ctypes.c_int32), ("tag", ctypes.c_uint32)]


# the full list of symbols include/moe_ep.h declares
EXPORTS = ("moe_status_str", "moe_size_hint", "moe_ctx_create", "moe_ctx_destroy", "moe_ctx_config",
           "moe_ctx_tune", "moe_dispatch_layout", "moe_dispatch", "moe_combine", "moe_dispatch_backward",
           "moe_combine_backward", "moe_ctx_set_max_workgroups", "moe_hook_create", "moe_hook_destroy",
           "moe_hook_record", "moe_hook_wait", "moe_poll_error", "moe_timing_begin", "moe_timing_end",
           "moe_timing_launches", "moe_dispatch_noalloc",
           "moe_dispatch_layout_prefetch")

_lib = None


def load_library(path=LIB_PATH):
    """Open libmoe_ep.so (raises if it has not been built) and declare the ABI."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libmoe_ep.so is not built (%s); run `python __graft_entry__.py` "
                           "or combine_moe_dispatch_layout_amd/_build.py" % path)
    lib = ctypes.CDLL(path)
    vp, i32, u32p = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_uint32)
    lib.moe_status_str.restype = ctypes.c_char_p
    lib.moe_status_str.argtypes = [ctypes.c_int]
    sigs = {
        "moe_size_hint": [ctypes.POINTER(moe_config), i32, ctypes.POINTER(ctypes.c_size_t)],
        "moe_ctx_create": [ctypes.POINTER(moe_config), ctypes.POINTER(vp)],
        "moe_ctx_destroy": [vp],
        "moe_ctx_config": [vp, ctypes.POINTER(moe_config)],
        "moe_ctx_tune": [vp, i32, i32],
        "moe_dispatch_layout": [vp, vp, i32, vp, vp, vp, vp],
        "moe_dispatch_layout_prefetch": [vp, vp, i32, vp, vp, vp, vp, vp],
        "moe_dispatch": [vp, vp, vp, i32, i32, ctypes.POINTER(moe_dispatch_buffers),
                         ctypes.POINTER(moe_handle), vp],
        "moe_combine": [vp, vp, vp, ctypes.POINTER(moe_handle), vp, vp],
        "moe_dispatch_backward": [vp, vp, ctypes.POINTER(moe_handle), vp, vp],
        "moe_combine_backward": [vp, vp, vp, vp, ctypes.POINTER(moe_handle), vp, vp, vp],
        "moe_ctx_set_max_workgroups": [vp, i32],
        "moe_hook_create": [ctypes.POINTER(vp)],
        "moe_hook_destroy": [vp],
        "moe_hook_record": [vp, vp],
        "moe_hook_wait": [vp, vp],
        "moe_poll_error": [vp, vp, u32p],
        "moe_timing_begin": [vp, i32],
        "moe_timing_end": [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)],
        "moe_timing_launches": [vp, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_float), i32,
                                ctypes.POINTER(ctypes.c_int32)],
        "moe_dispatch_noalloc": [ctypes.POINTER(moe_config), vp, vp, i32, ctypes.POINTER(moe_dispatch_buffers),
                                 ctypes.POINTER(moe_handle), vp, vp],
    }
    for name, args in sigs.items():
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = args
    _lib = lib
    return lib


def status_str(status):
    return load_library().moe_status_str(status).decode()


def _check(status, what):
    if status != MOE_OK:
        raise MoeError(status, what)


# Pointers and stream handles go to the C calls as plain ints (or None for
# NULL): ctypes converts them for c_void_p parameters, which costs less host
# time per call than building c_void_p objects.
def _ptr(t):
    return t.data_ptr() if t is not None else None


# torch's raw current-stream and device queries: ~0.1 us against ~2.7 us for
# building a torch.cuda.Stream object per call (half of an eager decode step's
# host time otherwise); the public API is the fallback where they are missing
_raw_current_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_raw_device = getattr(torch._C, "_cuda_getDevice", None) or torch.cuda.current_device


def _stream(stream=None):
    """HIP stream handle (an int; 0 = the null stream) of a torch stream
    (default: the current stream)."""
    if stream is None:
        if _raw_current_stream is not None:
            return _raw_current_stream(_raw_device())
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def make_config(max_tokens, hidden, num_experts, num_ranks, topk, src_rank=0,
                quant=MOE_QUANT_BF16, layout=MOE_LAYOUT_CONTIGUOUS):
    return moe_config(max_tokens, hidden, num_experts, num_ranks, topk, src_rank, quant, layout)


def moe_size_hint(cfg, kind):
    n = ctypes.c_size_t(0)
    _check(load_library().moe_size_hint(ctypes.byref(cfg), kind, ctypes.byref(n)), "moe_size_hint")
    return n.value


# ---------------------------------------------------------------- context
class Context:
    """A moe_ctx on the current device, plus the configuration it was made with."""

    def __init__(self, cfg):
        lib = load_library()
        self.cfg = cfg
        h = ctypes.c_void_p(0)
        _check(lib.moe_ctx_create(ctypes.byref(cfg), ctypes.byref(h)), "moe_ctx_create")
        self._h = h
        self.device = torch.cuda.current_device()
        # identifies this context (and so its configuration) to the buffer
        # checks of the calls; a fresh object per context
        self._fit_token = object()

    @property
    def handle(self):
        if self._h is None or not self._h.value:
            raise RuntimeError("context already destroyed")
        return self._h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            _check(load_library().moe_ctx_destroy(self._h), "moe_ctx_destroy")
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def hint(self, kind):
        """moe_size_hint for this context's configuration (fixed, so cached)."""
        cache = self.__dict__.setdefault("_hints", {})
        if kind not in cache:
            cache[kind] = moe_size_hint(self.cfg, kind)
        return cache[kind]

    def tune(self, dispatch_chunks=0, combine_chunks=0):
        _check(load_library().moe_ctx_tune(self.handle, dispatch_chunks, combine_chunks), "moe_ctx_tune")

    def set_max_workgroups(self, n):
        """Cap the workgroups of the dispatch, combine and backward kernels (0 = none)."""
        _check(load_library().moe_ctx_set_max_workgroups(self.handle, int(n)), "moe_ctx_set_max_workgroups")

    def timing_begin(self, max_launches):
        _check(load_library().moe_timing_begin(self.handle, max_launches), "moe_timing_begin")

    def timing_launches(self):
        """[(kernel name, ms)] of every launch timed so far, in launch order
        (before timing_end)."""
        lib = load_library()
        n = ctypes.c_int32(0)
        _check(lib.moe_timing_launches(self.handle, None, None, 0, ctypes.byref(n)), "moe_timing_launches")
        ids = (ctypes.c_int32 * max(n.value, 1))()
        ms = (ctypes.c_float * max(n.value, 1))()
        _check(lib.moe_timing_launches(self.handle, ids, ms, n.value, ctypes.byref(n)), "moe_timing_launches")
        return [(KERNEL_NAMES[ids[i]], ms[i]) for i in range(n.value)]

    def timing_end(self):
        n = len(KERNEL_NAMES)
        tot = (ctypes.c_double * n)()
        cnt = (ctypes.c_int64 * n)()
        _check(load_library().moe_timing_end(self.handle, tot, cnt), "moe_timing_end")
        return {KERNEL_NAMES[i]: {"total_ms": tot[i], "launches": cnt[i]} for i in range(n)}


class Hook:
    """Issue/complete split: record() after enqueuing dispatch or combine on a
    side stream, wait() on the stream that needs the results."""

    def __init__(self):
        self.h = ctypes.c_void_p()
        _check(load_library().moe_hook_create(ctypes.byref(self.h)), "moe_hook_create")

    def record(self, stream=None):
        _check(load_library().moe_hook_record(self.h, _stream(stream)), "moe_hook_record")

    def wait(self, stream=None):
        _check(load_library().moe_hook_wait(self.h, _stream(stream)), "moe_hook_wait")

    def close(self):
        if self.h:
            _check(load_library().moe_hook_destroy(self.h), "moe_hook_destroy")
            self.h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Handle:
    """Caller-owned device arrays of one dispatch (moe_handle), as torch tensors."""

    def __init__(self, ctx):
        c = ctx.cfg
        dev = torch.device("cuda", ctx.device)
        ksend = min(c.topk, c.num_ranks)
        i32 = torch.int32
        self.pos = torch.empty((c.max_tokens, c.topk), dtype=i32, device=dev)
        self.expert_offsets = torch.empty(c.num_experts + 1, dtype=i32, device=dev)
        self.rank_offsets = torch.empty(c.num_ranks + 1, dtype=i32, device=dev)
        self.send_src_idx = torch.empty(c.max_tokens * ksend, dtype=i32, device=dev)
        self.recv_src_idx = torch.empty(c.max_tokens * c.topk, dtype=i32, device=dev)
        self.recv_counts = torch.empty(c.num_experts, dtype=i32, device=dev)
        self.c = moe_handle(self.pos.data_ptr(), self.expert_offsets.data_ptr(),
                            self.rank_offsets.data_ptr(), self.send_src_idx.data_ptr(),
                            self.recv_src_idx.data_ptr(), self.recv_counts.data_ptr(), 0, 0)

    @property
    def num_tokens(self):
        return self.c.num_tokens


class DispatchBuffers:
    """Caller-owned dispatch outputs sized by moe_size_hint (full capacity)."""

    def __init__(self, ctx):
        c = ctx.cfg
        dev = torch.device("cuda", ctx.device)
        fp8 = c.quant == MOE_QUANT_FP8_E4M3
        ll = c.layout == MOE_LAYOUT_PADDED_LL
        H = c.hidden
        row_dt, row_w = (torch.uint8, H) if fp8 else (torch.bfloat16, H)
        row_bytes = H if fp8 else 2 * H
        n_send = ctx.hint(MOE_BUF_SEND_ROWS) // row_bytes
        n_recv = ctx.hint(MOE_BUF_RECV_ROWS) // row_bytes
        self.send_rows = None if ll else torch.empty((n_send, row_w), dtype=row_dt, device=dev)
        self.send_scales = (torch.empty((n_send, H // 128), dtype=torch.float32, device=dev)
                            if fp8 and not ll else None)
        self.recv_rows = torch.empty((n_recv, row_w), dtype=row_dt, device=dev)
        self.recv_scales = torch.empty((n_recv, H // 128), dtype=torch.float32, device=dev) if fp8 else None
        self.c = moe_dispatch_buffers(_ptr(self.send_rows), _ptr(self.send_scales),
                                      _ptr(self.recv_rows), _ptr(self.recv_scales))


# ---------------------------------------------------------------- the calls
def _as_dev(t, dtype, name):
    if not (t.is_cuda and t.dtype is dtype and t.is_contiguous()):
        raise TypeError("%s must be a contiguous %s CUDA tensor" % (name, dtype))
    return t


def _out(t, dtype, numel, name):
    """A caller-supplied output: contiguous, of the right dtype, at least numel elements."""
    _as_dev(t, dtype, name)
    if t.numel() < numel:
        raise ValueError("%s holds %d elements, needs %d" % (name, t.numel(), numel))
    return t


def _fits(ctx, obj, parts, what):
    """The kernels write a handle's arrays and the dispatch buffers through raw
    pointers, up to the sizes moe_size_hint gives for the context's
    configuration: check that every part is at least that large (and that the
    C struct still points at it), once per (object, context)."""
    key = ctx._fit_token
    if getattr(obj, "_fits_key", None) is key:
        return
    for t, kind, ptr in parts:
        need = ctx.hint(kind)
        if t is None:
            if need:
                raise ValueError("%s lacks a buffer this configuration needs (kind %d)" % (what, kind))
            continue
        if not t.is_cuda or not t.is_contiguous() or t.numel() * t.element_size() < need:
            raise ValueError("%s was not made for this context's configuration (kind %d: %d bytes, needs %d)"
                             % (what, kind, t.numel() * t.element_size(), need))
        if ptr != t.data_ptr():
            raise ValueError("%s: the C struct no longer points at its tensors" % what)
    obj._fits_key = key


def _check_handle(ctx, h):
    c = h.c
    _fits(ctx, h, ((h.pos, MOE_BUF_HANDLE_POS, c.pos), (h.expert_offsets, MOE_BUF_HANDLE_EXPERT_OFFSETS,
                                                       c.expert_offsets),
                   (h.rank_offsets, MOE_BUF_HANDLE_RANK_OFFSETS, c.rank_offsets),
                   (h.send_src_idx, MOE_BUF_HANDLE_SEND_SRC, c.send_src_idx),
                   (h.recv_src_idx, MOE_BUF_HANDLE_RECV_SRC, c.recv_src_idx),
                   (h.recv_counts, MOE_BUF_HANDLE_RECV_COUNTS, c.recv_counts)), "handle")


def _check_bufs(ctx, b):
    c = b.c
    _fits(ctx, b, ((b.send_rows, MOE_BUF_SEND_ROWS, c.send_rows or 0),
                   (b.send_scales, MOE_BUF_SEND_SCALES, c.send_scales or 0),
                   (b.recv_rows, MOE_BUF_RECV_ROWS, c.recv_rows or 0),
                   (b.recv_scales, MOE_BUF_RECV_SCALES, c.recv_scales or 0)), "dispatch buffers")


def moe_dispatch_layout(ctx, topk_idx, num_tokens_per_expert=None, num_tokens_per_rank=None,
                        is_token_in_rank=None, x=None):
    """Returns (num_tokens_per_expert int32[E], num_tokens_per_rank int32[R],
    is_token_in_rank uint8[T, R]).  x: the bf16 token rows [T, H] of the
    dispatch that will reuse this layout; given, the same launch reads them
    into the Infinity Cache (moe_dispatch_layout_prefetch)."""
    c = ctx.cfg
    _as_dev(topk_idx, torch.int64, "topk_idx")
    T = topk_idx.shape[0]
    if topk_idx.dim() != 2 or topk_idx.shape[1] != c.topk:
        raise ValueError("topk_idx must be [T, %d]" % c.topk)
    dev = topk_idx.device
    if num_tokens_per_expert is None:
        num_tokens_per_expert = torch.empty(c.num_experts, dtype=torch.int32, device=dev)
    if num_tokens_per_rank is None:
        num_tokens_per_rank = torch.empty(c.num_ranks, dtype=torch.int32, device=dev)
    if is_token_in_rank is None:
        is_token_in_rank = torch.empty((T, c.num_ranks), dtype=torch.uint8, device=dev)
    _out(num_tokens_per_expert, torch.int32, c.num_experts, "num_tokens_per_expert")
    _out(num_tokens_per_rank, torch.int32, c.num_ranks, "num_tokens_per_rank")
    _out(is_token_in_rank, torch.uint8, T * c.num_ranks, "is_token_in_rank")
    if x is None:
        _check(load_library().moe_dispatch_layout(
            ctx.handle, _ptr(topk_idx), T, _ptr(num_tokens_per_expert), _ptr(num_tokens_per_rank),
            _ptr(is_token_in_rank), _stream()), "moe_dispatch_layout")
    else:
        _as_dev(x, torch.bfloat16, "x")
        if x.dim() != 2 or tuple(x.shape) != (T, c.hidden):
            raise ValueError("x must be [T, %d]" % c.hidden)
        _check(load_library().moe_dispatch_layout_prefetch(
            ctx.handle, _ptr(topk_idx), T, _ptr(x), _ptr(num_tokens_per_expert), _ptr(num_tokens_per_rank),
            _ptr(is_token_in_rank), _stream()), "moe_dispatch_layout_prefetch")
    return num_tokens_per_expert, num_tokens_per_rank, is_token_in_rank


def moe_dispatch(ctx, x, topk_idx, reuse_layout=False, bufs=None, handle=None):
    """Returns (DispatchBuffers, Handle).  Pass preallocated bufs/handle to
    avoid any allocation (e.g. inside timed loops)."""
    c = ctx.cfg
    _as_dev(x, torch.bfloat16, "x")
    _as_dev(topk_idx, torch.int64, "topk_idx")
    xs = x.shape
    T = xs[0]
    if len(xs) != 2 or xs[1] != c.hidden or topk_idx.shape != (T, c.topk):
        raise ValueError("x must be [T, %d] and topk_idx [T, %d]" % (c.hidden, c.topk))
    if bufs is None:
        bufs = DispatchBuffers(ctx)
    if handle is None:
        handle = Handle(ctx)
    _check_bufs(ctx, bufs)
    _check_handle(ctx, handle)
    _check(load_library().moe_dispatch(ctx.handle, _ptr(x), _ptr(topk_idx), T, int(bool(reuse_layout)),
                                       ctypes.byref(bufs.c), ctypes.byref(handle.c), _stream()),
           "moe_dispatch")
    return bufs, handle


def moe_combine(ctx, expert_out, topk_weights, handle, out=None):
    """Returns out, bf16 [T, H]."""
    c = ctx.cfg
    _as_dev(expert_out, torch.bfloat16, "expert_out")
    _as_dev(topk_weights, torch.float32, "topk_weights")
    T = handle.num_tokens
    if topk_weights.shape != (T, c.topk):
        raise ValueError("topk_weights must be [T, %d]" % c.topk)
    if expert_out.numel() * 2 < ctx.hint(MOE_BUF_EXPERT_OUT):
        raise ValueError("expert_out smaller than MOE_BUF_EXPERT_OUT")
    if out is None:
        out = torch.empty((T, c.hidden), dtype=torch.bfloat16, device=expert_out.device)
    _out(out, torch.bfloat16, T * c.hidden, "out")
    _check(load_library().moe_combine(ctx.handle, _ptr(expert_out), _ptr(topk_weights),
                                      ctypes.byref(handle.c), _ptr(out), _stream()), "moe_combine")
    return out


def moe_dispatch_backward(ctx, grad_recv, handle, grad_x=None):
    """Gradient of dispatch: grad_x bf16 [T, H] from the receive-layout
    gradient rows (bf16, at least MOE_BUF_EXPERT_OUT bytes)."""
    c = ctx.cfg
    _as_dev(grad_recv, torch.bfloat16, "grad_recv")
    if grad_recv.numel() * 2 < ctx.hint(MOE_BUF_EXPERT_OUT):
        raise ValueError("grad_recv smaller than MOE_BUF_EXPERT_OUT")
    T = handle.num_tokens
    if grad_x is None:
        grad_x = torch.empty((T, c.hidden), dtype=torch.bfloat16, device=grad_recv.device)
    _as_dev(grad_x, torch.bfloat16, "grad_x")
    if grad_x.numel() < T * c.hidden:
        raise ValueError("grad_x must hold [T, %d]" % c.hidden)
    _check(load_library().moe_dispatch_backward(ctx.handle, _ptr(grad_recv), ctypes.byref(handle.c),
                                                _ptr(grad_x), _stream()), "moe_dispatch_backward")
    return grad_x


def moe_combine_backward(ctx, grad_out, topk_weights, expert_out, handle, grad_expert_out=None,
                         grad_weights=None):
    """Gradients of combine: returns (grad_expert_out bf16 in the receive layout,
    grad_weights fp32 [T, k])."""
    c = ctx.cfg
    T = handle.num_tokens
    _as_dev(grad_out, torch.bfloat16, "grad_out")
    _as_dev(topk_weights, torch.float32, "topk_weights")
    _as_dev(expert_out, torch.bfloat16, "expert_out")
    if tuple(topk_weights.shape) != (T, c.topk) or grad_out.numel() < T * c.hidden:
        raise ValueError("topk_weights must be [T, %d] and grad_out [T, %d]" % (c.topk, c.hidden))
    if expert_out.numel() * 2 < ctx.hint(MOE_BUF_EXPERT_OUT):
        raise ValueError("expert_out smaller than MOE_BUF_EXPERT_OUT")
    if grad_expert_out is None:
        grad_expert_out = torch.empty_like(expert_out)
    _as_dev(grad_expert_out, torch.bfloat16, "grad_expert_out")
    if grad_expert_out.numel() * 2 < ctx.hint(MOE_BUF_EXPERT_OUT):
        raise ValueError("grad_expert_out smaller than MOE_BUF_EXPERT_OUT")
    if grad_weights is None:
        grad_weights = torch.empty((T, c.topk), dtype=torch.float32, device=grad_out.device)
    _as_dev(grad_weights, torch.float32, "grad_weights")
    if grad_weights.numel() < T * c.topk:
        raise ValueError("grad_weights must hold [T, %d]" % c.topk)
    _check(load_library().moe_combine_backward(ctx.handle, _ptr(grad_out), _ptr(topk_weights),
                                               _ptr(expert_out), ctypes.byref(handle.c),
                                               _ptr(grad_expert_out), _ptr(grad_weights), _stream()),
           "moe_combine_backward")
    return grad_expert_out, grad_weights


# ---------------------------------------------------------------- prepared calls
# For tight host loops (decode steps): the arguments of a call are checked and
# marshalled once, and the returned callable only makes the C call, on the
# stream that was current when it was prepared.  The tensors must stay alive
# and keep their storage while the callable is used.
def prepare_dispatch(ctx, x, topk_idx, reuse_layout, bufs, handle, stream=None):
    c = ctx.cfg
    _as_dev(x, torch.bfloat16, "x")
    _as_dev(topk_idx, torch.int64, "topk_idx")
    T = x.shape[0]
    if x.dim() != 2 or x.shape[1] != c.hidden or tuple(topk_idx.shape) != (T, c.topk):
        raise ValueError("x must be [T, %d] and topk_idx [T, %d]" % (c.hidden, c.topk))
    _check_bufs(ctx, bufs)
    _check_handle(ctx, handle)
    f = load_library().moe_dispatch
    args = (ctx.handle, _ptr(x), _ptr(topk_idx), ctypes.c_int32(T), ctypes.c_int32(int(bool(reuse_layout))),
            ctypes.byref(bufs.c), ctypes.byref(handle.c), _stream(stream))

    def call():
        st = f(*args)
        if st != MOE_OK:
            raise MoeError(st, "moe_dispatch")
    return call


def prepare_combine(ctx, expert_out, topk_weights, handle, out, num_tokens, stream=None):
    """num_tokens: the token count of the dispatch whose handle is combined
    (checked against the handle at every call)."""
    c = ctx.cfg
    _as_dev(expert_out, torch.bfloat16, "expert_out")
    _as_dev(topk_weights, torch.float32, "topk_weights")
    _as_dev(out, torch.bfloat16, "out")
    if tuple(topk_weights.shape) != (num_tokens, c.topk) or out.numel() < num_tokens * c.hidden:
        raise ValueError("topk_weights must be [%d, %d] and out hold [%d, %d]" % (num_tokens, c.topk, num_tokens,
                                                                                 c.hidden))
    if expert_out.numel() * 2 < ctx.hint(MOE_BUF_EXPERT_OUT):
        raise ValueError("expert_out smaller than MOE_BUF_EXPERT_OUT")
    f = load_library().moe_combine
    hc = handle.c
    args = (ctx.handle, _ptr(expert_out), _ptr(topk_weights), ctypes.byref(hc), _ptr(out), _stream(stream))

    def call():
        if hc.num_tokens != num_tokens:
            raise ValueError("handle holds %d tokens, prepared for %d" % (hc.num_tokens, num_tokens))
        st = f(*args)
        if st != MOE_OK:
            raise MoeError(st, "moe_combine")
    return call


class StaticConfig:
    """A configuration without a context (for moe_dispatch_noalloc): sizes
    for Handle and DispatchBuffers on the current device, nothing allocated by
    the library."""

    def __init__(self, cfg):
        self.cfg = cfg
        self.device = torch.cuda.current_device()
        self._fit_token = object()

    def hint(self, kind):
        cache = self.__dict__.setdefault("_hints", {})
        if kind not in cache:
            cache[kind] = moe_size_hint(self.cfg, kind)
        return cache[kind]


def moe_dispatch_noalloc(scfg, x, topk_idx, bufs, handle, error_word=None):
    """moe_dispatch without a context or any allocation: the library's static
    per-GPU scratch holds the layout.  scfg: a StaticConfig (or a Context, for
    its configuration); bufs and handle sized for it.  error_word: optional
    int32/uint32 device tensor of one element that collects moe_poll_error's
    bits.  Returns (bufs, handle)."""
    c = scfg.cfg
    _as_dev(x, torch.bfloat16, "x")
    _as_dev(topk_idx, torch.int64, "topk_idx")
    T = x.shape[0]
    if x.dim() != 2 or x.shape[1] != c.hidden or tuple(topk_idx.shape) != (T, c.topk):
        raise ValueError("x must be [T, %d] and topk_idx [T, %d]" % (c.hidden, c.topk))
    _check_bufs(scfg, bufs)
    _check_handle(scfg, handle)
    if error_word is not None and not (error_word.is_cuda and error_word.element_size() == 4):
        raise TypeError("error_word must be a 4-byte CUDA tensor")
    _check(load_library().moe_dispatch_noalloc(ctypes.byref(c), _ptr(x), _ptr(topk_idx), T, ctypes.byref(bufs.c),
                                               ctypes.byref(handle.c), _ptr(error_word), _stream()),
           "moe_dispatch_noalloc")
    return bufs, handle


def moe_poll_error(ctx):
    """Synchronizes the current stream; returns (status, raw flags) and clears them."""
    flags = ctypes.c_uint32(0)
    st = load_library().moe_poll_error(ctx.handle, _stream(), ctypes.byref(flags))
    if st not in _POLL_STATUSES:
        raise MoeError(st, "moe_poll_error")
    return st, flags.value
