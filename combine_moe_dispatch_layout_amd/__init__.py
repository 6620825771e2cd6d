"""MI355X-native MoE token dispatch-layout / dispatch / combine.

The work happens in libmoe_ep.so (hand-written HIP for gfx950, C ABI in
include/moe_ep.h); this package is its thin Python binding.  PyTorch is used
only for device memory and streams.
"""
from ._binding import (  # noqa: F401
    EXPORTS, KERNEL_NAMES, LIB_PATH, Context, DispatchBuffers, Handle, Hook, MoeError,
    MOE_BUF_COMBINE_OUT, MOE_BUF_EXPERT_OUT, MOE_BUF_HANDLE_EXPERT_OFFSETS, MOE_BUF_HANDLE_POS,
    MOE_BUF_HANDLE_RANK_OFFSETS, MOE_BUF_HANDLE_RECV_COUNTS, MOE_BUF_HANDLE_RECV_SRC,
    MOE_BUF_HANDLE_SEND_SRC, MOE_BUF_LAYOUT_EXPERT_COUNTS, MOE_BUF_LAYOUT_RANK_COUNTS,
    MOE_BUF_LAYOUT_TOKEN_IN_RANK, MOE_BUF_RECV_ROWS, MOE_BUF_RECV_SCALES, MOE_BUF_SEND_ROWS,
    MOE_BUF_SEND_SCALES, MOE_BUF_WORKSPACE, MOE_ERR_BAD_TOPK, MOE_ERR_CAPACITY,
    MOE_ERR_DEVICE_BOUNDS, MOE_ERR_HANDLE, MOE_ERR_HIP, MOE_ERR_INVALID_ARG, MOE_ERR_NONFINITE,
    MOE_ERR_STALE_LAYOUT, MOE_ERR_UNSUPPORTED, ERR_FLAG_BAD_TOPK, ERR_FLAG_BOUNDS, ERR_FLAG_CAPACITY,
    ERR_FLAG_NONFINITE, ERR_FLAG_STALE, StaticConfig,
    MOE_KERNEL_COMBINE, MOE_KERNEL_COMBINE_BWD, MOE_KERNEL_DISPATCH, MOE_KERNEL_DISPATCH_BWD,
    MOE_KERNEL_LAYOUT, MOE_LAYOUT_CONTIGUOUS, MOE_LAYOUT_PADDED_LL, MOE_OK, MOE_QUANT_BF16,
    MOE_QUANT_FP8_E4M3, load_library, make_config, moe_combine, moe_combine_backward, moe_dispatch,
    moe_dispatch_backward, moe_dispatch_layout, moe_dispatch_noalloc, moe_poll_error, moe_size_hint, prepare_combine,
    prepare_dispatch, status_str)
