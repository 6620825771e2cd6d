/*
 * moe_ep.h -- C ABI of libmoe_ep.so: MoE token dispatch-layout, dispatch and
 * combine for one AMD Instinct MI355X (gfx950).
 *
 * What the library computes (the pages describe it in prose only):
 *  - "DeepEP cross-node optimisation guide" (cyqw.cn), opening paragraph: the
 *    all-to-all GPU kernels of an expert-parallel MoE library are "dispatch"
 *    (send each token's hidden vector to the experts its router picked) and
 *    "combine" (bring the expert outputs back and reduce them), with FP8
 *    support.
 *  - Same page, "Core API example": dispatch takes hidden_states, topk_idx,
 *    num_max_dispatch_tokens_per_rank and num_experts; combine takes the expert
 *    outputs, topk_weights and the handle returned by dispatch.
 *  - Same page, figure caption in "Technical analysis": the layout (per-expert
 *    and per-rank counts, token->rank map) is computed once and reused.
 *  - Same page, "Low-latency mode key features" and "Performance tuning":
 *    buffers are preallocated (with a size-hint call) and fixed-size, so no
 *    allocation happens at run time.
 *  - DeepTech release article on DeepEP (010bt.com), paragraph defining EP:
 *    different experts live on different ranks.  Here expert e lives on
 *    virtual rank e / (E / R).
 * With a single GPU the transfer to peer ranks is a local copy: dispatch
 * writes the per-destination-rank send buffers and the receive layout the
 * experts read, combine reads expert outputs from that receive layout.
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless marked "host".  The caller allocates
 *    and owns every buffer passed in or out (size them with moe_size_hint:
 *    all sizes are static upper bounds, so no call ever needs a host sync).
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Every
 *    data-path call only enqueues work on that stream and returns; it never
 *    blocks and never allocates device memory.
 *  - A context is bound to the HIP device current at moe_ctx_create and to
 *    one stream at a time; it is not thread-safe.  Calls made on another
 *    device return MOE_ERR_INVALID_ARG.
 *  - Argument errors are reported synchronously by the return value and leave
 *    nothing enqueued.  Data errors found by the kernels are recorded in a
 *    sticky device word that moe_poll_error reads: an expert id outside
 *    [-1, E) (the slot is treated as empty, -1), a row index outside its
 *    buffer or a low-latency window overflow (the row is not placed), a reused
 *    layout made from other routing (the changed tokens are dropped, see
 *    moe_dispatch) and Inf or NaN in an fp8 dispatch (those blocks'
 *    codes and scales are unspecified).
 *  - bf16 buffers are passed as raw 16-bit storage; fp8 buffers hold OCP
 *    E4M3FN codes, one byte per channel.
 *  - With MOE_EP_LOG=1 in the environment when a context is created, each
 *    kernel launch of that context is logged on stderr (host side only; no
 *    effect on results).
 */
#ifndef MOE_EP_H
#define MOE_EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_EP_ABI_VERSION 5   /* 3: moe_timing_launches; 4: stale-layout and non-finite
                                  flags, moe_dispatch_noalloc; 5: moe_dispatch_layout_prefetch */

/* ---------------------------------------------------------------- status */
typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,   /* NULL pointer, bad size, wrong device, bad config value */
    MOE_ERR_UNSUPPORTED = 2,   /* outside the supported limits below */
    MOE_ERR_CAPACITY = 3,      /* num_tokens > max_tokens (low-latency: > capacity per source rank);
                                  also from moe_poll_error: a low-latency slot window overflowed
                                  (a token repeated an expert), the rows past it were not placed */
    MOE_ERR_HANDLE = 4,        /* handle not produced by moe_dispatch on a compatible context */
    MOE_ERR_HIP = 5,           /* a HIP runtime call failed */
    MOE_ERR_BAD_TOPK = 6,      /* from moe_poll_error: an expert id outside [-1, E) was seen */
    MOE_ERR_DEVICE_BOUNDS = 7, /* from moe_poll_error: a computed row fell outside its buffer;
                                  the row was dropped */
    MOE_ERR_STALE_LAYOUT = 8,  /* from moe_poll_error: a moe_dispatch with reuse_layout = 1 found
                                  topk_idx entries that differ from the ones its layout was
                                  computed from (rewritten in place in between); every such
                                  token was dropped (pos -1, no rows written) */
    MOE_ERR_NONFINITE = 9      /* from moe_poll_error: an fp8 dispatch met Inf or NaN in a
                                  128-channel block of x; that block's codes and scale are
                                  unspecified (every other block is exact) */
} moe_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_str(moe_status s);

/* ---------------------------------------------------------------- config */
typedef enum moe_quant {
    MOE_QUANT_BF16 = 0,        /* payload rows are the bf16 input rows */
    MOE_QUANT_FP8_E4M3 = 1     /* payload rows are E4M3FN codes + one fp32 dequant scale
                                  per 128 channels (kdjingpai.com DeepEP tutorial,
                                  "Function 3: FP8 operation optimisation"; guide,
                                  production setting "FP8 dispatch") */
} moe_quant;

typedef enum moe_layout {
    MOE_LAYOUT_CONTIGUOUS = 0, /* normal (high-throughput) mode: packed rank-major send
                                  buffer + contiguous expert-major receive rows */
    MOE_LAYOUT_PADDED_LL = 1   /* low-latency mode: fixed slots, receive buffer
                                  [R][E/R][max_tokens*R][row], no send buffer */
} moe_layout;

/* Supported limits (checked by moe_ctx_create / moe_size_hint). */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_RANKS   64
#define MOE_MAX_TOPK    32
#define MOE_MAX_HIDDEN  32768

typedef struct moe_config {
    int32_t max_tokens;   /* M >= 1: upper bound on num_tokens of every call; in
                             MOE_LAYOUT_PADDED_LL it is also the per-source-rank slot
                             capacity (the pages' num_max_dispatch_tokens_per_rank) */
    int32_t hidden;       /* H: channels per token; multiple of 8 (bf16), of 128 (fp8) */
    int32_t num_experts;  /* E, 1..MOE_MAX_EXPERTS, multiple of num_ranks */
    int32_t num_ranks;    /* R, 1..MOE_MAX_RANKS: virtual EP ranks; expert e -> rank e/(E/R) */
    int32_t topk;         /* k, 1..MOE_MAX_TOPK: slots per token in topk_idx */
    int32_t src_rank;     /* s0 in [0, R): this GPU's rank (selects its low-latency slots) */
    int32_t quant;        /* moe_quant */
    int32_t layout;       /* moe_layout */
} moe_config;

/* ---------------------------------------------------------------- sizes */
typedef enum moe_buffer_kind {
    MOE_BUF_SEND_ROWS = 0,      /* [max_tokens*min(k,R), row_bytes]; 0 in PADDED_LL */
    MOE_BUF_SEND_SCALES = 1,    /* fp32 [max_tokens*min(k,R), H/128]; 0 unless fp8 and CONTIGUOUS */
    MOE_BUF_RECV_ROWS = 2,      /* CONTIGUOUS: [max_tokens*k, row_bytes];
                                   PADDED_LL: [E, max_tokens*R, row_bytes] */
    MOE_BUF_RECV_SCALES = 3,    /* fp32, same row count as RECV_ROWS, H/128 per row; 0 for bf16 */
    MOE_BUF_EXPERT_OUT = 4,     /* bf16 expert outputs read by combine: RECV_ROWS' row count x 2H */
    MOE_BUF_COMBINE_OUT = 5,    /* bf16 [max_tokens, H] */
    MOE_BUF_HANDLE_POS = 6,     /* int32 [max_tokens, k] */
    MOE_BUF_HANDLE_EXPERT_OFFSETS = 7,  /* int32 [E+1] */
    MOE_BUF_HANDLE_RANK_OFFSETS = 8,    /* int32 [R+1] */
    MOE_BUF_HANDLE_SEND_SRC = 9,        /* int32 [max_tokens*min(k,R)] */
    MOE_BUF_HANDLE_RECV_SRC = 10,       /* int32 [max_tokens*k] */
    MOE_BUF_HANDLE_RECV_COUNTS = 11,    /* int32 [E] */
    MOE_BUF_LAYOUT_EXPERT_COUNTS = 12,  /* int32 [E] */
    MOE_BUF_LAYOUT_RANK_COUNTS = 13,    /* int32 [R] */
    MOE_BUF_LAYOUT_TOKEN_IN_RANK = 14,  /* uint8 [max_tokens, R] */
    MOE_BUF_WORKSPACE = 15,             /* device scratch the context allocates itself */
    MOE_BUF_KIND_COUNT = 16
} moe_buffer_kind;

/* Bytes needed for one buffer kind under `cfg` (host pointers): the pages'
 * size-hint call for preallocated, fixed-size buffers (guide, "Low-latency
 * mode key features": a size hint and pre-allocation; "Performance tuning":
 * buffers made once with low_latency_mode=True, fixed-size buffers instead of
 * queues).  Every size is a static upper bound for num_tokens <= max_tokens.
 * Pure host computation; needs no GPU.  Returns MOE_ERR_INVALID_ARG /
 * UNSUPPORTED for a bad config or kind. */
moe_status moe_size_hint(const moe_config* cfg, int32_t kind, size_t* bytes);

/* ---------------------------------------------------------------- context */
typedef struct moe_ctx moe_ctx;

/* Validate `cfg` (host) and allocate the context and its device workspace
 * (per-tile histograms and scan state, within-tile ranks, error word) on the
 * current HIP device: the pages' preallocated Buffer (guide, "Low-latency mode
 * key features": pre-allocation to avoid run-time allocation; "Performance
 * tuning": the buffer is created once, in low-latency mode with
 * low_latency_mode=True).  The only call that allocates.  On error *out is
 * NULL. */
moe_status moe_ctx_create(const moe_config* cfg, moe_ctx** out);

/* Free the context.  Synchronizes the device first.  NULL is a no-op. */
moe_status moe_ctx_destroy(moe_ctx* ctx);

/* Copy of the configuration the context was created with (host). */
moe_status moe_ctx_config(const moe_ctx* ctx, moe_config* out);

/* Launch-geometry override, for measurement sweeps: 16-byte chunks each lane
 * moves per work item in the dispatch and combine kernels (1, 2, 4, 8 or 16;
 * the combine value also applies to both backward kernels).  0 = the built-in
 * choice: one chunk per lane for the dispatch, two for the combine and the
 * dispatch backward, at most 8 row slices per token for the combine backward,
 * fewer chunks per lane when there are too few tokens to fill the chip.  The
 * fused low-latency dispatch ignores it.  Results do not depend on it. */
moe_status moe_ctx_tune(moe_ctx* ctx, int32_t dispatch_chunks, int32_t combine_chunks);

/* ---------------------------------------------------------------- layout */
/* Dispatch layout (guide, figure caption in "Technical analysis": computed once,
 * reused by dispatch and combine).
 *   topk_idx               int64 [num_tokens, k], row-major; -1 = empty slot
 *   num_tokens_per_expert  int32 [E]:  valid slots routed to expert e
 *   num_tokens_per_rank    int32 [R]:  tokens with at least one expert on rank r
 *   is_token_in_rank       uint8 [num_tokens, R]: 1 iff token t goes to rank r
 *                          (any alignment; 32-bit stores when it is 4-byte
 *                          aligned and R % 4 == 0, byte stores otherwise)
 * Any output pointer may be NULL (not written).  0 <= num_tokens <= max_tokens.
 * Also keeps, in the context's workspace, the scan state a following
 * moe_dispatch(..., reuse_layout = 1) consumes. */
moe_status moe_dispatch_layout(moe_ctx* ctx, const int64_t* topk_idx, int32_t num_tokens,
                               int32_t* num_tokens_per_expert, int32_t* num_tokens_per_rank,
                               uint8_t* is_token_in_rank, void* stream);

/* The dispatch layout, plus a read of the token rows the dispatch reusing
 * this layout will copy (an MI355X-specific addition; the pages' layout call
 * takes topk_idx only).  The layout runs on one workgroup per 256 tokens and is
 * bound by dependent latencies for several microseconds, while HBM is idle; the
 * launch's other workgroups, on the compute units the layout leaves free, read
 * x meanwhile (its first 96 MB), so that the dispatch finds those rows in the
 * 256 MB Infinity Cache instead of HBM.  Outputs, checks and the reused state
 * are those of moe_dispatch_layout; results are identical.
 *   x   bf16 [num_tokens, H], 16-byte aligned, only read; NULL = exactly
 *       moe_dispatch_layout.  Rows of under 2 MB in all are not read.  Under
 *       a workgroup cap (moe_ctx_set_max_workgroups) the extra workgroups,
 *       512 threads each, stay within it (none below a cap of 2).
 * moe_dispatch with reuse_layout = 0 does the same inside its own layout
 * launch. */
moe_status moe_dispatch_layout_prefetch(moe_ctx* ctx, const int64_t* topk_idx, int32_t num_tokens,
                                        const void* x, int32_t* num_tokens_per_expert,
                                        int32_t* num_tokens_per_rank, uint8_t* is_token_in_rank,
                                        void* stream);

/* ---------------------------------------------------------------- dispatch */
/* Output buffers of one dispatch (host struct of device pointers).
 * row_bytes = 2H (bf16) or H (fp8).  Row order:
 *   send:  rank-major; rows [rank_offsets[r], rank_offsets[r+1]) go to rank r,
 *          ascending token index inside each rank.
 *   recv:  CONTIGUOUS: expert-major, rows [expert_offsets[e], expert_offsets[e+1])
 *          for expert e, ordered by (token, slot);
 *          PADDED_LL: row e*cap + s0*M + i (cap = M*R) holds the i-th token
 *          routed to expert e, for i < M; other slots are never written.  A
 *          row with i >= M (possible only when a token repeats an expert)
 *          is not placed: its pos is -1 and moe_poll_error reports
 *          MOE_ERR_CAPACITY.
 * Scales (fp8 only) are fp32 [rows, H/128], row-parallel to the data rows. */
typedef struct moe_dispatch_buffers {
    void*  send_rows;     /* CONTIGUOUS: required; PADDED_LL: must be NULL */
    float* send_scales;   /* fp8 + CONTIGUOUS: required; else NULL */
    void*  recv_rows;     /* required */
    float* recv_scales;   /* fp8: required; else NULL */
} moe_dispatch_buffers;

/* Routing record written by moe_dispatch and read by moe_combine (host struct
 * of caller-owned device buffers, sized by the MOE_BUF_HANDLE_* hints).  The
 * pages' handle is returned by dispatch and passed to combine (guide, "Core
 * API example").  Here the caller owns the storage and the handle carries a
 * tag of the configuration that produced it, instead of a generation counter
 * held by the library: a handle stays valid until the caller reuses its
 * arrays, and moe_combine rejects one from an incompatible configuration
 * (MOE_ERR_HANDLE) rather than reporting a stale generation.
 *   pos[t, j]        row of slot j of token t in the receive layout
 *                    (CONTIGUOUS: expert-major row; PADDED_LL: e*cap + slot),
 *                    -1 for an empty slot or a row that was not placed
 *   expert_offsets   exclusive prefix sum of the per-expert counts (E+1)
 *   rank_offsets     exclusive prefix sum of the per-rank token counts (R+1)
 *   send_src_idx[i]  token of send row i (rank_offsets[R] entries)
 *   recv_src_idx[i]  token of expert-major row i (expert_offsets[E] entries;
 *                    in PADDED_LL the i-th row of expert e is slot s0*M + i -
 *                    expert_offsets[e])
 *   recv_counts[e]   rows received by expert e
 * num_tokens and tag are written by moe_dispatch (host) and checked by
 * moe_combine. */
typedef struct moe_handle {
    int32_t* pos;
    int32_t* expert_offsets;
    int32_t* rank_offsets;
    int32_t* send_src_idx;
    int32_t* recv_src_idx;
    int32_t* recv_counts;
    int32_t  num_tokens;
    uint32_t tag;
} moe_handle;

/* MoE dispatch (guide, "Core API example"; DeepTech article, feature list).
 *   x          bf16 [num_tokens, H] token hidden states
 *   topk_idx   int64 [num_tokens, k]; -1 = empty slot
 *   reuse_layout  0: compute the layout first (one extra kernel; in
 *                    MOE_LAYOUT_PADDED_LL with num_tokens * topk <= 2048 and
 *                    num_tokens <= 512 the
 *                    routing and the copy run as one fused launch instead);
 *                 1: reuse the scan state of the last layout computed on this
 *                    context (by moe_dispatch_layout, or inside a moe_dispatch
 *                    with reuse_layout = 0), which must have seen the same
 *                    topk_idx pointer and num_tokens (checked on the host).
 *                    The contents must not have changed either: the kernel
 *                    compares every entry with the expert id the layout
 *                    recorded, drops each token with a changed entry and sets
 *                    MOE_ERR_STALE_LAYOUT (moe_poll_error)
 *   bufs       output rows (and scales for fp8)
 *   handle     host struct; its device arrays are written, num_tokens/tag set
 * fp8 rows: per token and 128-channel block, a = max|x|, a' = max(a, 1e-4),
 * codes = E4M3(x * (448/a')) with round-to-nearest-even (saturating), stored
 * scale = a'/448.  Every destination gets the same bytes.  The rows must be
 * finite: for a block holding Inf or NaN the codes and scale are unspecified
 * and moe_poll_error reports MOE_ERR_NONFINITE (bf16 rows are copied bit for
 * bit whatever they hold). */
moe_status moe_dispatch(moe_ctx* ctx, const void* x, const int64_t* topk_idx, int32_t num_tokens,
                        int32_t reuse_layout, const moe_dispatch_buffers* bufs,
                        moe_handle* handle, void* stream);

/* ---------------------------------------------------------------- combine */
/* MoE combine (guide, "Core API example" and the production setting's
 * "BF16 combine").
 *   expert_out   bf16 rows in the receive layout of the handle (row pos[t, j])
 *   topk_weights fp32 [num_tokens, k]
 *   out          bf16 [num_tokens, H]
 * out[t, h] = bf16_rne( sum over valid j, ascending, of w[t, j] * y[pos[t, j], h] ),
 * accumulated in fp32 from +0 with separately rounded multiply and add. */
moe_status moe_combine(moe_ctx* ctx, const void* expert_out, const float* topk_weights,
                       const moe_handle* handle, void* out, void* stream);

/* ---------------------------------------------------------------- backward */
/* Gradients of dispatch and combine for training (DeepTech release article,
 * feature list: the high-throughput kernels serve training).  The pages give
 * no formulas; these are the derivatives of the forward definitions above,
 * with the bf16 roundings and the FP8 quantisation passed through as the
 * identity.  Gradients are bf16 in every quant mode.  Both calls read the
 * routing from a handle of the last moe_dispatch (same checks as moe_combine)
 * and return MOE_OK at once when it holds no tokens.
 *
 * moe_dispatch_backward: the adjoint of dispatch's copy into the receive rows.
 *   grad_recv  bf16 rows in the receive layout of the handle (row pos[t, j]
 *              holds the gradient of the copy of token t for slot j)
 *   grad_x     bf16 [num_tokens, H] output
 * grad_x[t, h] = bf16_rne( sum over valid j, ascending, of grad_recv[pos[t, j], h] ),
 * accumulated in fp32 from +0 (combine with every weight 1; a token with no
 * valid slot gets +0).  Send rows carry no gradient of their own: in a
 * multi-GPU exchange they are the transport of the receive rows. */
moe_status moe_dispatch_backward(moe_ctx* ctx, const void* grad_recv, const moe_handle* handle,
                                 void* grad_x, void* stream);

/* moe_combine_backward: gradients of combine with respect to the expert outputs
 * and the weights.
 *   grad_out         bf16 [num_tokens, H] gradient of combine's output
 *   topk_weights     fp32 [num_tokens, k], as passed to moe_combine
 *   expert_out       bf16 rows in the receive layout, as passed to moe_combine
 *   grad_expert_out  bf16 output rows in the receive layout: for each valid
 *                    slot, row pos[t, j] = bf16_rne(w[t, j] * grad_out[t])
 *                    (fp32 product, then one rounding); rows no slot points
 *                    at are not written
 *   grad_weights     fp32 [num_tokens, k] output: the dot product of
 *                    grad_out[t] with expert_out[pos[t, j]] (fp32 sums of the
 *                    exact bf16 products, in a fixed order; 0 for an empty slot) */
moe_status moe_combine_backward(moe_ctx* ctx, const void* grad_out, const float* topk_weights,
                                const void* expert_out, const moe_handle* handle,
                                void* grad_expert_out, float* grad_weights, void* stream);

/* ---------------------------------------------------------------- overlap */
/* Resource control (DeepTech release article, feature list: flexible GPU
 * resource control and SM-count control for the high-throughput kernels; the
 * guide's resource-control section sets an SM limit).  At most
 * `max_workgroups` workgroups (0 = no cap, the default) run the dispatch
 * (layout-reusing or two-launch path), combine and backward kernels of this
 * context; each workgroup then loops over more rows, so results are
 * unchanged.  A workgroup is 256 threads for the dispatch and 64 threads per
 * row slice (up to 1024) for the combine backward; the combine and the
 * dispatch backward run one-wavefront workgroups, 4 * max_workgroups of them
 * (the wavefronts of max_workgroups 256-thread workgroups).  The layout's
 * tile workgroups (one per 256 tokens) and the fused low-latency dispatch
 * (the pages: low-latency kernels need no SM control) are not capped; the
 * extra workgroups a layout launch uses to read x are (512 threads each, so
 * max_workgroups / 2 of them).  Capping leaves
 * compute units to kernels on other streams, e.g. GEMMs overlapped with
 * dispatch and combine. */
moe_status moe_ctx_set_max_workgroups(moe_ctx* ctx, int32_t max_workgroups);

/* Issue/complete split (the guide's hook-based communication-computation
 * overlap, "Technical analysis"): enqueue dispatch or combine on a side stream,
 * record a hook there right after it (the issue side returns at once), keep
 * enqueuing compute on the main stream, and call moe_hook_wait on the main
 * stream where the results are first needed (the complete side).  No kernel
 * waits on the device in between.  A hook is a host object bound to the
 * device current at moe_hook_create; it may be recorded again after each
 * wait.  moe_hook_wait with a never-recorded hook returns at once. */
typedef struct moe_hook moe_hook;
moe_status moe_hook_create(moe_hook** out);
moe_status moe_hook_destroy(moe_hook* hook);
moe_status moe_hook_record(moe_hook* hook, void* stream);
moe_status moe_hook_wait(const moe_hook* hook, void* stream);

/* ---------------------------------------------------------------- errors */
/* Synchronize `stream`, read and clear the sticky device error word.
 * Returns MOE_OK, MOE_ERR_BAD_TOPK, MOE_ERR_STALE_LAYOUT, MOE_ERR_CAPACITY,
 * MOE_ERR_DEVICE_BOUNDS or MOE_ERR_NONFINITE (the first set, in that order);
 * *flags (host, may be NULL) receives the raw bits (1: bad expert id, 2: row
 * outside its buffer, 4: low-latency window overflow, 8: stale reused layout,
 * 16: non-finite fp8 input). */
moe_status moe_poll_error(moe_ctx* ctx, void* stream, uint32_t* flags);

/* ---------------------------------------------------------------- timing */
/* Per-kernel timing with HIP events recorded on the launch stream around each
 * kernel the context enqueues.  Off by default.  moe_timing_begin allocates
 * `max_launches` event pairs (host-side HIP objects, not device memory);
 * moe_timing_end synchronizes on the last event, writes per-kernel totals
 * (milliseconds) and launch counts (host arrays of MOE_KERNEL_COUNT entries)
 * and frees the events.  Launches beyond max_launches are not timed. */
typedef enum moe_kernel_id {
    MOE_KERNEL_LAYOUT = 0,   /* count + scan */
    MOE_KERNEL_DISPATCH = 1, /* pack / permute / quantise */
    MOE_KERNEL_COMBINE = 2,  /* gather-reduce */
    MOE_KERNEL_DISPATCH_BWD = 3,  /* dispatch backward (gather-sum) */
    MOE_KERNEL_COMBINE_BWD = 4,   /* combine backward (weighted scatter + dot products) */
    MOE_KERNEL_COUNT = 5
} moe_kernel_id;

moe_status moe_timing_begin(moe_ctx* ctx, int32_t max_launches);
moe_status moe_timing_end(moe_ctx* ctx, double* total_ms, int64_t* launches);

/* Per-launch durations of the timing window opened by moe_timing_begin, for
 * percentiles (call before moe_timing_end, which frees the events).  Writes
 * the kernel id (moe_kernel_id) and duration in milliseconds of the first
 * min(capacity, count) timed launches, in launch order, into the host arrays
 * kernel_ids and ms, and the number of timed launches into *count (host).
 * Synchronizes on each launch's end event.  MOE_ERR_INVALID_ARG without an
 * open timing window or with NULL arrays for capacity > 0. */
moe_status moe_timing_launches(moe_ctx* ctx, int32_t* kernel_ids, float* ms, int32_t capacity,
                               int32_t* count);

/* ---------------------------------------------------------------- no allocation */
/* For callers that cannot allocate device memory at all: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same result
 * as moe_dispatch(reuse_layout = 0) on a context created with *cfg (the same
 * rows, scales and handle arrays; the handle is accepted by moe_combine and
 * the backward calls of any context with an equal configuration), without a
 * context: the layout workspace is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES per GPU, loaded with the library and held until
 * the process ends, and this call makes no allocation of any kind.
 *   cfg         host; checked like moe_ctx_create.  MOE_ERR_CAPACITY when the
 *               workspace it needs (MOE_BUF_WORKSPACE) exceeds the scratch.
 *   x, topk_idx, num_tokens, bufs, handle: as in moe_dispatch.
 *   error_word  device uint32, nullable: the kernels OR the moe_poll_error
 *               bits into it (the caller clears it); NULL = not reported.
 * The scratch keeps the last call's contents; the words that must start at
 * zero are zeroed on the first call on each device and left zero by every
 * call.  Calls that overlap on one GPU (other streams, other threads) race on
 * the scratch and give wrong results: serialize them.  No launch tuning or
 * workgroup cap applies, and no kernel timing is recorded. */
#define MOE_NOALLOC_SCRATCH_BYTES (8u << 20)
moe_status moe_dispatch_noalloc(const moe_config* cfg, const void* x, const int64_t* topk_idx,
                                int32_t num_tokens, const moe_dispatch_buffers* bufs,
                                moe_handle* handle, uint32_t* error_word, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_EP_H */
