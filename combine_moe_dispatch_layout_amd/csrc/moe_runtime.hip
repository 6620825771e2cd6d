// Host runtime behind the C ABI in include/moe_ep.h: configuration checks,
// buffer sizing, the context and its device workspace, launch geometry,
// handle validation, the sticky device error word and optional kernel timing.
//
// Nothing here allocates after moe_ctx_create (the pages' "pre-allocation"
// and "fixed-size buffers instead of queues": "DeepEP cross-node optimisation
// guide", "Low-latency mode key features" and "Performance tuning").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "moe_ep.h"
#include "moe_internal.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

using namespace moe;

namespace {

constexpr uint32_t kTagMagic = 0x4d6f4500u;   // "MoE\0"

struct Geometry {
    int El, ksend, ntiles_max, rbits;
    int64_t cap, row_bytes, nb;
    int64_t send_rows, recv_rows;
};

int bits_for(int n) {   // bits needed to hold values 0..n-1
    int b = 0;
    while ((1 << b) < n) ++b;
    return b;
}

moe_status check_config(const moe_config* c, Geometry* g) {
    if (c == nullptr) return MOE_ERR_INVALID_ARG;
    if (c->max_tokens < 1 || c->hidden < 1 || c->num_experts < 1 || c->num_ranks < 1 || c->topk < 1)
        return MOE_ERR_INVALID_ARG;
    if (c->src_rank < 0 || c->src_rank >= c->num_ranks) return MOE_ERR_INVALID_ARG;
    if (c->quant != MOE_QUANT_BF16 && c->quant != MOE_QUANT_FP8_E4M3) return MOE_ERR_INVALID_ARG;
    if (c->layout != MOE_LAYOUT_CONTIGUOUS && c->layout != MOE_LAYOUT_PADDED_LL) return MOE_ERR_INVALID_ARG;
    if (c->num_experts > MOE_MAX_EXPERTS || c->num_ranks > MOE_MAX_RANKS || c->topk > MOE_MAX_TOPK ||
        c->hidden > MOE_MAX_HIDDEN)
        return MOE_ERR_UNSUPPORTED;
    if (c->num_experts % c->num_ranks != 0) return MOE_ERR_UNSUPPORTED;
    if (c->hidden % (c->quant == MOE_QUANT_FP8_E4M3 ? 128 : 8) != 0) return MOE_ERR_UNSUPPORTED;
    Geometry q;
    q.El = c->num_experts / c->num_ranks;
    q.ksend = std::min(c->topk, c->num_ranks);
    q.ntiles_max = (c->max_tokens + kTileTokens - 1) / kTileTokens;
    q.rbits = bits_for(c->num_ranks);
    q.cap = (int64_t)c->max_tokens * c->num_ranks;
    q.row_bytes = c->quant == MOE_QUANT_FP8_E4M3 ? c->hidden : 2 * (int64_t)c->hidden;
    q.nb = c->hidden / 128;
    q.send_rows = c->layout == MOE_LAYOUT_PADDED_LL ? 0 : (int64_t)c->max_tokens * q.ksend;
    q.recv_rows = c->layout == MOE_LAYOUT_PADDED_LL ? (int64_t)c->num_experts * q.cap
                                                    : (int64_t)c->max_tokens * c->topk;
    // row indices and flat (token, slot) indices are int32 on the device
    if ((int64_t)c->max_tokens * c->topk >= INT32_MAX || q.recv_rows >= INT32_MAX ||
        (int64_t)c->max_tokens * c->num_ranks >= INT32_MAX)
        return MOE_ERR_UNSUPPORTED;
    if (g) *g = q;
    return MOE_OK;
}

// Workspace layout (device, one allocation, 256-byte aligned pieces).  The
// first pieces -- error word, arrival counter and the grand totals, sized for
// the largest supported E + R -- sit at the same offsets for every
// configuration, so that a workspace shared by calls of different
// configurations (the allocation-free dispatch's static scratch) keeps the
// words that must read zero at the start of a layout zero: each layout zeroes
// the totals it used before it ends.
struct Workspace {
    size_t off_err, off_done, off_sink, off_cnt_e, off_cnt_r, off_eoff, off_roff, off_tile_cnt, off_grand_tot,
        off_erank, off_srank, total;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int tile_stride(const Geometry& g) { return (g.ntiles_max + 3) & ~3; }

int cnt_stride(const moe_config* c) { return (c->num_experts + c->num_ranks + 63) & ~63; }

Workspace plan_workspace(const moe_config* c, const Geometry& g) {
    Workspace w;
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
    w.off_err = take(4);
    w.off_done = take(4);
    w.off_sink = take(4);
    w.off_grand_tot = take(4 * ((size_t)MOE_MAX_EXPERTS + MOE_MAX_RANKS));
    w.off_cnt_e = take(4 * (size_t)c->num_experts);
    w.off_cnt_r = take(4 * (size_t)c->num_ranks);
    w.off_eoff = take(4 * ((size_t)c->num_experts + 1));
    w.off_roff = take(4 * ((size_t)c->num_ranks + 1));
    // per-tile counts in either arrangement (column by column, or tile by tile)
    w.off_tile_cnt = take(4 * std::max((size_t)tile_stride(g) * (c->num_experts + c->num_ranks),
                                       (size_t)g.ntiles_max * cnt_stride(c)));
    w.off_erank = take(4 * (size_t)c->max_tokens * c->topk);
    w.off_srank = take(2 * (size_t)c->max_tokens * c->num_ranks);
    w.total = o;
    return w;
}

uint32_t config_tag(const moe_config* c) {
    uint32_t h = 2166136261u;   // FNV-1a over the config fields
    const int32_t f[8] = {c->max_tokens, c->hidden, c->num_experts, c->num_ranks,
                          c->topk, c->src_rank, c->quant, c->layout};
    const unsigned char* b = reinterpret_cast<const unsigned char*>(f);
    for (size_t i = 0; i < sizeof(f); ++i) h = (h ^ b[i]) * 16777619u;
    return (h & 0xffffff00u) ^ kTagMagic;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Work split of a row-streaming kernel: each wavefront handles `chunks`
// 16-byte chunks per lane of one token row (a "slice"), at most `cap`.  Rows
// are cut into more slices when there are too few tokens to keep ~8
// wavefronts per CU in flight.  Measured on MI355X: with its non-temporal
// row stores the dispatch is fastest with one chunk per lane (5-11% ahead of
// whole rows per wavefront on the prefill, grouped and skewed shapes).  The
// combine (and the dispatch backward, the same kernel) takes two: one chunk
// per lane is within 1% on the prefill shape in every cache state and 2%
// faster on skewed shapes; four are 7-20% slower.  The combine backward wants at most 8
// slices per token (one chunk per lane up to 512 chunks per row, then two),
// which is faster in every cache state measured.
void row_split(int64_t T, int64_t nchunk, int forced, int cap, int* chunks, int* nslices) {
    int c;
    if (forced > 0) {
        c = forced;
    } else {
        const int64_t per_lane = (nchunk + 63) / 64;
        c = 1;
        while (c < cap && c < per_lane) c *= 2;
        const int64_t target_items = 256 * 8;
        while (c > 1 && T * ((nchunk + 64 * c - 1) / (64 * c)) < target_items) c /= 2;
    }
    *chunks = c;
    *nslices = (int)((nchunk + 64 * c - 1) / (64 * c));
}

// The status moe_poll_error reports for a set of device error bits.
moe_status status_of_flags(uint32_t v) {
    if (v & kErrBadTopk) return MOE_ERR_BAD_TOPK;
    if (v & kErrStale) return MOE_ERR_STALE_LAYOUT;
    if (v & kErrCapacity) return MOE_ERR_CAPACITY;
    if (v & kErrBounds) return MOE_ERR_DEVICE_BOUNDS;
    if (v & kErrNonFinite) return MOE_ERR_NONFINITE;
    return MOE_OK;
}

}  // namespace

struct moe_ctx {
    moe_config cfg;
    Geometry g;
    Workspace wl;
    int device;
    char* ws;
    uint32_t tag;
    // last layout computed into the workspace, and the mode it ran in
    const int64_t* layout_idx;
    int32_t layout_T;
    int32_t layout_mode;
    bool layout_valid;
    // tuning overrides (0 = heuristic)
    int pack_chunks, combine_chunks;
    // cap on the workgroups of the high-throughput kernels (0 = none)
    int max_blocks;
    // host-side launch log on stderr (environment MOE_EP_LOG=1 at context creation)
    bool log;
    // timing
    bool timing;
    int max_launches;
    std::vector<hipEvent_t> ev0, ev1;
    std::vector<int> kid;

    uint32_t* err() { return reinterpret_cast<uint32_t*>(ws + wl.off_err); }
};

namespace {

bool on_ctx_device(const moe_ctx* ctx) {
    int dev = -1;
    return hipGetDevice(&dev) == hipSuccess && dev == ctx->device;
}

const char* kernel_name(int id) {
    static const char* names[MOE_KERNEL_COUNT] = {"layout", "dispatch", "combine", "dispatch_backward",
                                                  "combine_backward"};
    return id >= 0 && id < MOE_KERNEL_COUNT ? names[id] : "?";
}

// Record timing events around one launch when timing is on; log it when asked.
// ctx may be NULL (the allocation-free dispatch): then nothing is recorded.
struct TimedLaunch {
    moe_ctx* ctx;
    hipStream_t s;
    int slot;
    TimedLaunch(moe_ctx* c, hipStream_t st, int id) : ctx(c), s(st), slot(-1) {
        if (c == nullptr) return;
        if (c->log)
            std::fprintf(stderr, "[moe_ep] ctx %p: %s on stream %p (max_workgroups %d)\n", static_cast<void*>(c),
                         kernel_name(id), static_cast<void*>(st), c->max_blocks);
        if (c->timing && (int)c->kid.size() < c->max_launches) {
            slot = (int)c->kid.size();
            c->kid.push_back(id);
            (void)hipEventRecord(c->ev0[slot], st);
        }
    }
    void done() {
        if (slot >= 0) (void)hipEventRecord(ctx->ev1[slot], s);
    }
};

// What the launches of one call need besides their arguments: the
// configuration, the device workspace (a context's, or the static scratch of
// the allocation-free dispatch), the error word and the launch tuning.
struct Exec {
    const moe_config* c;
    const Geometry* g;
    const Workspace* wl;
    char* ws;
    uint32_t* err;
    int pack_chunks;
    int max_blocks;
    moe_ctx* ctx;   // timing and launch log; NULL for none
    int32_t* i32(size_t off) const { return reinterpret_cast<int32_t*>(ws + off); }
    uint16_t* u16(size_t off) const { return reinterpret_cast<uint16_t*>(ws + off); }
    uint32_t* u32(size_t off) const { return reinterpret_cast<uint32_t*>(ws + off); }
};

Exec ctx_exec(moe_ctx* ctx) {
    Exec x;
    x.c = &ctx->cfg;
    x.g = &ctx->g;
    x.wl = &ctx->wl;
    x.ws = ctx->ws;
    x.err = ctx->err();
    x.pack_chunks = ctx->pack_chunks;
    x.max_blocks = ctx->max_blocks;
    x.ctx = ctx;
    return x;
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Compute units of a device (cached per device; 0 if the query fails).
int device_cus(int dev) {
    static std::mutex mu;
    static int cus[64];
    if (dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lock(mu);
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess) cus[dev] = n;
    }
    return cus[dev];
}

// Token rows of at least this many bytes are read into the Infinity Cache
// during the layout; at most this many (the first rows, which the dispatch
// reads first; the cache is 256 MB).
constexpr int64_t kWarmMinBytes = 2ll << 20;
constexpr int64_t kWarmMaxBytes = 96ll << 20;
// A workgroup cap counts 256-thread workgroups; the layout's are 512 threads.
constexpr int kLayoutBlockUnits = 2;

// Count + scan launch into the workspace.  *mode receives the layout mode it
// ran in (the dispatch that consumes this layout is told the same mode).
// warm_x (nullable): the bf16 token rows [T, H] of the dispatch that follows;
// the compute units the layout leaves idle read them meanwhile (see k_layout).
moe_status run_layout(const Exec& x, const int64_t* topk_idx, int32_t T, int32_t* out_cnt_e,
                      int32_t* out_cnt_r, uint8_t* out_in_rank, const void* warm_x, hipStream_t s, int* mode) {
    const moe_config& c = *x.c;
    const int ntiles = std::max(1, (T + kTileTokens - 1) / kTileTokens);
    int warm_blocks = 0;
    int64_t warm_bytes = warm_x != nullptr ? std::min<int64_t>((int64_t)T * c.hidden * 2, kWarmMaxBytes) : 0;
    if (warm_bytes >= kWarmMinBytes) {
        int dev = -1;
        (void)hipGetDevice(&dev);
        warm_blocks = std::max(0, device_cus(dev) - ntiles);
        // under a workgroup cap the extra workgroups stay within it too
        if (x.max_blocks > 0) warm_blocks = std::min(warm_blocks, x.max_blocks / kLayoutBlockUnits);
    }
    if (warm_blocks == 0) warm_bytes = 0;
    LayoutArgs a;
    a.topk_idx = topk_idx;
    a.T = T;
    a.k = c.topk;
    a.E = c.num_experts;
    a.R = c.num_ranks;
    a.El = x.g->El;
    a.k_magic = (uint32_t)(((1u << 20) + c.topk - 1) / c.topk);
    a.el_magic = (uint32_t)(((1u << 20) + x.g->El - 1) / x.g->El);
    a.max_tokens = c.max_tokens;
    a.mode = layout_mode(ntiles);
    a.in_rank_vec4 = (c.num_ranks % 4 == 0 && aligned4(out_in_rank)) ? 1 : 0;
    a.tile_cnt = x.i32(x.wl->off_tile_cnt);
    a.tile_stride = tile_stride(*x.g);
    a.cnt_stride = cnt_stride(x.c);
    a.grand_tot = x.i32(x.wl->off_grand_tot);
    a.erank = x.u32(x.wl->off_erank);
    a.srank = x.u16(x.wl->off_srank);
    a.cnt_e = x.i32(x.wl->off_cnt_e);
    a.cnt_r = x.i32(x.wl->off_cnt_r);
    a.eoff = x.i32(x.wl->off_eoff);
    a.roff = x.i32(x.wl->off_roff);
    a.out_cnt_e = out_cnt_e;
    a.out_cnt_r = out_cnt_r;
    a.out_in_rank = out_in_rank;
    a.err = x.err;
    a.done = x.u32(x.wl->off_done);
    a.ntiles = ntiles;
    a.warm = warm_x;
    a.warm_chunks = warm_bytes / 16;
    a.warm_sink = x.u32(x.wl->off_sink);
    TimedLaunch tl(x.ctx, s, MOE_KERNEL_LAYOUT);
    hipError_t e = launch_layout(a, ntiles, warm_blocks, s);
    tl.done();
    *mode = a.mode;
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status check_dispatch_args(const moe_config& c, const void* x, const int64_t* topk_idx, int32_t num_tokens,
                               const moe_dispatch_buffers* bufs, const moe_handle* handle) {
    const bool fp8 = c.quant == MOE_QUANT_FP8_E4M3;
    const bool ll = c.layout == MOE_LAYOUT_PADDED_LL;
    if (bufs == nullptr || handle == nullptr) return MOE_ERR_INVALID_ARG;
    if (num_tokens < 0) return MOE_ERR_INVALID_ARG;
    if (num_tokens > c.max_tokens) return MOE_ERR_CAPACITY;
    if (num_tokens > 0 && (x == nullptr || topk_idx == nullptr)) return MOE_ERR_INVALID_ARG;
    if (bufs->recv_rows == nullptr || !aligned16(x) || !aligned16(bufs->recv_rows)) return MOE_ERR_INVALID_ARG;
    if (ll) {
        if (bufs->send_rows != nullptr || bufs->send_scales != nullptr) return MOE_ERR_INVALID_ARG;
    } else {
        if (bufs->send_rows == nullptr || !aligned16(bufs->send_rows)) return MOE_ERR_INVALID_ARG;
        if (fp8 != (bufs->send_scales != nullptr)) return MOE_ERR_INVALID_ARG;
    }
    if (fp8 != (bufs->recv_scales != nullptr)) return MOE_ERR_INVALID_ARG;
    if (handle->pos == nullptr || handle->expert_offsets == nullptr || handle->rank_offsets == nullptr ||
        handle->send_src_idx == nullptr || handle->recv_src_idx == nullptr || handle->recv_counts == nullptr)
        return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

// The dispatch proper (arguments already checked).  reuse_mode >= 0: reuse
// the layout already in the workspace, computed in that mode; -1: compute it
// here first (or, for decode-sized padded batches, run the fused launch,
// which leaves the workspace alone).  *new_layout_mode receives the mode of a
// layout computed here, else -1.
moe_status run_dispatch(const Exec& xc, const void* x, const int64_t* topk_idx, int32_t num_tokens,
                        int reuse_mode, const moe_dispatch_buffers* bufs, moe_handle* handle, uint32_t tag,
                        hipStream_t s, int* new_layout_mode) {
    *new_layout_mode = -1;
    const moe_config& c = *xc.c;
    const bool fp8 = c.quant == MOE_QUANT_FP8_E4M3;
    const bool ll = c.layout == MOE_LAYOUT_PADDED_LL;
    // low latency without a reused layout: one fused launch when the routing is small
    const bool fused = reuse_mode < 0 && ll && (int64_t)num_tokens * c.topk <= kFusedMaxEntries &&
                       num_tokens <= kFusedMaxTokens;
    int mode = reuse_mode;
    if (reuse_mode < 0 && !fused) {
        moe_status st = run_layout(xc, topk_idx, num_tokens, nullptr, nullptr, nullptr, x, s, &mode);
        if (st != MOE_OK) return st;
        *new_layout_mode = mode;
    }

    PackArgs a;
    a.x = static_cast<const uint16_t*>(x);
    a.topk_idx = topk_idx;
    a.T = num_tokens;
    a.k = c.topk;
    a.E = c.num_experts;
    a.R = c.num_ranks;
    a.El = xc.g->El;
    a.H = c.hidden;
    a.rbits = xc.g->rbits;
    a.max_tokens = c.max_tokens;
    a.s0 = c.src_rank;
    a.cap = xc.g->cap;
    a.tile_cnt = xc.i32(xc.wl->off_tile_cnt);
    a.tile_stride = tile_stride(*xc.g);
    a.cnt_stride = cnt_stride(xc.c);
    a.mode = mode;
    a.erank = xc.u32(xc.wl->off_erank);
    a.srank = xc.u16(xc.wl->off_srank);
    a.cnt_e = xc.i32(xc.wl->off_cnt_e);
    a.eoff = xc.i32(xc.wl->off_eoff);
    a.roff = xc.i32(xc.wl->off_roff);
    a.send_rows = bufs->send_rows;
    a.send_scales = bufs->send_scales;
    a.recv_rows = bufs->recv_rows;
    a.recv_scales = bufs->recv_scales;
    a.send_cap_rows = xc.g->send_rows;
    a.recv_cap_rows = xc.g->recv_rows;
    a.pairs_cap = (int64_t)c.max_tokens * c.topk;
    a.h_pos = handle->pos;
    a.h_eoff = handle->expert_offsets;
    a.h_roff = handle->rank_offsets;
    a.h_send_src = handle->send_src_idx;
    a.h_recv_src = handle->recv_src_idx;
    a.h_recv_counts = handle->recv_counts;
    a.err = xc.err;
    int chunks, nslices;
    row_split(num_tokens, c.hidden / 8, xc.pack_chunks, 1, &chunks, &nslices);
    a.nslices = nslices;
    a.ll_bpt = 1;
    TimedLaunch tl(xc.ctx, s, MOE_KERNEL_DISPATCH);
    hipError_t e;
    if (fused) {
        // ll_bpt blocks per token whose wavefronts each copy one 64-chunk slice:
        // 512-thread blocks when the row has more than 256 chunks (the
        // workspace is neither read nor written here)
        const int64_t nchunk = c.hidden / 8;
        const int nt = nchunk > kBlockThreads ? 512 : kBlockThreads;
        a.nslices = (int)((nchunk + 63) / 64);
        a.ll_bpt = (a.nslices + nt / 64 - 1) / (nt / 64);
        e = launch_ll_fused(a, 1, nt, fp8, s);
    } else if (num_tokens == 0) {
        // grid of one block: block 0 copies the offsets, every wave exits (no
        // items); at least one block so that the handle's offsets and counts
        // are written for T = 0
        a.nslices = 1;
        e = launch_pack(a, 1, fp8, ll, !ll, xc.max_blocks, s);
    } else {
        e = launch_pack(a, chunks, fp8, ll, !ll, xc.max_blocks, s);
    }
    tl.done();
    if (e != hipSuccess) return MOE_ERR_HIP;
    handle->num_tokens = num_tokens;
    handle->tag = tag;
    return MOE_OK;
}

}  // namespace

// ============================================================== C ABI
MOE_API const char* moe_status_str(moe_status s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_CAPACITY: return "MOE_ERR_CAPACITY";
        case MOE_ERR_HANDLE: return "MOE_ERR_HANDLE";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
        case MOE_ERR_BAD_TOPK: return "MOE_ERR_BAD_TOPK";
        case MOE_ERR_DEVICE_BOUNDS: return "MOE_ERR_DEVICE_BOUNDS";
        case MOE_ERR_STALE_LAYOUT: return "MOE_ERR_STALE_LAYOUT";
        case MOE_ERR_NONFINITE: return "MOE_ERR_NONFINITE";
    }
    return "MOE_ERR_UNKNOWN";
}

MOE_API moe_status moe_size_hint(const moe_config* cfg, int32_t kind, size_t* bytes) {
    if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
    *bytes = 0;
    Geometry g;
    moe_status st = check_config(cfg, &g);
    if (st != MOE_OK) return st;
    const bool fp8 = cfg->quant == MOE_QUANT_FP8_E4M3;
    const bool ll = cfg->layout == MOE_LAYOUT_PADDED_LL;
    const size_t M = (size_t)cfg->max_tokens, E = (size_t)cfg->num_experts, R = (size_t)cfg->num_ranks,
                 k = (size_t)cfg->topk, H = (size_t)cfg->hidden;
    switch (kind) {
        case MOE_BUF_SEND_ROWS: *bytes = (size_t)g.send_rows * g.row_bytes; break;
        case MOE_BUF_SEND_SCALES: *bytes = fp8 && !ll ? (size_t)g.send_rows * g.nb * 4 : 0; break;
        case MOE_BUF_RECV_ROWS: *bytes = (size_t)g.recv_rows * g.row_bytes; break;
        case MOE_BUF_RECV_SCALES: *bytes = fp8 ? (size_t)g.recv_rows * g.nb * 4 : 0; break;
        case MOE_BUF_EXPERT_OUT: *bytes = (size_t)g.recv_rows * H * 2; break;
        case MOE_BUF_COMBINE_OUT: *bytes = M * H * 2; break;
        case MOE_BUF_HANDLE_POS: *bytes = M * k * 4; break;
        case MOE_BUF_HANDLE_EXPERT_OFFSETS: *bytes = (E + 1) * 4; break;
        case MOE_BUF_HANDLE_RANK_OFFSETS: *bytes = (R + 1) * 4; break;
        case MOE_BUF_HANDLE_SEND_SRC: *bytes = M * (size_t)g.ksend * 4; break;
        case MOE_BUF_HANDLE_RECV_SRC: *bytes = M * k * 4; break;
        case MOE_BUF_HANDLE_RECV_COUNTS: *bytes = E * 4; break;
        case MOE_BUF_LAYOUT_EXPERT_COUNTS: *bytes = E * 4; break;
        case MOE_BUF_LAYOUT_RANK_COUNTS: *bytes = R * 4; break;
        case MOE_BUF_LAYOUT_TOKEN_IN_RANK: *bytes = M * R; break;
        case MOE_BUF_WORKSPACE: *bytes = plan_workspace(cfg, g).total; break;
        default: return MOE_ERR_INVALID_ARG;
    }
    return MOE_OK;
}

MOE_API moe_status moe_ctx_create(const moe_config* cfg, moe_ctx** out) {
    if (out == nullptr) return MOE_ERR_INVALID_ARG;
    *out = nullptr;
    Geometry g;
    moe_status st = check_config(cfg, &g);
    if (st != MOE_OK) return st;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    moe_ctx* ctx = new (std::nothrow) moe_ctx();
    if (ctx == nullptr) return MOE_ERR_INVALID_ARG;
    ctx->cfg = *cfg;
    ctx->g = g;
    ctx->wl = plan_workspace(cfg, g);
    ctx->device = dev;
    ctx->ws = nullptr;
    ctx->tag = config_tag(cfg);
    ctx->layout_idx = nullptr;
    ctx->layout_T = -1;
    ctx->layout_mode = -1;
    ctx->layout_valid = false;
    ctx->pack_chunks = 0;
    ctx->combine_chunks = 0;
    ctx->max_blocks = 0;
    {
        const char* v = std::getenv("MOE_EP_LOG");
        ctx->log = v != nullptr && v[0] == '1';
    }
    ctx->timing = false;
    ctx->max_launches = 0;
    if (hipMalloc(reinterpret_cast<void**>(&ctx->ws), ctx->wl.total) != hipSuccess) {
        delete ctx;
        return MOE_ERR_HIP;
    }
    // error word, arrival counter and grand totals start at zero
    if (hipMemset(ctx->ws, 0, ctx->wl.total) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
        (void)hipFree(ctx->ws);
        delete ctx;
        return MOE_ERR_HIP;
    }
    *out = ctx;
    return MOE_OK;
}

MOE_API moe_status moe_ctx_destroy(moe_ctx* ctx) {
    if (ctx == nullptr) return MOE_OK;
    moe_status st = MOE_OK;
    if (hipDeviceSynchronize() != hipSuccess) st = MOE_ERR_HIP;
    for (hipEvent_t e : ctx->ev0) (void)hipEventDestroy(e);
    for (hipEvent_t e : ctx->ev1) (void)hipEventDestroy(e);
    if (ctx->ws && hipFree(ctx->ws) != hipSuccess) st = MOE_ERR_HIP;
    delete ctx;
    return st;
}

MOE_API moe_status moe_ctx_config(const moe_ctx* ctx, moe_config* out) {
    if (ctx == nullptr || out == nullptr) return MOE_ERR_INVALID_ARG;
    *out = ctx->cfg;
    return MOE_OK;
}

// Tuning override for sweeps: chunks per lane of the dispatch / combine kernels
// (0 = heuristic; else 1, 2, 4, 8 or 16).
MOE_API moe_status moe_ctx_tune(moe_ctx* ctx, int32_t pack_chunks, int32_t combine_chunks) {
    if (ctx == nullptr) return MOE_ERR_INVALID_ARG;
    auto ok = [](int v) { return v == 0 || v == 1 || v == 2 || v == 4 || v == 8 || v == 16; };
    if (!ok(pack_chunks) || !ok(combine_chunks)) return MOE_ERR_INVALID_ARG;
    ctx->pack_chunks = pack_chunks;
    ctx->combine_chunks = combine_chunks;
    return MOE_OK;
}

MOE_API moe_status moe_ctx_set_max_workgroups(moe_ctx* ctx, int32_t max_workgroups) {
    if (ctx == nullptr || max_workgroups < 0) return MOE_ERR_INVALID_ARG;
    ctx->max_blocks = max_workgroups;
    return MOE_OK;
}

// ---------------------------------------------------------------- hooks
struct moe_hook {
    hipEvent_t ev;
    int device;
};

MOE_API moe_status moe_hook_create(moe_hook** out) {
    if (out == nullptr) return MOE_ERR_INVALID_ARG;
    *out = nullptr;
    moe_hook* h = new (std::nothrow) moe_hook;
    if (h == nullptr) return MOE_ERR_HIP;
    if (hipGetDevice(&h->device) != hipSuccess ||
        hipEventCreateWithFlags(&h->ev, hipEventDisableTiming) != hipSuccess) {
        delete h;
        return MOE_ERR_HIP;
    }
    *out = h;
    return MOE_OK;
}

MOE_API moe_status moe_hook_destroy(moe_hook* hook) {
    if (hook == nullptr) return MOE_OK;
    const hipError_t e = hipEventDestroy(hook->ev);
    delete hook;
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

MOE_API moe_status moe_hook_record(moe_hook* hook, void* stream) {
    if (hook == nullptr) return MOE_ERR_INVALID_ARG;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != hook->device) return MOE_ERR_INVALID_ARG;
    return hipEventRecord(hook->ev, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

MOE_API moe_status moe_hook_wait(const moe_hook* hook, void* stream) {
    if (hook == nullptr) return MOE_ERR_INVALID_ARG;
    return hipStreamWaitEvent(reinterpret_cast<hipStream_t>(stream), hook->ev, 0) == hipSuccess ? MOE_OK
                                                                                                 : MOE_ERR_HIP;
}

namespace {

moe_status layout_call(moe_ctx* ctx, const int64_t* topk_idx, int32_t num_tokens, const void* x,
                       int32_t* num_tokens_per_expert, int32_t* num_tokens_per_rank, uint8_t* is_token_in_rank,
                       void* stream) {
    if (ctx == nullptr || !on_ctx_device(ctx)) return MOE_ERR_INVALID_ARG;
    if (num_tokens < 0) return MOE_ERR_INVALID_ARG;
    if (num_tokens > ctx->cfg.max_tokens) return MOE_ERR_CAPACITY;
    if (num_tokens > 0 && topk_idx == nullptr) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x)) return MOE_ERR_INVALID_ARG;
    int mode = -1;
    const moe_status st = run_layout(ctx_exec(ctx), topk_idx, num_tokens, num_tokens_per_expert,
                                     num_tokens_per_rank, is_token_in_rank, x, reinterpret_cast<hipStream_t>(stream),
                                     &mode);
    ctx->layout_valid = st == MOE_OK;
    ctx->layout_idx = topk_idx;
    ctx->layout_T = num_tokens;
    ctx->layout_mode = mode;
    return st;
}

}  // namespace

MOE_API moe_status moe_dispatch_layout(moe_ctx* ctx, const int64_t* topk_idx, int32_t num_tokens,
                                       int32_t* num_tokens_per_expert, int32_t* num_tokens_per_rank,
                                       uint8_t* is_token_in_rank, void* stream) {
    return layout_call(ctx, topk_idx, num_tokens, nullptr, num_tokens_per_expert, num_tokens_per_rank,
                       is_token_in_rank, stream);
}

MOE_API moe_status moe_dispatch_layout_prefetch(moe_ctx* ctx, const int64_t* topk_idx, int32_t num_tokens,
                                                const void* x, int32_t* num_tokens_per_expert,
                                                int32_t* num_tokens_per_rank, uint8_t* is_token_in_rank,
                                                void* stream) {
    return layout_call(ctx, topk_idx, num_tokens, x, num_tokens_per_expert, num_tokens_per_rank, is_token_in_rank,
                       stream);
}

MOE_API moe_status moe_dispatch(moe_ctx* ctx, const void* x, const int64_t* topk_idx, int32_t num_tokens,
                                int32_t reuse_layout, const moe_dispatch_buffers* bufs, moe_handle* handle,
                                void* stream) {
    if (ctx == nullptr || !on_ctx_device(ctx)) return MOE_ERR_INVALID_ARG;
    const moe_status st = check_dispatch_args(ctx->cfg, x, topk_idx, num_tokens, bufs, handle);
    if (st != MOE_OK) return st;
    if (reuse_layout != 0 && reuse_layout != 1) return MOE_ERR_INVALID_ARG;
    if (reuse_layout && (!ctx->layout_valid || ctx->layout_idx != topk_idx || ctx->layout_T != num_tokens))
        return MOE_ERR_INVALID_ARG;
    int computed = -1;
    const moe_status rs = run_dispatch(ctx_exec(ctx), x, topk_idx, num_tokens, reuse_layout ? ctx->layout_mode : -1,
                                       bufs, handle, ctx->tag, reinterpret_cast<hipStream_t>(stream), &computed);
    if (computed >= 0) {   // a layout computed inside this call is now the context's last one
        ctx->layout_valid = true;
        ctx->layout_idx = topk_idx;
        ctx->layout_T = num_tokens;
        ctx->layout_mode = computed;
    }
    return rs;
}

MOE_API moe_status moe_combine(moe_ctx* ctx, const void* expert_out, const float* topk_weights,
                               const moe_handle* handle, void* out, void* stream) {
    if (ctx == nullptr || handle == nullptr || !on_ctx_device(ctx)) return MOE_ERR_INVALID_ARG;
    const moe_config& c = ctx->cfg;
    if (handle->tag != ctx->tag || handle->num_tokens < 0 || handle->num_tokens > c.max_tokens ||
        handle->pos == nullptr)
        return MOE_ERR_HANDLE;
    const int32_t T = handle->num_tokens;
    if (T == 0) return MOE_OK;
    if (expert_out == nullptr || topk_weights == nullptr || out == nullptr) return MOE_ERR_INVALID_ARG;
    if (!aligned16(expert_out) || !aligned16(out)) return MOE_ERR_INVALID_ARG;
    CombineArgs a;
    a.y = static_cast<const uint16_t*>(expert_out);
    a.w = topk_weights;
    a.pos = handle->pos;
    a.out = static_cast<uint16_t*>(out);
    a.T = T;
    a.k = c.topk;
    a.H = c.hidden;
    a.rows_cap = ctx->g.recv_rows;
    a.err = ctx->err();
    int chunks, nslices;
    row_split(T, c.hidden / 8, ctx->combine_chunks, 2, &chunks, &nslices);
    a.nslices = nslices;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    TimedLaunch tl(ctx, s, MOE_KERNEL_COMBINE);
    hipError_t e = launch_combine(a, chunks, c.topk, ctx->max_blocks, s);
    tl.done();
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

MOE_API moe_status moe_dispatch_backward(moe_ctx* ctx, const void* grad_recv, const moe_handle* handle,
                                         void* grad_x, void* stream) {
    if (ctx == nullptr || handle == nullptr || !on_ctx_device(ctx)) return MOE_ERR_INVALID_ARG;
    const moe_config& c = ctx->cfg;
    if (handle->tag != ctx->tag || handle->num_tokens < 0 || handle->num_tokens > c.max_tokens ||
        handle->pos == nullptr)
        return MOE_ERR_HANDLE;
    const int32_t T = handle->num_tokens;
    if (T == 0) return MOE_OK;
    if (grad_recv == nullptr || grad_x == nullptr) return MOE_ERR_INVALID_ARG;
    if (!aligned16(grad_recv) || !aligned16(grad_x)) return MOE_ERR_INVALID_ARG;
    // the adjoint of the copy into the receive rows: combine with unit weights
    CombineArgs a;
    a.y = static_cast<const uint16_t*>(grad_recv);
    a.w = nullptr;
    a.pos = handle->pos;
    a.out = static_cast<uint16_t*>(grad_x);
    a.T = T;
    a.k = c.topk;
    a.H = c.hidden;
    a.rows_cap = ctx->g.recv_rows;
    a.err = ctx->err();
    int chunks, nslices;
    row_split(T, c.hidden / 8, ctx->combine_chunks, 2, &chunks, &nslices);
    a.nslices = nslices;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    TimedLaunch tl(ctx, s, MOE_KERNEL_DISPATCH_BWD);
    hipError_t e = launch_combine(a, chunks, c.topk, ctx->max_blocks, s);
    tl.done();
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

MOE_API moe_status moe_combine_backward(moe_ctx* ctx, const void* grad_out, const float* topk_weights,
                                        const void* expert_out, const moe_handle* handle,
                                        void* grad_expert_out, float* grad_weights, void* stream) {
    if (ctx == nullptr || handle == nullptr || !on_ctx_device(ctx)) return MOE_ERR_INVALID_ARG;
    const moe_config& c = ctx->cfg;
    if (handle->tag != ctx->tag || handle->num_tokens < 0 || handle->num_tokens > c.max_tokens ||
        handle->pos == nullptr)
        return MOE_ERR_HANDLE;
    const int32_t T = handle->num_tokens;
    if (T == 0) return MOE_OK;
    if (grad_out == nullptr || topk_weights == nullptr || expert_out == nullptr || grad_expert_out == nullptr ||
        grad_weights == nullptr)
        return MOE_ERR_INVALID_ARG;
    if (!aligned16(grad_out) || !aligned16(expert_out) || !aligned16(grad_expert_out)) return MOE_ERR_INVALID_ARG;
    CombineBwdArgs a;
    a.go = static_cast<const uint16_t*>(grad_out);
    a.w = topk_weights;
    a.y = static_cast<const uint16_t*>(expert_out);
    a.pos = handle->pos;
    a.gy = static_cast<uint16_t*>(grad_expert_out);
    a.gw = grad_weights;
    a.T = T;
    a.k = c.topk;
    a.H = c.hidden;
    a.rows_cap = ctx->g.recv_rows;
    a.err = ctx->err();
    // one block per token with one wavefront per slice: widen the slices until
    // they fit in one block
    int chunks, nslices;
    row_split(T, c.hidden / 8, ctx->combine_chunks, 1, &chunks, &nslices);
    if (ctx->combine_chunks == 0 && nslices > 8) {   // measured: at most 8 slices per token, else 2 chunks
        chunks = 2;
        nslices = (int)((c.hidden / 8 + 127) / 128);
    }
    while (nslices > bwd_max_waves(c.topk)) {
        chunks *= 2;
        nslices = (int)((c.hidden / 8 + 64 * chunks - 1) / (64 * chunks));
    }
    a.nslices = nslices;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    TimedLaunch tl(ctx, s, MOE_KERNEL_COMBINE_BWD);
    hipError_t e = launch_combine_bwd(a, chunks, c.topk, ctx->max_blocks, s);
    tl.done();
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

MOE_API moe_status moe_poll_error(moe_ctx* ctx, void* stream, uint32_t* flags) {
    if (ctx == nullptr || !on_ctx_device(ctx)) return MOE_ERR_INVALID_ARG;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint32_t v = 0;
    if (hipStreamSynchronize(s) != hipSuccess) return MOE_ERR_HIP;
    if (hipMemcpy(&v, ctx->err(), 4, hipMemcpyDeviceToHost) != hipSuccess) return MOE_ERR_HIP;
    if (v != 0 && hipMemset(ctx->err(), 0, 4) != hipSuccess) return MOE_ERR_HIP;
    if (hipDeviceSynchronize() != hipSuccess) return MOE_ERR_HIP;
    if (flags) *flags = v;
    return status_of_flags(v);
}

MOE_API moe_status moe_timing_begin(moe_ctx* ctx, int32_t max_launches) {
    if (ctx == nullptr || max_launches < 1 || ctx->timing) return MOE_ERR_INVALID_ARG;
    ctx->ev0.clear();
    ctx->ev1.clear();
    ctx->ev0.reserve(max_launches);
    ctx->ev1.reserve(max_launches);
    for (int i = 0; i < max_launches; ++i) {
        hipEvent_t a = nullptr, b = nullptr;
        if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) {
            // release what was created; the context stays without timing
            if (a != nullptr) (void)hipEventDestroy(a);
            for (hipEvent_t e : ctx->ev0) (void)hipEventDestroy(e);
            for (hipEvent_t e : ctx->ev1) (void)hipEventDestroy(e);
            ctx->ev0.clear();
            ctx->ev1.clear();
            return MOE_ERR_HIP;
        }
        ctx->ev0.push_back(a);
        ctx->ev1.push_back(b);
    }
    ctx->kid.clear();
    ctx->kid.reserve(max_launches);
    ctx->max_launches = max_launches;
    ctx->timing = true;
    return MOE_OK;
}

MOE_API moe_status moe_timing_launches(moe_ctx* ctx, int32_t* kernel_ids, float* ms, int32_t capacity,
                                       int32_t* count) {
    if (ctx == nullptr || !ctx->timing || count == nullptr || capacity < 0 ||
        (capacity > 0 && (kernel_ids == nullptr || ms == nullptr)))
        return MOE_ERR_INVALID_ARG;
    const int32_t n = (int32_t)ctx->kid.size();
    *count = n;
    for (int32_t i = 0; i < n && i < capacity; ++i) {
        float v = 0.f;
        if (hipEventSynchronize(ctx->ev1[i]) != hipSuccess ||
            hipEventElapsedTime(&v, ctx->ev0[i], ctx->ev1[i]) != hipSuccess)
            return MOE_ERR_HIP;
        kernel_ids[i] = ctx->kid[i];
        ms[i] = v;
    }
    return MOE_OK;
}

MOE_API moe_status moe_timing_end(moe_ctx* ctx, double* total_ms, int64_t* launches) {
    if (ctx == nullptr || !ctx->timing) return MOE_ERR_INVALID_ARG;
    moe_status st = MOE_OK;
    double tot[MOE_KERNEL_COUNT] = {};
    int64_t cnt[MOE_KERNEL_COUNT] = {};
    for (size_t i = 0; i < ctx->kid.size(); ++i) {
        float ms = 0.f;
        if (hipEventSynchronize(ctx->ev1[i]) != hipSuccess ||
            hipEventElapsedTime(&ms, ctx->ev0[i], ctx->ev1[i]) != hipSuccess) {
            st = MOE_ERR_HIP;
            break;
        }
        tot[ctx->kid[i]] += ms;
        cnt[ctx->kid[i]] += 1;
    }
    for (hipEvent_t e : ctx->ev0) (void)hipEventDestroy(e);
    for (hipEvent_t e : ctx->ev1) (void)hipEventDestroy(e);
    ctx->ev0.clear();
    ctx->ev1.clear();
    ctx->kid.clear();
    ctx->timing = false;
    for (int i = 0; i < MOE_KERNEL_COUNT; ++i) {
        if (total_ms) total_ms[i] = tot[i];
        if (launches) launches[i] = cnt[i];
    }
    return st;
}

// ============================================================== allocation-free dispatch
// Device scratch of moe_dispatch_noalloc: the layout workspace for callers
// that cannot allocate.  One copy per GPU, loaded with the code object and
// held until the process ends.  In host code `scratch` is only a stand-in for
// the symbol: its device address, per device, comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxScratchDevices];   // device address of `scratch` on each device, once looked up

// The current device's copy of the scratch: on the first call on a device,
// look up its address (with that device current) and zero its fixed header
// (error word, arrival counter, grand totals) with a kernel on `s`, ahead of
// the call's own launches; afterwards every layout leaves that header zero.
moe_status scratch_for_device(int dev, const Workspace& wl, hipStream_t s, char** out) {
    if (dev < 0 || dev >= kMaxScratchDevices) return MOE_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ERR_HIP;
        if (launch_zero_words(static_cast<uint32_t*>(p), (int64_t)(wl.off_cnt_e / 4), s) != hipSuccess)
            return MOE_ERR_HIP;
        g_scratch_ptr[dev] = static_cast<char*>(p);
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace

MOE_API moe_status moe_dispatch_noalloc(const moe_config* cfg, const void* x, const int64_t* topk_idx,
                                        int32_t num_tokens, const moe_dispatch_buffers* bufs, moe_handle* handle,
                                        uint32_t* error_word, void* stream) {
    Geometry g;
    moe_status st = check_config(cfg, &g);
    if (st != MOE_OK) return st;
    const Workspace wl = plan_workspace(cfg, g);
    if (wl.total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_CAPACITY;
    st = check_dispatch_args(*cfg, x, topk_idx, num_tokens, bufs, handle);
    if (st != MOE_OK) return st;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* ws = nullptr;
    st = scratch_for_device(dev, wl, s, &ws);
    if (st != MOE_OK) return st;
    Exec xc;
    xc.c = cfg;
    xc.g = &g;
    xc.wl = &wl;
    xc.ws = ws;
    xc.err = error_word != nullptr ? error_word : reinterpret_cast<uint32_t*>(ws + wl.off_err);
    xc.pack_chunks = 0;
    xc.max_blocks = 0;
    xc.ctx = nullptr;
    int computed = -1;
    return run_dispatch(xc, x, topk_idx, num_tokens, -1, bufs, handle, config_tag(cfg), s, &computed);
}
