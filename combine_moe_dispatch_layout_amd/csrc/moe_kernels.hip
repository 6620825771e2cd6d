// HIP kernels for MoE dispatch-layout / dispatch / combine on gfx950 (CDNA4).
//
// All three steps are bound by memory traffic, not arithmetic: layout reads
// topk_idx once, dispatch reads each token row once and writes it to every
// destination, combine reads every expert-output row once and writes each
// token row once.  Design points:
//  * Layout: one block per 256-token tile, 8 wavefronts of 32 tokens.  Stable
//    (token, slot) ranks come from per-expert lane masks built with LDS ORs
//    (the lanes holding one expert find each other) plus per-wavefront LDS
//    histograms -- no atomic decides any order, so results are deterministic.
//    The last tile block to arrive (device-scope counter) scans the tile
//    totals into global row bases (and, for large batches, turns the per-tile
//    counts into prefixes over the tiles), so count and scan are one launch;
//    each block arrives before writing its in-tile ranks, overlapping the two.
//  * Dispatch: one wavefront per (token, row slice).  The slice is loaded once
//    into registers with 16-byte loads, optionally quantised to E4M3 in
//    registers (block amax by cross-lane max over the 16 lanes holding one
//    128-channel block), then stored with 16-byte (8-byte for fp8) stores to
//    every destination row: up to min(k, R) send rows and k receive rows.
//    Destination row indices are wave-uniform (readlane -> SGPR), so the store
//    loop has no divergence.  Rows are written with non-temporal stores at
//    system scope (buffer stores, sc0 sc1 nt), one 16-byte chunk per lane per
//    work item: on MI355X non-temporal beats cached stores by 4% (prefill), 30%
//    (fp8 grouped) and 10% (skewed) on its own, and cached stores would push
//    ~0.9 GB per prefill launch through the 256 MB Infinity Cache, slowing a
//    concurrent bf16 GEMM by 1.3x (its operands are evicted); among the
//    non-temporal forms, system scope measured never slower and up to 3 us
//    faster per launch.
//  * Combine: one wavefront per (token, row slice); all k routed rows of the
//    slice are loaded before any arithmetic, accumulated in fp32 in slot order
//    with separately rounded multiply and add, rounded once to bf16 (RNE).  The
//    expert outputs are read exactly once, so they use non-temporal loads
//    (measured ~35% faster than cached loads here); short slices (2 chunks per
//    lane) keep many small wavefronts in flight.
//  * Fused low-latency dispatch (decode-sized batches, padded layout): one
//    launch computes the routing counts, the slot positions and the handle and
//    copies the rows; no grid-wide scan is needed because a padded slot's row
//    depends only on counts of earlier tokens.
//  * Backward: dispatch backward is the combine kernel with unit weights (the
//    adjoint of copying a token to k rows is adding those k rows back).  The
//    combine backward kernel has combine's shape: it reads the output gradient
//    and the k routed expert-output rows once, writes the weighted gradient to
//    each routed row, and reduces one dot product per slot for grad_w.
// There is no contraction to put on MFMA: the grad_w dot products are one
// multiply-add per loaded element (k of them per 16-byte gradient chunk).
#include "moe_internal.h"
#include "moe_ep.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint64_t lanes_below(int lane) { return (1ull << lane) - 1ull; }

// Lanes of the wavefront, among those with `active`, whose `key` equals this
// lane's key (one ballot per key bit).
__device__ __forceinline__ uint64_t match_any(int key, bool active, int bits) {
    uint64_t m = __ballot(active);
    for (int b = 0; b < bits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t on = __ballot(bit);
        m &= bit ? on : ~on;
    }
    return active ? m : 0ull;
}

__device__ __forceinline__ int readlane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }
__device__ __forceinline__ float readlane(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// binary32 -> bf16 bits, round to nearest even; NaN stays (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Sum of the first n entries of a 16-byte aligned int row (per-tile counts of
// one expert or rank), 16 entries (4 x 16-byte loads) in flight per step.
__device__ __forceinline__ int tile_prefix(const int32_t* row, int n) {
    typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
    const i32x4* v = reinterpret_cast<const i32x4*>(row);
    int s = 0;
    for (int q = 0; q < n; q += 16) {
        i32x4 x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = q + 4 * u < n ? v[(q >> 2) + u] : i32x4{0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int b = q + 4 * u;
            s += (b + 0 < n ? x[u].x : 0) + (b + 1 < n ? x[u].y : 0) + (b + 2 < n ? x[u].z : 0) +
                 (b + 3 < n ? x[u].w : 0);
        }
    }
    return s;
}

// ============================================================== layout
// floor(n / d) as (n * magic) >> 20 with magic = ceil(2^20 / d) = (2^20 + r) / d,
// r < d: exact while n * r < 2^20, which covers the two uses here (entry index
// n < 2^11 over k <= 32; expert id n < 2^10 over E/R <= 2^10; checked
// exhaustively on the host).
__device__ __forceinline__ int div_magic(int n, uint32_t magic) { return (int)(((uint32_t)n * magic) >> 20); }

// Inclusive sum over the 64 lanes of a wavefront.
__device__ __forceinline__ int wave_inclusive_sum(int v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_up(v, off, 64);
        if (lane >= off) v += u;
    }
    return v;
}

// Exclusive prefix sum of v[0..n) into out[0..n) for a block of NT threads,
// returns the total; all threads of the block must call it.  `wsum` is NT / 64
// ints of LDS scratch.
template <int NT = kBlockThreads>
__device__ __forceinline__ int block_exclusive_scan(const int32_t* v, int32_t* out, int n, int32_t* wsum) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    const int per = (n + NT - 1) / NT;
    const int lo = tid * per < n ? tid * per : n;
    const int hi = lo + per < n ? lo + per : n;
    int own = 0;
    for (int i = lo; i < hi; ++i) own += v[i];
    const int incl = wave_inclusive_sum(own, lane);
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int ww = 0; ww < NT / 64; ++ww) {
        const int s = wsum[ww];
        base += ww < w ? s : 0;
        total += s;
    }
    int run = base + incl - own;
    for (int i = lo; i < hi; ++i) {
        const int c = v[i];
        out[i] = run;
        run += c;
    }
    __syncthreads();
    return total;
}

// The layout's tile is 256 tokens; 8 wavefronts of 32 tokens each keep every
// wavefront's serial chain (one pass per 64-entry chunk) short.
constexpr int kLayoutWaves = 8;
constexpr int kLayoutThreads = 64 * kLayoutWaves;
constexpr int kWaveTokens = kTileTokens / kLayoutWaves;

template <int KMAX>
__global__ __launch_bounds__(kLayoutThreads) void k_layout(LayoutArgs a) {
    __shared__ unsigned long long peer_mask[kLayoutWaves * MOE_MAX_EXPERTS];  // per chunk: lanes holding e
    __shared__ unsigned long long rank_toks[kLayoutWaves * MOE_MAX_RANKS];    // tokens of the wave sent to r
    __shared__ unsigned long long tok_mask[kTileTokens];                       // ranks each token is sent to
    __shared__ int32_t hist_e[kLayoutWaves * MOE_MAX_EXPERTS];
    __shared__ int32_t hist_r[kLayoutWaves * MOE_MAX_RANKS];
    __shared__ int32_t tot[MOE_MAX_EXPERTS + MOE_MAX_RANKS];
    __shared__ int32_t off[MOE_MAX_EXPERTS + MOE_MAX_RANKS];
    __shared__ int32_t wsum[kLayoutWaves];
    __shared__ int s_last;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    const int E = a.E, R = a.R, k = a.k;
    const int ntiles = a.ntiles;
    if ((int)blockIdx.x >= ntiles) {
        // ---- the layout occupies a few compute units for several microseconds
        // of dependent latencies while HBM sits idle: the other workgroups read
        // the token rows the dispatch will read next, so that they come from
        // the Infinity Cache then instead of HBM.  Cached loads (they allocate
        // in the caches); the bits are folded into one word that is stored
        // only if it hits one value, so that the loads are kept.
        const u32x4* p = static_cast<const u32x4*>(a.warm);
        const int64_t stride = (int64_t)(gridDim.x - ntiles) * kLayoutThreads;
        uint32_t acc = 0u;
        for (int64_t i = (int64_t)(blockIdx.x - ntiles) * kLayoutThreads + tid; i < a.warm_chunks; i += 8 * stride) {
            u32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = i + u * stride < a.warm_chunks ? p[i + u * stride] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].w;
        }
        if (acc == 0x9e3779b9u) *a.warm_sink = acc;
        return;
    }
    const int64_t tok0 = (int64_t)blockIdx.x * kTileTokens + w * kWaveTokens;   // this wave's first token
    const int64_t t = tok0 + lane;          // lane = token of the wave (lanes < kWaveTokens)
    const bool tok_ok = lane < kWaveTokens && t < a.T;
    const int64_t ntok = a.T - tok0 < 0 ? 0 : (a.T - tok0 > kWaveTokens ? kWaveTokens : a.T - tok0);
    const int64_t nent = ntok * k;          // (token, slot) entries of this wave, row-major
    const int nch = (kWaveTokens * k + 63) / 64;   // 64-entry chunks of a full wave
    const int64_t ent0 = tok0 * k;
    const uint64_t below = lanes_below(lane);

    // ---- all loads of this wave's entries first, in flight together (nothing
    // with a side effect between them), then the LDS is cleared meanwhile
    int64_t raw[KMAX];
#pragma unroll
    for (int c = 0; c < KMAX; ++c) {
        const int64_t i = (int64_t)c * 64 + lane;
        raw[c] = c < nch && i < nent ? a.topk_idx[ent0 + i] : -1;
    }
    for (int i = tid; i < kLayoutWaves * E; i += kLayoutThreads) {
        peer_mask[i] = 0ull;
        hist_e[i] = 0;
    }
    for (int i = tid; i < kLayoutWaves * R; i += kLayoutThreads) rank_toks[i] = 0ull;
    if (tid < kTileTokens) tok_mask[tid] = 0ull;
    int ev[KMAX];
    bool bad = false;
#pragma unroll
    for (int c = 0; c < KMAX; ++c) {
        const int64_t v = raw[c];
        const bool ok = v >= 0 && v < E;
        bad |= !ok && v != -1;
        ev[c] = ok ? (int)v : -1;
    }
    if (bad) atomicOr(a.err, kErrBadTopk);
    __syncthreads();

    // ---- phase 1: for every 64-entry chunk (row-major order), the lanes holding
    // the same expert find each other through one LDS bitmask; an entry's rank
    // inside this wavefront = rows of its expert in earlier chunks + earlier
    // lanes of its chunk.  Rank sets are OR-ed into per-rank token masks.
    int erl[KMAX];
#pragma unroll
    for (int c = 0; c < KMAX; ++c) {
        erl[c] = 0;
        if (c < nch) {
            const int e = ev[c];
            unsigned long long* pm = &peer_mask[w * E + (e >= 0 ? e : 0)];
            if (e >= 0) {
                const int tl = div_magic(c * 64 + lane, a.k_magic);   // token within the wave
                const int r = div_magic(e, a.el_magic);
                atomicOr(pm, 1ull << lane);
                atomicOr(&rank_toks[w * R + r], 1ull << tl);
                atomicOr(&tok_mask[w * kWaveTokens + tl], 1ull << r);
            }
            __builtin_amdgcn_wave_barrier();
            if (e >= 0) {
                const uint64_t peers = *pm;
                const int before = hist_e[w * E + e];
                erl[c] = before + __popcll(peers & below);
                __builtin_amdgcn_wave_barrier();
                if ((peers & below) == 0) {       // lowest lane of the group
                    hist_e[w * E + e] = before + __popcll(peers);
                    *pm = 0ull;
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
    __syncthreads();

    // ---- per-wavefront rank counts; exclusive prefixes over the wavefronts;
    // tile totals: kept in LDS for a single tile; up to kWalkTiles tiles
    // published column by column for the dispatch kernel to sum, plus atomic
    // grand totals for the last block; beyond, published tile by tile with
    // device-scope exchanges for the last block to read back
    for (int i = tid; i < kLayoutWaves * R; i += kLayoutThreads) hist_r[i] = __popcll(rank_toks[i]);
    __syncthreads();
    const int mode = a.mode;   // matches the grid (chosen on the host from the tile count)
    int seen = 0;   // returned values: using them makes the atomics complete before the arrival below
    for (int col = tid; col < E + R; col += kLayoutThreads) {
        const bool is_e = col < E;
        int32_t* h = is_e ? hist_e + col : hist_r + (col - E);
        const int stride = is_e ? E : R;
        int run = 0;
#pragma unroll
        for (int ww = 0; ww < kLayoutWaves; ++ww) {
            const int c = h[ww * stride];
            h[ww * stride] = run;
            run += c;
        }
        if (mode == kLayoutOneTile) {
            tot[col] = run;
        } else if (mode == kLayoutWalk) {
            a.tile_cnt[(int64_t)col * a.tile_stride + blockIdx.x] = run;
            if (run != 0) seen |= atomicAdd(&a.grand_tot[col], run);
        } else {
            seen |= __hip_atomic_exchange(&a.tile_cnt[(int64_t)blockIdx.x * a.cnt_stride + col], run,
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (seen == -1) s_last = 2;   // never true (counts are >= 0): consumes the returned values before the arrival
    __syncthreads();
    // ---- arrival (see below), issued now so that its round trip overlaps phase 2
    unsigned arrived = 0u;
    if (mode != kLayoutOneTile && tid == 0) arrived = atomicAdd(a.done, 1u);

    // ---- phase 2: tile-local ranks out, each with its expert id (every entry,
    // empty ones too, so that a dispatch reusing the layout can check them)
#pragma unroll
    for (int c = 0; c < KMAX; ++c) {
        const int64_t i = (int64_t)c * 64 + lane;
        if (c < nch && i < nent)
            a.erank[ent0 + i] = erank_pack(ev[c], ev[c] >= 0 ? hist_e[w * E + ev[c]] + erl[c] : 0);
    }
    const uint64_t rmask = lane < kWaveTokens ? tok_mask[w * kWaveTokens + lane] : 0ull;   // 0 past T
    if (tok_ok) {
        for (uint64_t m = rmask; m != 0; m &= m - 1) {
            const int r = __ffsll((unsigned long long)m) - 1;
            const int rk = hist_r[w * R + r] + __popcll(rank_toks[w * R + r] & below);
            a.srank[(int64_t)r * a.max_tokens + t] = (uint16_t)rk;
        }
        if (a.out_in_rank != nullptr) {
            if (a.in_rank_vec4) {   // 4 flags per 32-bit store (aligned, R % 4 == 0)
                uint32_t* dst = reinterpret_cast<uint32_t*>(a.out_in_rank + t * R);
                for (int r = 0; r < R; r += 4) {
                    const uint32_t b = (uint32_t)(rmask >> r);
                    dst[r >> 2] = (b & 1u) | ((b & 2u) << 7) | ((b & 4u) << 14) | ((b & 8u) << 21);
                }
            } else {
                for (int r = 0; r < R; ++r) a.out_in_rank[t * R + r] = (uint8_t)((rmask >> r) & 1);
            }
        }
    }

    // ---- arrival: the last block reads (and resets) the grand totals, or
    // (beyond kWalkTiles tiles) sums every column's per-tile counts into its
    // total and rewrites them in place as exclusive prefixes over the tiles --
    // one thread per column, consecutive columns in a wavefront's lanes, so
    // each load and store covers a contiguous stretch of one tile's row; a
    // batch of loads is issued before any is used.  Only device-scope atomics
    // cross blocks here (the totals or counts, read back with atomic loads, and
    // the arrival counter); each block's atomics have completed (their returned
    // values were consumed before the barrier ahead of its arrival), so no
    // memory fence is needed -- on this chip a device-scope release fence
    // writes back the whole L2.
    if (mode != kLayoutOneTile) {
        if (tid == 0) s_last = (arrived == (unsigned)ntiles - 1);
        __syncthreads();
        if (!s_last) return;
        if (mode == kLayoutWalk) {
            for (int col = tid; col < E + R; col += kLayoutThreads) {
                tot[col] = __hip_atomic_load(&a.grand_tot[col], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                a.grand_tot[col] = 0;
            }
        } else {
            constexpr int kBatch = 32;
            for (int col = tid; col < E + R; col += kLayoutThreads) {
                int32_t* p = a.tile_cnt + col;
                int run = 0;
                for (int t0 = 0; t0 < ntiles; t0 += kBatch) {
                    int32_t c[kBatch];
#pragma unroll
                    for (int u = 0; u < kBatch; ++u)
                        c[u] = t0 + u < ntiles ? __hip_atomic_load(p + (int64_t)(t0 + u) * a.cnt_stride,
                                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                               : 0;
#pragma unroll
                    for (int u = 0; u < kBatch; ++u) {
                        if (t0 + u < ntiles) p[(int64_t)(t0 + u) * a.cnt_stride] = run;
                        run += c[u];
                    }
                }
                tot[col] = run;
            }
        }
        __syncthreads();
    }

    // offsets: one exclusive scan over the expert counts followed by the rank
    // counts; the rank offsets are the second part minus the expert total
    const int total = block_exclusive_scan<kLayoutThreads>(tot, off, E + R, wsum);
    const int total_e = off[E];
    const int total_r = total - total_e;
    for (int e = tid; e < E; e += kLayoutThreads) {
        a.eoff[e] = off[e];
        a.cnt_e[e] = tot[e];
        if (a.out_cnt_e != nullptr) a.out_cnt_e[e] = tot[e];
    }
    for (int r = tid; r < R; r += kLayoutThreads) {
        a.roff[r] = off[E + r] - total_e;
        a.cnt_r[r] = tot[E + r];
        if (a.out_cnt_r != nullptr) a.out_cnt_r[r] = tot[E + r];
    }
    if (tid == 0) {
        a.eoff[E] = total_e;
        a.roff[R] = total_r;
        if (mode != kLayoutOneTile) *a.done = 0u;
    }
}

// Chunk i of a wavefront's slice starts at 16-byte chunk gi = gbase + 64 i.
// Whole iterations (gi + 64 <= nchunk) need no per-lane guard: the test is
// wave-uniform, so the stores are issued unmasked; only a ragged last
// iteration masks lanes.
enum ChunkState { kChunkFull, kChunkPart, kChunkNone };
__device__ __forceinline__ ChunkState chunk_state(int64_t gi, int64_t nchunk) {
    return gi + 64 <= nchunk ? kChunkFull : (gi < nchunk ? kChunkPart : kChunkNone);
}

// ============================================================== dispatch
// Cache policy of the dispatch's row stores (the cache-policy operand of the
// gfx950 buffer store: bit 0 sc0, bit 1 nt, bit 4 sc1): non-temporal at
// system scope (sc0 sc1 nt).  Measured on MI355X against plain non-temporal
// stores (dispatch, after a 1 GiB write flush): prefill 180 -> 176 us, skewed
// 118 -> 115 us, grouped fp8 81 -> 80 us, and the decode step 10.65 -> 9.8 us
// graph-replayed.  System scope without nt makes the rows allocate in the Infinity Cache:
// prefill 171 us, but skewed 124 us and grouped fp8 98 us, so nt stays.
constexpr int kStoreRows = 0x13;   // sc0 sc1 nt

// Store a slice (C chunks per lane) of one row of nchunk chunks: buffer stores
// over the row (a chunk past its end falls out of the buffer and is dropped by
// the hardware).
template <int C, typename V>
__device__ __forceinline__ void store_row(V* dst, const V* v, int64_t gbase, int lane, int64_t nchunk) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(dst, 0, (int)(nchunk * sizeof(V)), 0x00020000);
#pragma unroll
    for (int i = 0; i < C; ++i) {
        const int64_t gi = gbase + i * 64;
        if (chunk_state(gi, nchunk) == kChunkNone) continue;
        const int off = (int)((gi + lane) * sizeof(V));
        if constexpr (sizeof(V) == 16) __builtin_amdgcn_raw_buffer_store_b128(v[i], r, off, 0, kStoreRows);
        else __builtin_amdgcn_raw_buffer_store_b64(v[i], r, off, 0, kStoreRows);
    }
}

// Per-block scales of a slice: the first lane of each 16-lane block group.
template <int C>
__device__ __forceinline__ void store_scales(float* sdst, const float* sinv, int64_t g0, int lane, int64_t nchunk) {
    if ((lane & 15) == 0) {
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const int64_t g = g0 + i * 64;
            if (g < nchunk) sdst[g >> 4] = sinv[i];
        }
    }
}

// Max over each 16-lane row of the wavefront with DPP lane permutations
// (quad xor 1, quad xor 2, mirror within 8, mirror within 16); inputs are
// non-negative, so every lane ends with its row's maximum.
__device__ __forceinline__ float dpp_f(float v, int ctrl_sel) {
    const int x = __float_as_int(v);
    int y;
    switch (ctrl_sel) {
        case 0: y = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false); break;   // quad_perm [1,0,3,2]
        case 1: y = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false); break;   // quad_perm [2,3,0,1]
        case 2: y = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false); break;  // row_half_mirror
        default: y = __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false); break; // row_mirror
    }
    return __int_as_float(y);
}
__device__ __forceinline__ float row16_max(float m) {
    m = fmaxf(m, dpp_f(m, 0));
    m = fmaxf(m, dpp_f(m, 1));
    m = fmaxf(m, dpp_f(m, 2));
    m = fmaxf(m, dpp_f(m, 3));
    return m;
}

// E4M3 quantisation of a slice held in registers (C 16-byte bf16 chunks per
// lane): the 16 lanes holding one 128-channel block reduce |x| with a DPP
// row max; scale 448/a' and stored dequant scale a'/448 are correctly
// rounded binary32 divisions (a' = max(amax, 1e-4)); codes come from
// v_cvt_pk_fp8_f32 (OCP E4M3 on gfx950, round to nearest even).
template <int C>
__device__ __forceinline__ void quantize_slice(const u32x4* v, u32x2* q, float* sinv) {
#pragma unroll
    for (int i = 0; i < C; ++i) {
        float f[8] = {bf16_lo(v[i].x), bf16_hi(v[i].x), bf16_lo(v[i].y), bf16_hi(v[i].y),
                      bf16_lo(v[i].z), bf16_hi(v[i].z), bf16_lo(v[i].w), bf16_hi(v[i].w)};
        float m = 0.0f;
#pragma unroll
        for (int u = 0; u < 8; ++u) m = fmaxf(m, fabsf(f[u]));
        m = row16_max(m);
        const float ap = m > 1e-4f ? m : 1e-4f;
        const float sc = 448.0f / ap;
        sinv[i] = ap / 448.0f;
        int lo = 0, hi = 0;
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(__fmul_rn(f[0], sc), __fmul_rn(f[1], sc), lo, false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(__fmul_rn(f[2], sc), __fmul_rn(f[3], sc), lo, true);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(__fmul_rn(f[4], sc), __fmul_rn(f[5], sc), hi, false);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(__fmul_rn(f[6], sc), __fmul_rn(f[7], sc), hi, true);
        q[i] = u32x2{(uint32_t)lo, (uint32_t)hi};
    }
}

// Whether any bf16 value of a slice (C 16-byte chunks per lane) is Inf or NaN
// (exponent bits all ones); the E4M3 codes of such a block are unspecified.
template <int C>
__device__ __forceinline__ bool slice_nonfinite(const u32x4* v) {
    uint32_t bad = 0u;
#pragma unroll
    for (int i = 0; i < C; ++i) {
        const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            bad |= (w[u] & 0x7f80u) == 0x7f80u;
            bad |= (w[u] & 0x7f800000u) == 0x7f800000u;
        }
    }
    return bad != 0u;
}

// One (token, row slice) work item of the dispatch, done by one wavefront.
template <int C, bool FP8, bool LL, bool SEND>
__device__ __forceinline__ void pack_item(const PackArgs& a, int64_t item, int lane) {
    const int t = (int)(item / a.nslices);
    const int s = (int)(item - (int64_t)t * a.nslices);
    const int k = a.k;
    const uint64_t below = lanes_below(lane);

    // ---- load this slice of the row once (issued before the routing lookups,
    // which it does not depend on)
    const int64_t nchunk = a.H / 8;                   // 16-byte bf16 chunks per row
    const int64_t gbase = (int64_t)s * 64 * C;        // first chunk of this slice
    const int64_t g0 = gbase + lane;
    const u32x4* src = reinterpret_cast<const u32x4*>(a.x + (int64_t)t * a.H);
    u32x4 v[C];
#pragma unroll
    for (int i = 0; i < C; ++i) {
        const int64_t g = g0 + i * 64;
        const ChunkState cs = chunk_state(gbase + i * 64, nchunk);
        v[i] = u32x4{0u, 0u, 0u, 0u};
        if (cs == kChunkFull || (cs == kChunkPart && g < nchunk)) v[i] = src[g];
    }

    // ---- routing of token t: lane j < k owns slot j; with it the layout's
    // record of the slot (its expert id and in-tile rank)
    int e = -1;
    uint32_t er = erank_pack(-1, 0);
    if (lane < k) {
        const int64_t v = a.topk_idx[(int64_t)t * k + lane];
        er = a.erank[(int64_t)t * k + lane];
        if (v >= 0 && v < a.E) e = (int)v;
    }
    // a layout made from other routing (topk_idx rewritten in place before a
    // dispatch that reuses it): the token is dropped and the error recorded
    if (__ballot(lane < k && (er >> 16) != (erank_pack(e, 0) >> 16)) != 0) {
        if (s == 0 && lane == 0) atomicOr(a.err, kErrStale);
        e = -1;
    }
    const int tile = t / kTileTokens;
    const int r = e >= 0 ? e / a.El : 0;
    const uint64_t peers = match_any(r, e >= 0, a.rbits);
    const bool first_of_rank = e >= 0 && (peers & below) == 0;
    // rows of this expert (and tokens of this rank) in earlier tiles: the sum
    // of their per-tile counts, or beyond kWalkTiles tiles the layout kernel's
    // prefix over the tiles
    int pre_e = 0, pre_r = 0;
    if (e >= 0 && tile > 0 && a.mode != kLayoutOneTile) {
        if (a.mode == kLayoutWalk) {
            pre_e = tile_prefix(a.tile_cnt + (int64_t)e * a.tile_stride, tile);
            if (SEND && first_of_rank) pre_r = tile_prefix(a.tile_cnt + (int64_t)(a.E + r) * a.tile_stride, tile);
        } else {
            pre_e = a.tile_cnt[(int64_t)tile * a.cnt_stride + e];
            if (SEND && first_of_rank) pre_r = a.tile_cnt[(int64_t)tile * a.cnt_stride + a.E + r];
        }
    }
    int cpos = -1;   // contiguous expert-major row (index into recv_src_idx)
    int rrow = -1;   // receive row (contiguous, or padded low-latency slot)
    if (e >= 0) {
        const int in_expert = pre_e + (int)(er & 0xFFFFu);   // rank among expert e's rows
        cpos = a.eoff[e] + in_expert;
        int64_t row = cpos;
        if (LL) row = (int64_t)e * a.cap + (int64_t)a.s0 * a.max_tokens + in_expert;
        if (cpos < 0 || cpos >= a.pairs_cap) {
            atomicOr(a.err, kErrBounds);
            cpos = -1;
        } else if (LL && in_expert >= a.max_tokens) {
            // past this source's window of the expert (possible only when a
            // token repeats an expert): the row is not placed
            atomicOr(a.err, kErrCapacity);
        } else if (row < 0 || row >= a.recv_cap_rows) {
            atomicOr(a.err, kErrBounds);
        } else {
            rrow = (int)row;
        }
    }
    int srow = -1;   // send row: only for the first slot of each destination rank
    if (SEND && first_of_rank) {
        const int64_t row = (int64_t)a.roff[r] + pre_r + a.srank[(int64_t)r * a.max_tokens + t];
        if (row < 0 || row >= a.send_cap_rows) atomicOr(a.err, kErrBounds);
        else srow = (int)row;
    }
    if (s == 0 && lane < k) {
        a.h_pos[(int64_t)t * k + lane] = rrow;
        if (cpos >= 0) a.h_recv_src[cpos] = t;
        if (srow >= 0) a.h_send_src[srow] = t;
    }


    if constexpr (!FP8) {
        for (int j = 0; j < k; ++j) {
            const int rr = readlane(rrow, j);
            if (rr >= 0) store_row<C>(reinterpret_cast<u32x4*>(a.recv_rows) + (int64_t)rr * nchunk, v, gbase, lane, nchunk);
            if constexpr (SEND) {
                const int sr = readlane(srow, j);
                if (sr >= 0) store_row<C>(reinterpret_cast<u32x4*>(a.send_rows) + (int64_t)sr * nchunk, v, gbase, lane, nchunk);
            }
        }
    } else {
        // ---- E4M3 quantisation, once per token; 16 lanes hold one 128-channel block
        if (__ballot(slice_nonfinite<C>(v)) != 0 && lane == 0) atomicOr(a.err, kErrNonFinite);
        u32x2 q[C];
        float sinv[C];
        quantize_slice<C>(v, q, sinv);
        const int nb = a.H / 128;
        for (int j = 0; j < k; ++j) {
            const int rr = readlane(rrow, j);
            if (rr >= 0) {
                store_row<C>(reinterpret_cast<u32x2*>(a.recv_rows) + (int64_t)rr * nchunk, q, gbase, lane, nchunk);
                store_scales<C>(a.recv_scales + (int64_t)rr * nb, sinv, g0, lane, nchunk);
            }
            if constexpr (SEND) {
                const int sr = readlane(srow, j);
                if (sr >= 0) {
                    store_row<C>(reinterpret_cast<u32x2*>(a.send_rows) + (int64_t)sr * nchunk, q, gbase, lane, nchunk);
                    store_scales<C>(a.send_scales + (int64_t)sr * nb, sinv, g0, lane, nchunk);
                }
            }
        }
    }
}

// Grid-stride over the work items, so that the grid can be capped (a cap on
// the workgroups the dispatch occupies) without changing any result.
template <int C, bool FP8, bool LL, bool SEND>
__global__ __launch_bounds__(kBlockThreads) void k_pack(PackArgs a) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    if (blockIdx.x == 0) {   // handle copies of the layout offsets and counts
        for (int i = tid; i <= a.E; i += kBlockThreads) a.h_eoff[i] = a.eoff[i];
        for (int i = tid; i < a.E; i += kBlockThreads) a.h_recv_counts[i] = a.cnt_e[i];
        for (int i = tid; i <= a.R; i += kBlockThreads) a.h_roff[i] = a.roff[i];
    }
    const int64_t total = (int64_t)a.T * a.nslices;
    const int64_t stride = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + w; item < total; item += stride)
        pack_item<C, FP8, LL, SEND>(a, item, lane);
}

// ============================================================== fused low-latency dispatch
// In the padded low-latency layout a slot's row is e * cap + s0 * M + (its
// rank among the rows of expert e), so no global scan stands between the
// routing and the copy: one launch does both.  Grid = 1 + T * B blocks.
//  * Blocks 1..T*B: B consecutive blocks per token, one 16-byte chunk per lane;
//    each wavefront copies one 64-chunk slice of the row.  Rows of up to 256
//    chunks take one 256-thread block; longer rows take 512-thread blocks, B
//    of them (a 7168-wide row: 14 slices, B = 2), which spreads the stores of
//    a 128-token batch over all compute units (measured on MI355X: 6.65 ->
//    6.28 us per launch against one 1024-thread block per token; 256-thread
//    blocks, B = 4, are slower, 7.8 us).  Every block counts the routing for
//    its token (cheap); only the first writes the handle entries.  A slot of
//    expert e needs two counts over the T * k routing entries: entries of e
//    in earlier tokens (its rank, plus earlier slots of its own token with the
//    same expert) and valid entries with a smaller expert id (its expert-major
//    position, for the handle's recv_src_idx).  Each wavefront counts its share of the
//    entries against the token's k experts with ballots; one barrier and a
//    sum over the wavefronts give both counts (integer sums: order-free).
//  * Block 0: the handle's summary -- per-expert counts (an LDS histogram of
//    all entries), their exclusive scan, tokens per rank and its scan -- and
//    the bad-id flag.
// For T * k <= kFusedMaxEntries and T <= kFusedMaxTokens.
template <int NT>
__device__ __forceinline__ void ll_summary(const PackArgs& a) {
    __shared__ int32_t tot[MOE_MAX_EXPERTS + MOE_MAX_RANKS];   // entries per expert, then tokens per rank
    __shared__ int32_t off[MOE_MAX_EXPERTS + MOE_MAX_RANKS];   // exclusive scans of tot
    __shared__ unsigned long long tok_mask[kFusedMaxTokens];    // ranks of each token
    __shared__ int32_t wsum[NT / 64];
    constexpr int kPerThread = kFusedMaxEntries / NT;
    const int tid = threadIdx.x;
    const int k = a.k, E = a.E, R = a.R, T = a.T;
    const int nent = T * k;
    int64_t ent[kPerThread];
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
        const int i = u * NT + tid;
        ent[u] = i < nent ? a.topk_idx[i] : -1;
    }
    for (int i = tid; i < E + R; i += NT) tot[i] = 0;
    for (int i = tid; i < T; i += NT) tok_mask[i] = 0ull;
    __syncthreads();
    bool bad = false;
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
        const int i = u * NT + tid;
        const int64_t ee = ent[u];
        if (ee >= 0 && ee < E) {
            atomicAdd(&tot[(int)ee], 1);
            atomicOr(&tok_mask[i / k], 1ull << ((int)ee / a.El));
        } else if (i < nent && ee != -1) {
            bad = true;
        }
    }
    if (bad) atomicOr(a.err, kErrBadTopk);
    __syncthreads();
    for (int i = tid; i < T; i += NT)
        for (uint64_t m = tok_mask[i]; m != 0; m &= m - 1) atomicAdd(&tot[E + __ffsll((unsigned long long)m) - 1], 1);
    __syncthreads();
    const int total_e = block_exclusive_scan<NT>(tot, off, E, wsum);
    const int total_r = block_exclusive_scan<NT>(tot + E, off + E, R, wsum);
    for (int ee = tid; ee < E; ee += NT) {
        a.h_eoff[ee] = off[ee];
        a.h_recv_counts[ee] = tot[ee];
    }
    for (int r = tid; r < R; r += NT) a.h_roff[r] = off[E + r];
    if (tid == 0) {
        a.h_eoff[E] = total_e;
        a.h_roff[R] = total_r;
    }
}

template <int C, bool FP8, int NT>
__global__ __launch_bounds__(NT) void k_ll_dispatch(PackArgs a) {
    if (blockIdx.x == 0) {
        ll_summary<NT>(a);
        return;
    }
    __shared__ int32_t cnt_hb[NT / 64][MOE_MAX_TOPK];    // per wavefront: entries of e_j in earlier tokens
    __shared__ int32_t cnt_lt[NT / 64][MOE_MAX_TOPK];    // per wavefront: valid entries with id < e_j
    constexpr int kPerThread = kFusedMaxEntries / NT;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int k = a.k, E = a.E;
    const int nent = a.T * k;
    const int t = (blockIdx.x - 1) / a.ll_bpt;                            // this block's token
    const int s = (blockIdx.x - 1 - t * a.ll_bpt) * (NT / 64) + w;        // this wavefront's row slice
    const bool has_slice = s < a.nslices;
    const int before = t * k;                 // entries of earlier tokens

    // ---- row slice, the token's own slots and the routing entries: all loads first
    const int64_t nchunk = a.H / 8;
    const int64_t gbase = (int64_t)s * 64 * C;
    const int64_t g0 = gbase + lane;
    u32x4 v[C];
    if (has_slice) {
        const u32x4* src = reinterpret_cast<const u32x4*>(a.x + (int64_t)t * a.H);
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const int64_t g = g0 + i * 64;
            const ChunkState cs = chunk_state(gbase + i * 64, nchunk);
            v[i] = u32x4{0u, 0u, 0u, 0u};
            if (cs == kChunkFull || (cs == kChunkPart && g < nchunk)) v[i] = src[g];
        }
    }
    int64_t mine = -1;
    if (lane < k) mine = a.topk_idx[(int64_t)before + lane];
    int64_t ent[kPerThread];
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
        const int i = u * NT + tid;
        ent[u] = i < nent ? a.topk_idx[i] : -1;
    }
    const int e = mine >= 0 && mine < E ? (int)mine : -1;   // lane j < k: expert of slot j

    // ---- this wavefront's share of the two counts, for every slot of the token
    // (entry group u holds entries u * NT .. u * NT + NT - 1: groups at or past
    // T * k hold none, groups at or past this token's first entry none of the
    // earlier ones -- both limits are uniform, so those ballots are skipped)
    for (int j = 0; j < k; ++j) {
        const int ej = readlane(e, j);
        if (ej < 0) continue;
        int c_hb = 0, c_lt = 0;
#pragma unroll
        for (int u = 0; u < kPerThread; ++u) {
            if (u * NT >= nent) break;
            const int i = u * NT + tid;
            if (u * NT < before) c_hb += __popcll(__ballot(ent[u] == ej && i < before));
            c_lt += __popcll(__ballot(ent[u] >= 0 && ent[u] < ej));
        }
        if (lane == 0) {
            cnt_hb[w][j] = c_hb;
            cnt_lt[w][j] = c_lt;
        }
    }
    __syncthreads();
    if (!has_slice) return;

    // ---- slot j (lane j): rank among the rows of its expert and expert-major position
    int rank = 0, lessv = 0;
    if (lane < k && e >= 0) {
#pragma unroll
        for (int q = 0; q < NT / 64; ++q) {
            rank += cnt_hb[q][lane];
            lessv += cnt_lt[q][lane];
        }
    }
    for (int j = 0; j < k; ++j) {             // earlier slots of this token with the same expert
        const int ej = readlane(e, j);
        rank += (j < lane && ej == e && e >= 0) ? 1 : 0;
    }
    int rrow = -1;
    if (e >= 0) {
        const int64_t row = (int64_t)e * a.cap + (int64_t)a.s0 * a.max_tokens + rank;
        if (rank >= a.max_tokens) {
            // past this source's window of the expert (only when a token repeats
            // an expert): the row is not placed
            if (s == 0) atomicOr(a.err, kErrCapacity);
        } else if (row >= a.recv_cap_rows) {
            atomicOr(a.err, kErrBounds);
        } else {
            rrow = (int)row;
        }
    }
    if (s == 0 && lane < k) {
        a.h_pos[(int64_t)t * k + lane] = rrow;
        const int64_t cp = (int64_t)lessv + rank;   // expert-major position
        if (e >= 0 && cp < a.pairs_cap) a.h_recv_src[cp] = t;
    }

    // ---- copy (and quantise) the slice into the token's slots
    if constexpr (!FP8) {
        for (int j = 0; j < k; ++j) {
            const int rr = readlane(rrow, j);
            if (rr >= 0) store_row<C>(reinterpret_cast<u32x4*>(a.recv_rows) + (int64_t)rr * nchunk, v, gbase, lane, nchunk);
        }
    } else {
        if (__ballot(slice_nonfinite<C>(v)) != 0 && lane == 0) atomicOr(a.err, kErrNonFinite);
        u32x2 q[C];
        float sinv[C];
        quantize_slice<C>(v, q, sinv);
        const int nbk = a.H / 128;
        for (int j = 0; j < k; ++j) {
            const int rr = readlane(rrow, j);
            if (rr >= 0) {
                store_row<C>(reinterpret_cast<u32x2*>(a.recv_rows) + (int64_t)rr * nchunk, q, gbase, lane, nchunk);
                store_scales<C>(a.recv_scales + (int64_t)rr * nbk, sinv, g0, lane, nchunk);
            }
        }
    }
}

// ============================================================== combine
// One output chunk (8 channels) from the KMAX row chunks in v: fp32 from +0,
// w_j * y_j rounded, then added, slot by slot in ascending order; bf16 RNE.
template <int KMAX>
__device__ __forceinline__ u32x4 combine_chunk(const u32x4 (&v)[KMAX], const int* pj, const float* wj) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        if (pj[j] >= 0) {
            const float wv = wj[j];
            acc[0] = __fadd_rn(acc[0], __fmul_rn(wv, bf16_lo(v[j].x)));
            acc[1] = __fadd_rn(acc[1], __fmul_rn(wv, bf16_hi(v[j].x)));
            acc[2] = __fadd_rn(acc[2], __fmul_rn(wv, bf16_lo(v[j].y)));
            acc[3] = __fadd_rn(acc[3], __fmul_rn(wv, bf16_hi(v[j].y)));
            acc[4] = __fadd_rn(acc[4], __fmul_rn(wv, bf16_lo(v[j].z)));
            acc[5] = __fadd_rn(acc[5], __fmul_rn(wv, bf16_hi(v[j].z)));
            acc[6] = __fadd_rn(acc[6], __fmul_rn(wv, bf16_lo(v[j].w)));
            acc[7] = __fadd_rn(acc[7], __fmul_rn(wv, bf16_hi(v[j].w)));
        }
    }
    u32x4 o;
    o.x = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
    o.y = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
    o.z = f32_to_bf16(acc[4]) | (f32_to_bf16(acc[5]) << 16);
    o.w = f32_to_bf16(acc[6]) | (f32_to_bf16(acc[7]) << 16);
    return o;
}

template <int C, int KMAX>
__device__ __forceinline__ void combine_item(const CombineArgs& a, int64_t item, int lane) {
    const int t = (int)(item / a.nslices);
    const int s = (int)(item - (int64_t)t * a.nslices);
    const int k = a.k;

    int p = -1;
    float wt = 0.0f;
    if (lane < k) {
        p = a.pos[(int64_t)t * k + lane];
        wt = a.w != nullptr ? a.w[(int64_t)t * k + lane] : 1.0f;   // no weights: dispatch backward
        if (p < -1 || p >= a.rows_cap) {
            atomicOr(a.err, kErrBounds);
            p = -1;
        }
    }
    int pj[KMAX];
    float wj[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        pj[j] = readlane(p, j);   // lanes >= k hold -1
        wj[j] = readlane(wt, j);
    }

    const int64_t nchunk = a.H / 8;
    const int64_t g0 = (int64_t)s * 64 * C + lane;
    const u32x4* __restrict__ y = reinterpret_cast<const u32x4*>(a.y);
    // output row as a buffer: non-temporal stores at system scope (as the
    // dispatch's rows; decode step 9.8 -> 9.6 us, prefill unchanged); a chunk
    // past the row end falls out of it
    const __amdgpu_buffer_rsrc_t out = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<u32x4*>(a.out) + (int64_t)t * nchunk, 0, (int)(nchunk * 16), 0x00020000);
    if (C * KMAX <= 16 && g0 - lane + C * 64 <= nchunk) {
        // whole slice inside the row: every load of the slice is issued before
        // any arithmetic, so that all C * k row chunks are in flight at once
        // (chunk by chunk the wavefront waits for each chunk's rows in turn;
        // measured on MI355X, ~1.5% slower on the prefill shape); at most 16
        // chunks held, which keeps the kernel under 80 registers
        u32x4 v[C][KMAX];
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
#pragma unroll
            for (int i = 0; i < C; ++i)
                if (pj[j] >= 0) v[i][j] = __builtin_nontemporal_load(y + (int64_t)pj[j] * nchunk + g0 + i * 64);
#pragma unroll
        for (int i = 0; i < C; ++i)
            __builtin_amdgcn_raw_buffer_store_b128(combine_chunk<KMAX>(v[i], pj, wj), out, (int)((g0 + i * 64) * 16), 0,
                                                   kStoreRows);
        return;
    }
#pragma unroll
    for (int i = 0; i < C; ++i) {   // ragged row tail, or too many chunks to hold: chunk by chunk
        const int64_t g = g0 + i * 64;
        const ChunkState cs = chunk_state(g0 - lane + i * 64, nchunk);
        if (cs == kChunkFull || (cs == kChunkPart && g < nchunk)) {
            u32x4 v[KMAX];
#pragma unroll
            for (int j = 0; j < KMAX; ++j)
                if (pj[j] >= 0) v[j] = __builtin_nontemporal_load(y + (int64_t)pj[j] * nchunk + g);
            __builtin_amdgcn_raw_buffer_store_b128(combine_chunk<KMAX>(v, pj, wj), out, (int)(g * 16), 0, kStoreRows);
        }
    }
}

template <int C, int KMAX>
__global__ __launch_bounds__(kCombineThreads) void k_combine(CombineArgs a) {
    constexpr int kWaves = kCombineThreads / 64;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    const int64_t total = (int64_t)a.T * a.nslices;
    const int64_t stride = (int64_t)gridDim.x * kWaves;
    for (int64_t item = (int64_t)blockIdx.x * kWaves + w; item < total; item += stride)
        combine_item<C, KMAX>(a, item, lane);
}

// ============================================================== combine backward
// Sum over the 64 lanes; every lane gets the total (fixed butterfly order).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// One chunk (8 channels) of the output gradient gv against eight routed rows
// v: grad_y rows get bf16(w_j * go), and dot[j] accumulates go * y_j (each
// product of two bf16 values is exact in fp32, so the fused multiply-add
// rounds as a separate add would).
__device__ __forceinline__ void combine_bwd_chunk(const u32x4& gv, const u32x4 (&v)[8], const int* pj,
                                                  const float* wj, float* dot, u32x4* gy, int64_t nchunk,
                                                  int64_t g) {
    const float gf[8] = {bf16_lo(gv.x), bf16_hi(gv.x), bf16_lo(gv.y), bf16_hi(gv.y),
                         bf16_lo(gv.z), bf16_hi(gv.z), bf16_lo(gv.w), bf16_hi(gv.w)};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (pj[j] >= 0) {
            float d = dot[j];
            d = __builtin_fmaf(gf[0], bf16_lo(v[j].x), d);
            d = __builtin_fmaf(gf[1], bf16_hi(v[j].x), d);
            d = __builtin_fmaf(gf[2], bf16_lo(v[j].y), d);
            d = __builtin_fmaf(gf[3], bf16_hi(v[j].y), d);
            d = __builtin_fmaf(gf[4], bf16_lo(v[j].z), d);
            d = __builtin_fmaf(gf[5], bf16_hi(v[j].z), d);
            d = __builtin_fmaf(gf[6], bf16_lo(v[j].w), d);
            d = __builtin_fmaf(gf[7], bf16_hi(v[j].w), d);
            dot[j] = d;
            const float wv = wj[j];
            u32x4 o;
            o.x = f32_to_bf16(__fmul_rn(wv, gf[0])) | (f32_to_bf16(__fmul_rn(wv, gf[1])) << 16);
            o.y = f32_to_bf16(__fmul_rn(wv, gf[2])) | (f32_to_bf16(__fmul_rn(wv, gf[3])) << 16);
            o.z = f32_to_bf16(__fmul_rn(wv, gf[4])) | (f32_to_bf16(__fmul_rn(wv, gf[5])) << 16);
            o.w = f32_to_bf16(__fmul_rn(wv, gf[6])) | (f32_to_bf16(__fmul_rn(wv, gf[7])) << 16);
            __builtin_nontemporal_store(o, gy + (int64_t)pj[j] * nchunk + g);
        }
    }
}

// One block per token, one wavefront per row slice (blockDim.x / 64 slices of
// C 16-byte chunks per lane).  For each chunk of the token's output gradient:
// load it and the routed expert-output rows (eight slots at a time, to bound
// registers; with at most eight slots and the whole slice inside the row,
// every load of the slice first), write bf16(w_j * go) to each routed row of
// grad_y, and accumulate the chunk's products go * y_j into one fp32 partial
// dot product per slot (combine_bwd_chunk).  Partials are reduced
// over the wavefront (fixed butterfly), then over the block's wavefronts in
// wavefront order through LDS: deterministic, and no device-scope fence (on
// this chip a release fence writes back the L2, which costs more than the
// whole kernel when every wavefront issues one).  Measured on MI355X:
// non-temporal loads and stores, ~3% ahead of cached ones; the time does not
// depend on the slice width.
template <int C, int KMAX>
__device__ __forceinline__ void combine_bwd_token(const CombineBwdArgs& a, int t, int s, int lane,
                                                  float (*red)[KMAX]) {
    const int nw = blockDim.x >> 6;
    const int k = a.k;

    int p = -1;
    float wt = 0.0f;
    if (lane < k) {
        p = a.pos[(int64_t)t * k + lane];
        wt = a.w[(int64_t)t * k + lane];
        if (p < -1 || p >= a.rows_cap) {
            if (s == 0) atomicOr(a.err, kErrBounds);
            p = -1;
        }
    }
    int pj[KMAX];
    float wj[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        pj[j] = readlane(p, j);
        wj[j] = readlane(wt, j);
    }

    const int64_t nchunk = a.H / 8;
    const int64_t g0 = (int64_t)s * 64 * C + lane;
    const u32x4* __restrict__ go = reinterpret_cast<const u32x4*>(a.go) + (int64_t)t * nchunk;
    const u32x4* __restrict__ y = reinterpret_cast<const u32x4*>(a.y);
    u32x4* __restrict__ gy = reinterpret_cast<u32x4*>(a.gy);
    float dot[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) dot[j] = 0.0f;
    if (KMAX == 8 && C <= 2 && g0 - lane + C * 64 <= nchunk) {
        // whole slice inside the row and at most eight slots: every load of the
        // slice first, as in the combine (up to two chunks per lane: more would
        // not fit the 128 registers of a 1024-thread block)
        u32x4 gv[C], v[C][8];
#pragma unroll
        for (int i = 0; i < C; ++i) gv[i] = __builtin_nontemporal_load(go + g0 + i * 64);
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int i = 0; i < C; ++i)
                if (pj[j] >= 0) v[i][j] = __builtin_nontemporal_load(y + (int64_t)pj[j] * nchunk + g0 + i * 64);
#pragma unroll
        for (int i = 0; i < C; ++i) combine_bwd_chunk(gv[i], v[i], pj, wj, dot, gy, nchunk, g0 + i * 64);
    } else {
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const int64_t g = g0 + i * 64;
            const ChunkState cs = chunk_state(g0 - lane + i * 64, nchunk);
            if (cs == kChunkFull || (cs == kChunkPart && g < nchunk)) {
                const u32x4 gv = __builtin_nontemporal_load(go + g);
#pragma unroll
                for (int jb = 0; jb < KMAX; jb += 8) {   // eight slots at a time
                    if (jb >= k) break;
                    u32x4 v[8];
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj)
                        if (pj[jb + jj] >= 0) v[jj] = __builtin_nontemporal_load(y + (int64_t)pj[jb + jj] * nchunk + g);
                    combine_bwd_chunk(gv, v, pj + jb, wj + jb, dot + jb, gy, nchunk, g);
                }
            }
        }
    }

    // wavefront totals -> LDS (lane j holds slot j), then wavefront 0 adds the
    // slices in order
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        if (j < k && pj[j] >= 0) {
            const float tot = wave_sum(dot[j]);
            if (lane == 0) red[s][j] = tot;
        }
    }
    __syncthreads();
    if (s == 0 && lane < k) {
        float acc = 0.0f;
        if (p >= 0)
            for (int q = 0; q < nw; ++q) acc += red[q][lane];
        a.gw[(int64_t)t * k + lane] = acc;
    }
    __syncthreads();   // red is reused by the block's next token
}

// One block per token; with a capped grid each block takes every
// gridDim.x-th token.
template <int C, int KMAX>
__global__ __launch_bounds__(64 * bwd_max_waves(KMAX)) void k_combine_bwd(CombineBwdArgs a) {
    __shared__ float red[bwd_max_waves(KMAX)][KMAX];
    const int lane = threadIdx.x & 63;
    const int s = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // slice = wavefront
    for (int t = blockIdx.x; t < a.T; t += gridDim.x) combine_bwd_token<C, KMAX>(a, t, s, lane, red);
}

template <int C>
hipError_t pack_c(const PackArgs& a, bool fp8, bool ll, bool send, dim3 grid, hipStream_t st) {
    if (!fp8 && !ll && send) hipLaunchKernelGGL((k_pack<C, false, false, true>), grid, dim3(kBlockThreads), 0, st, a);
    else if (!fp8 && !ll && !send) hipLaunchKernelGGL((k_pack<C, false, false, false>), grid, dim3(kBlockThreads), 0, st, a);
    else if (!fp8 && ll) hipLaunchKernelGGL((k_pack<C, false, true, false>), grid, dim3(kBlockThreads), 0, st, a);
    else if (fp8 && !ll && send) hipLaunchKernelGGL((k_pack<C, true, false, true>), grid, dim3(kBlockThreads), 0, st, a);
    else if (fp8 && !ll && !send) hipLaunchKernelGGL((k_pack<C, true, false, false>), grid, dim3(kBlockThreads), 0, st, a);
    else hipLaunchKernelGGL((k_pack<C, true, true, false>), grid, dim3(kBlockThreads), 0, st, a);
    return hipGetLastError();
}

template <int C>
hipError_t combine_c(const CombineArgs& a, int kmax, dim3 grid, hipStream_t st) {
    if (kmax <= 8) hipLaunchKernelGGL((k_combine<C, 8>), grid, dim3(kCombineThreads), 0, st, a);
    else if (kmax <= 16) hipLaunchKernelGGL((k_combine<C, 16>), grid, dim3(kCombineThreads), 0, st, a);
    else hipLaunchKernelGGL((k_combine<C, 32>), grid, dim3(kCombineThreads), 0, st, a);
    return hipGetLastError();
}

template <int C>
hipError_t combine_bwd_c(const CombineBwdArgs& a, int kmax, int waves, int max_blocks, hipStream_t st) {
    const int blocks = max_blocks > 0 && a.T > max_blocks ? max_blocks : a.T;
    const dim3 grid((unsigned)blocks), block((unsigned)(64 * waves));
    if (kmax <= 8) hipLaunchKernelGGL((k_combine_bwd<C, 8>), grid, block, 0, st, a);
    else if (kmax <= 16) hipLaunchKernelGGL((k_combine_bwd<C, 16>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_combine_bwd<C, 32>), grid, block, 0, st, a);
    return hipGetLastError();
}

__global__ __launch_bounds__(kBlockThreads) void k_zero_words(uint32_t* p, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kBlockThreads;
    for (int64_t i = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

// At least one block: block 0 of the dispatch kernel also writes the handle's
// offsets and counts, which must happen even when there are no tokens.
// max_blocks > 0 caps the grid (the kernels loop over their items).
dim3 items_grid(int64_t items, int64_t max_blocks, int waves_per_block = kWavesPerBlock) {
    int64_t blocks = (items + waves_per_block - 1) / waves_per_block;
    if (max_blocks > 0 && blocks > max_blocks) blocks = max_blocks;
    return dim3((unsigned)(blocks > 0 ? blocks : 1));
}

}  // namespace

hipError_t launch_layout(const LayoutArgs& a, int ntiles, int warm_blocks, hipStream_t s) {
    if (ntiles < 1 || a.ntiles != ntiles || a.mode != layout_mode(ntiles) || warm_blocks < 0 ||
        (warm_blocks > 0 && (a.warm == nullptr || a.warm_sink == nullptr)))
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)(ntiles + warm_blocks));
    if (a.k <= 8) hipLaunchKernelGGL(k_layout<8>, grid, dim3(kLayoutThreads), 0, s, a);
    else if (a.k <= 16) hipLaunchKernelGGL(k_layout<16>, grid, dim3(kLayoutThreads), 0, s, a);
    else hipLaunchKernelGGL(k_layout<32>, grid, dim3(kLayoutThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_pack(const PackArgs& a, int chunks, bool fp8, bool ll, bool send, int max_blocks,
                       hipStream_t s) {
    const dim3 grid = items_grid((int64_t)a.T * a.nslices, max_blocks);
    switch (chunks) {
        case 1: return pack_c<1>(a, fp8, ll, send, grid, s);
        case 2: return pack_c<2>(a, fp8, ll, send, grid, s);
        case 4: return pack_c<4>(a, fp8, ll, send, grid, s);
        case 8: return pack_c<8>(a, fp8, ll, send, grid, s);
        case 16: return pack_c<16>(a, fp8, ll, send, grid, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_ll_fused(const PackArgs& a, int chunks, int threads, bool fp8, hipStream_t s) {
    // block 0: the handle's summary; then ll_bpt blocks per token
    const dim3 grid((unsigned)((int64_t)a.T * a.ll_bpt + 1));
#define MOE_LL_CASE(CC, NT)                                                                          \
    if (chunks == CC && threads == NT) {                                                              \
        if (fp8) hipLaunchKernelGGL((k_ll_dispatch<CC, true, NT>), grid, dim3(NT), 0, s, a);          \
        else hipLaunchKernelGGL((k_ll_dispatch<CC, false, NT>), grid, dim3(NT), 0, s, a);             \
        return hipGetLastError();                                                                     \
    }
    MOE_LL_CASE(1, 256)   // rows of up to 256 chunks
    MOE_LL_CASE(1, 512)   // longer rows, ll_bpt blocks per token
#undef MOE_LL_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_zero_words(uint32_t* p, int64_t words, hipStream_t s) {
    if (words <= 0) return hipSuccess;
    int64_t blocks = (words + kBlockThreads - 1) / kBlockThreads;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(k_zero_words, dim3((unsigned)blocks), dim3(kBlockThreads), 0, s, p, words);
    return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, int chunks, int kmax, int max_blocks, hipStream_t s) {
    // a cap counts 256-thread workgroups: the same wavefronts as one-wavefront workgroups
    const int64_t cap = max_blocks > 0 ? (int64_t)max_blocks * (kBlockThreads / kCombineThreads) : 0;
    const dim3 grid = items_grid((int64_t)a.T * a.nslices, cap, kCombineThreads / 64);
    switch (chunks) {
        case 1: return combine_c<1>(a, kmax, grid, s);
        case 2: return combine_c<2>(a, kmax, grid, s);
        case 4: return combine_c<4>(a, kmax, grid, s);
        case 8: return combine_c<8>(a, kmax, grid, s);
        case 16: return combine_c<16>(a, kmax, grid, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_combine_bwd(const CombineBwdArgs& a, int chunks, int kmax, int max_blocks, hipStream_t s) {
    // one block per token, one wavefront per slice
    if (a.T < 1 || a.nslices < 1 || a.nslices > bwd_max_waves(kmax)) return hipErrorInvalidValue;
    switch (chunks) {
        case 1: return combine_bwd_c<1>(a, kmax, a.nslices, max_blocks, s);
        case 2: return combine_bwd_c<2>(a, kmax, a.nslices, max_blocks, s);
        case 4: return combine_bwd_c<4>(a, kmax, a.nslices, max_blocks, s);
        case 8: return combine_bwd_c<8>(a, kmax, a.nslices, max_blocks, s);
        case 16: return combine_bwd_c<16>(a, kmax, a.nslices, max_blocks, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
