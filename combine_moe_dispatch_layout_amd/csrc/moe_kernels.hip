// HIP kernels for MoE dispatch-layout / dispatch / combine on gfx950 (CDNA4).
//
// All three steps are bound by memory traffic, not arithmetic: layout reads
// topk_idx once, dispatch reads each token row once and writes it to every
// destination, combine reads every expert-output row once and writes each
// token row once.  Design points:
//  * Layout: one block per 256-token tile, 4 wavefronts of 64 tokens.  Stable
//    (token, slot) ranks come from a wavefront "match-any" (one ballot per key
//    bit) plus per-wavefront LDS histograms -- no atomics decide any order, so
//    results are deterministic.  The last tile block to arrive (device-scope
//    counter) scans the per-tile histograms into global row bases, so count and
//    scan are one launch.
//  * Dispatch: one wavefront per (token, row slice).  The slice is loaded once
//    into registers with 16-byte loads, optionally quantised to E4M3 in
//    registers (block amax by cross-lane max over the 16 lanes holding one
//    128-channel block), then stored with 16-byte (8-byte for fp8) non-temporal
//    stores to every destination row: up to min(k, R) send rows and k
//    receive rows.  Destination row indices are wave-uniform (readlane ->
//    SGPR), so the store loop has no divergence.
//  * Combine: one wavefront per (token, row slice); for each 16-byte chunk the
//    k routed rows are loaded together, accumulated in fp32 in slot order with
//    separately rounded multiply and add, rounded once to bf16 (RNE).
// There is no contraction to put on MFMA.
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

// ============================================================== layout
__global__ __launch_bounds__(kBlockThreads) void k_layout(LayoutArgs a) {
    __shared__ int32_t hist_e[kWavesPerBlock * MOE_MAX_EXPERTS];
    __shared__ int32_t hist_r[kWavesPerBlock * MOE_MAX_RANKS];
    __shared__ int32_t scan_buf[kBlockThreads];
    __shared__ int s_last;

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int E = a.E, R = a.R, k = a.k;
    for (int i = tid; i < kWavesPerBlock * E; i += kBlockThreads) hist_e[i] = 0;
    for (int i = tid; i < kWavesPerBlock * R; i += kBlockThreads) hist_r[i] = 0;
    __syncthreads();

    const int64_t tok0 = (int64_t)blockIdx.x * kTileTokens + w * 64;   // this wave's first token
    const int64_t t = tok0 + lane;
    const bool tok_ok = t < a.T;
    const int64_t ntok = a.T - tok0 < 0 ? 0 : (a.T - tok0 > 64 ? 64 : a.T - tok0);
    const int64_t nent = ntok * k;          // (token, slot) entries of this wave, row-major
    const int64_t ent0 = tok0 * k;
    const uint64_t below = lanes_below(lane);

    // ---- phase 1: per-wavefront expert and rank histograms
    for (int c = 0; c < k; ++c) {
        const int64_t i = (int64_t)c * 64 + lane;
        int e = -1;
        if (i < nent) {
            const int64_t v = a.topk_idx[ent0 + i];
            if (v >= 0 && v < E) e = (int)v;
            else if (v != -1) atomicOr(a.err, kErrBadTopk);
        }
        const uint64_t peers = match_any(e, e >= 0, a.ebits);
        if (e >= 0 && (peers & below) == 0) hist_e[w * E + e] += __popcll(peers);
    }
    uint64_t rmask = 0;
    if (tok_ok) {
        for (int j = 0; j < k; ++j) {
            const int64_t v = a.topk_idx[t * k + j];
            if (v >= 0 && v < E) rmask |= 1ull << ((int)v / a.El);
        }
    }
    for (int r = 0; r < R; ++r) {
        const uint64_t bal = __ballot((rmask >> r) & 1);
        if (lane == 0) hist_r[w * R + r] = __popcll(bal);
    }
    if (tok_ok && a.out_in_rank != nullptr) {
        for (int r = 0; r < R; ++r) a.out_in_rank[t * R + r] = (uint8_t)((rmask >> r) & 1);
    }
    __syncthreads();

    // ---- exclusive prefix over the 4 wavefronts; tile totals to global
    for (int e = tid; e < E; e += kBlockThreads) {
        int run = 0;
        for (int ww = 0; ww < kWavesPerBlock; ++ww) {
            const int c = hist_e[ww * E + e];
            hist_e[ww * E + e] = run;
            run += c;
        }
        a.tile_e[(int64_t)blockIdx.x * E + e] = run;
    }
    for (int r = tid; r < R; r += kBlockThreads) {
        int run = 0;
        for (int ww = 0; ww < kWavesPerBlock; ++ww) {
            const int c = hist_r[ww * R + r];
            hist_r[ww * R + r] = run;
            run += c;
        }
        a.tile_r[(int64_t)blockIdx.x * R + r] = run;
    }
    __syncthreads();

    // ---- phase 2: stable rank of every entry inside the tile
    for (int c = 0; c < k; ++c) {
        const int64_t i = (int64_t)c * 64 + lane;
        int e = -1;
        if (i < nent) {
            const int64_t v = a.topk_idx[ent0 + i];
            if (v >= 0 && v < E) e = (int)v;
        }
        const uint64_t peers = match_any(e, e >= 0, a.ebits);
        if (e >= 0) {
            const int base = hist_e[w * E + e];
            a.erank[ent0 + i] = (uint16_t)(base + __popcll(peers & below));
            if ((peers & below) == 0) hist_e[w * E + e] = base + __popcll(peers);
        }
    }
    for (int r = 0; r < R; ++r) {
        const bool in = (rmask >> r) & 1;
        const uint64_t bal = __ballot(in);
        if (in) a.srank[(int64_t)r * a.max_tokens + t] = (uint16_t)(hist_r[w * R + r] + __popcll(bal & below));
    }

    // ---- arrival; the last block turns tile totals into global row bases
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = (atomicAdd(a.done, 1u) == gridDim.x - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    const int ntiles = gridDim.x;
    int32_t* tot_e = hist_e;                       // [E] totals
    int32_t* off_e = hist_e + MOE_MAX_EXPERTS;     // [E] exclusive offsets
    int32_t* tot_r = hist_r;
    int32_t* off_r = hist_r + MOE_MAX_RANKS;
    for (int e = tid; e < E; e += kBlockThreads) {
        int run = 0;
        for (int tl = 0; tl < ntiles; ++tl) {
            const int64_t o = (int64_t)tl * E + e;
            const int c = a.tile_e[o];
            a.tile_e[o] = run;
            run += c;
        }
        tot_e[e] = run;
    }
    for (int r = tid; r < R; r += kBlockThreads) {
        int run = 0;
        for (int tl = 0; tl < ntiles; ++tl) {
            const int64_t o = (int64_t)tl * R + r;
            const int c = a.tile_r[o];
            a.tile_r[o] = run;
            run += c;
        }
        tot_r[r] = run;
    }
    __syncthreads();

    // exclusive scan of the expert totals: thread tid owns a run of `per` experts
    const int per = (E + kBlockThreads - 1) / kBlockThreads;
    const int lo = tid * per < E ? tid * per : E;
    const int hi = lo + per < E ? lo + per : E;
    int own = 0;
    for (int e = lo; e < hi; ++e) own += tot_e[e];
    scan_buf[tid] = own;
    __syncthreads();
    for (int off = 1; off < kBlockThreads; off <<= 1) {
        const int v = tid >= off ? scan_buf[tid - off] : 0;
        __syncthreads();
        scan_buf[tid] += v;
        __syncthreads();
    }
    int run = scan_buf[tid] - own;
    for (int e = lo; e < hi; ++e) {
        const int c = tot_e[e];
        off_e[e] = run;
        a.eoff[e] = run;
        a.cnt_e[e] = c;
        if (a.out_cnt_e != nullptr) a.out_cnt_e[e] = c;
        run += c;
    }
    if (tid == kBlockThreads - 1) a.eoff[E] = scan_buf[tid];
    if (tid == 0) {
        int rr = 0;
        for (int r = 0; r < R; ++r) {
            const int c = tot_r[r];
            off_r[r] = rr;
            a.roff[r] = rr;
            a.cnt_r[r] = c;
            if (a.out_cnt_r != nullptr) a.out_cnt_r[r] = c;
            rr += c;
        }
        a.roff[R] = rr;
    }
    __syncthreads();
    for (int e = tid; e < E; e += kBlockThreads) {
        const int b = off_e[e];
        for (int tl = 0; tl < ntiles; ++tl) a.tile_e[(int64_t)tl * E + e] += b;
    }
    for (int r = tid; r < R; r += kBlockThreads) {
        const int b = off_r[r];
        for (int tl = 0; tl < ntiles; ++tl) a.tile_r[(int64_t)tl * R + r] += b;
    }
    if (tid == 0) *a.done = 0u;
}

// ============================================================== dispatch
template <int C, bool FP8, bool LL, bool SEND>
__global__ __launch_bounds__(kBlockThreads) void k_pack(PackArgs a) {
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    if (blockIdx.x == 0) {   // handle copies of the layout offsets and counts
        for (int i = tid; i <= a.E; i += kBlockThreads) a.h_eoff[i] = a.eoff[i];
        for (int i = tid; i < a.E; i += kBlockThreads) a.h_recv_counts[i] = a.cnt_e[i];
        for (int i = tid; i <= a.R; i += kBlockThreads) a.h_roff[i] = a.roff[i];
    }
    const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + w;
    if (item >= (int64_t)a.T * a.nslices) return;
    const int t = (int)(item / a.nslices);
    const int s = (int)(item - (int64_t)t * a.nslices);
    const int k = a.k;
    const uint64_t below = lanes_below(lane);

    // ---- routing of token t: lane j < k owns slot j
    int e = -1;
    if (lane < k) {
        const int64_t v = a.topk_idx[(int64_t)t * k + lane];
        if (v >= 0 && v < a.E) e = (int)v;
    }
    const int tile = t / kTileTokens;
    int cpos = -1;   // contiguous expert-major row (index into recv_src_idx)
    int rrow = -1;   // receive row (contiguous, or padded low-latency slot)
    if (e >= 0) {
        cpos = a.tile_e[(int64_t)tile * a.E + e] + a.erank[(int64_t)t * k + lane];
        int64_t row = cpos;
        if (LL) row = (int64_t)e * a.cap + (int64_t)a.s0 * a.max_tokens + (cpos - a.eoff[e]);
        if (cpos < 0 || cpos >= a.pairs_cap || row < 0 || row >= a.recv_cap_rows) {
            atomicOr(a.err, kErrBounds);
            cpos = -1;
        } else {
            rrow = (int)row;
        }
    }
    const int r = e >= 0 ? e / a.El : 0;
    const uint64_t peers = match_any(r, e >= 0, a.rbits);
    int srow = -1;   // send row: only for the first slot of each destination rank
    if (SEND && e >= 0 && (peers & below) == 0) {
        const int64_t row = (int64_t)a.tile_r[(int64_t)tile * a.R + r] + a.srank[(int64_t)r * a.max_tokens + t];
        if (row < 0 || row >= a.send_cap_rows) atomicOr(a.err, kErrBounds);
        else srow = (int)row;
    }
    if (s == 0 && lane < k) {
        a.h_pos[(int64_t)t * k + lane] = rrow;
        if (cpos >= 0) a.h_recv_src[cpos] = t;
        if (srow >= 0) a.h_send_src[srow] = t;
    }

    // ---- load this slice of the row once
    const int64_t nchunk = a.H / 8;                   // 16-byte bf16 chunks per row
    const int64_t g0 = (int64_t)s * 64 * C + lane;
    const u32x4* src = reinterpret_cast<const u32x4*>(a.x + (int64_t)t * a.H);
    u32x4 v[C];
#pragma unroll
    for (int i = 0; i < C; ++i) {
        const int64_t g = g0 + i * 64;
        v[i] = g < nchunk ? __builtin_nontemporal_load(src + g) : u32x4{0u, 0u, 0u, 0u};
    }

    if constexpr (!FP8) {
        for (int j = 0; j < k; ++j) {
            const int rr = readlane(rrow, j);
            if (rr >= 0) {
                u32x4* dst = reinterpret_cast<u32x4*>(a.recv_rows) + (int64_t)rr * nchunk;
#pragma unroll
                for (int i = 0; i < C; ++i) {
                    const int64_t g = g0 + i * 64;
                    if (g < nchunk) __builtin_nontemporal_store(v[i], dst + g);
                }
            }
            if constexpr (SEND) {
                const int sr = readlane(srow, j);
                if (sr >= 0) {
                    u32x4* dst = reinterpret_cast<u32x4*>(a.send_rows) + (int64_t)sr * nchunk;
#pragma unroll
                    for (int i = 0; i < C; ++i) {
                        const int64_t g = g0 + i * 64;
                        if (g < nchunk) __builtin_nontemporal_store(v[i], dst + g);
                    }
                }
            }
        }
    } else {
        // ---- E4M3 quantisation, once per token; 16 lanes hold one 128-channel block
        u32x2 q[C];
        float sinv[C];
#pragma unroll
        for (int i = 0; i < C; ++i) {
            float f[8] = {bf16_lo(v[i].x), bf16_hi(v[i].x), bf16_lo(v[i].y), bf16_hi(v[i].y),
                          bf16_lo(v[i].z), bf16_hi(v[i].z), bf16_lo(v[i].w), bf16_hi(v[i].w)};
            float m = 0.0f;
#pragma unroll
            for (int u = 0; u < 8; ++u) m = fmaxf(m, fabsf(f[u]));
            m = fmaxf(m, __shfl_xor(m, 8, 16));
            m = fmaxf(m, __shfl_xor(m, 4, 16));
            m = fmaxf(m, __shfl_xor(m, 2, 16));
            m = fmaxf(m, __shfl_xor(m, 1, 16));
            const float ap = m > 1e-4f ? m : 1e-4f;
            const float sc = 448.0f / ap;     // correctly rounded binary32 divide
            sinv[i] = ap / 448.0f;
            int lo = 0, hi = 0;
            lo = __builtin_amdgcn_cvt_pk_fp8_f32(__fmul_rn(f[0], sc), __fmul_rn(f[1], sc), lo, false);
            lo = __builtin_amdgcn_cvt_pk_fp8_f32(__fmul_rn(f[2], sc), __fmul_rn(f[3], sc), lo, true);
            hi = __builtin_amdgcn_cvt_pk_fp8_f32(__fmul_rn(f[4], sc), __fmul_rn(f[5], sc), hi, false);
            hi = __builtin_amdgcn_cvt_pk_fp8_f32(__fmul_rn(f[6], sc), __fmul_rn(f[7], sc), hi, true);
            q[i] = u32x2{(uint32_t)lo, (uint32_t)hi};
        }
        const int nb = a.H / 128;
        for (int j = 0; j < k; ++j) {
            const int rr = readlane(rrow, j);
            if (rr >= 0) {
                u32x2* dst = reinterpret_cast<u32x2*>(a.recv_rows) + (int64_t)rr * nchunk;
                float* sdst = a.recv_scales + (int64_t)rr * nb;
#pragma unroll
                for (int i = 0; i < C; ++i) {
                    const int64_t g = g0 + i * 64;
                    if (g < nchunk) {
                        __builtin_nontemporal_store(q[i], dst + g);
                        if ((lane & 15) == 0) sdst[g >> 4] = sinv[i];
                    }
                }
            }
            if constexpr (SEND) {
                const int sr = readlane(srow, j);
                if (sr >= 0) {
                    u32x2* dst = reinterpret_cast<u32x2*>(a.send_rows) + (int64_t)sr * nchunk;
                    float* sdst = a.send_scales + (int64_t)sr * nb;
#pragma unroll
                    for (int i = 0; i < C; ++i) {
                        const int64_t g = g0 + i * 64;
                        if (g < nchunk) {
                            __builtin_nontemporal_store(q[i], dst + g);
                            if ((lane & 15) == 0) sdst[g >> 4] = sinv[i];
                        }
                    }
                }
            }
        }
    }
}

// ============================================================== combine
template <int C, int KMAX>
__global__ __launch_bounds__(kBlockThreads) void k_combine(CombineArgs a) {
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + w;
    if (item >= (int64_t)a.T * a.nslices) return;
    const int t = (int)(item / a.nslices);
    const int s = (int)(item - (int64_t)t * a.nslices);
    const int k = a.k;

    int p = -1;
    float wt = 0.0f;
    if (lane < k) {
        p = a.pos[(int64_t)t * k + lane];
        wt = a.w[(int64_t)t * k + lane];
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
    const u32x4* y = reinterpret_cast<const u32x4*>(a.y);
    u32x4* out = reinterpret_cast<u32x4*>(a.out) + (int64_t)t * nchunk;
#pragma unroll
    for (int i = 0; i < C; ++i) {
        const int64_t g = g0 + i * 64;
        if (g < nchunk) {
            u32x4 v[KMAX];
#pragma unroll
            for (int j = 0; j < KMAX; ++j)
                if (pj[j] >= 0) v[j] = __builtin_nontemporal_load(y + (int64_t)pj[j] * nchunk + g);
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
            __builtin_nontemporal_store(o, out + g);
        }
    }
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
    if (kmax <= 8) hipLaunchKernelGGL((k_combine<C, 8>), grid, dim3(kBlockThreads), 0, st, a);
    else if (kmax <= 16) hipLaunchKernelGGL((k_combine<C, 16>), grid, dim3(kBlockThreads), 0, st, a);
    else hipLaunchKernelGGL((k_combine<C, 32>), grid, dim3(kBlockThreads), 0, st, a);
    return hipGetLastError();
}

// At least one block: block 0 of the dispatch kernel also writes the handle's
// offsets and counts, which must happen even when there are no tokens.
dim3 items_grid(int64_t items) {
    const int64_t blocks = (items + kWavesPerBlock - 1) / kWavesPerBlock;
    return dim3((unsigned)(blocks > 0 ? blocks : 1));
}

}  // namespace

hipError_t launch_layout(const LayoutArgs& a, int ntiles, hipStream_t s) {
    hipLaunchKernelGGL(k_layout, dim3(ntiles), dim3(kBlockThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_pack(const PackArgs& a, int chunks, bool fp8, bool ll, bool send, hipStream_t s) {
    const dim3 grid = items_grid((int64_t)a.T * a.nslices);
    switch (chunks) {
        case 1: return pack_c<1>(a, fp8, ll, send, grid, s);
        case 2: return pack_c<2>(a, fp8, ll, send, grid, s);
        case 4: return pack_c<4>(a, fp8, ll, send, grid, s);
        case 8: return pack_c<8>(a, fp8, ll, send, grid, s);
        case 16: return pack_c<16>(a, fp8, ll, send, grid, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_combine(const CombineArgs& a, int chunks, int kmax, hipStream_t s) {
    const dim3 grid = items_grid((int64_t)a.T * a.nslices);
    switch (chunks) {
        case 1: return combine_c<1>(a, kmax, grid, s);
        case 2: return combine_c<2>(a, kmax, grid, s);
        case 4: return combine_c<4>(a, kmax, grid, s);
        case 8: return combine_c<8>(a, kmax, grid, s);
        case 16: return combine_c<16>(a, kmax, grid, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
