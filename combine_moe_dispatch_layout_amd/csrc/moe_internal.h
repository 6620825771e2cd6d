// Internal declarations shared by the kernels (moe_kernels.hip) and the host
// runtime (moe_runtime.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// One layout tile = 256 tokens = 4 wavefronts x 64 tokens (one token per lane).
constexpr int kTileTokens = 256;
constexpr int kBlockThreads = 256;
constexpr int kWavesPerBlock = kBlockThreads / 64;
// The combine (and the dispatch backward, the same kernel) runs one wavefront
// per workgroup: measured on MI355X, ~2% faster than four, warm or cold.
constexpr int kCombineThreads = 64;

// The fused low-latency dispatch handles up to this many (token, slot) entries
// and tokens.
// Layouts of at most this many 256-token tiles publish per-tile counts
// column by column ([column][tile]) for the dispatch to sum (a few 16-byte
// loads); larger ones publish them tile by tile ([tile][column]) and the last
// layout block turns them into prefixes over the tiles, so that the dispatch
// reads one value per column at any size.  Measured on MI355X: the sums are
// faster up to 16384 tokens (by ~1 us per step at 4096 and 1-2% of a dispatch
// after a cache flush), the stored prefixes make the dispatch 12% and 28%
// faster at 32768 and 65536 tokens.
constexpr int kWalkTiles = 64;
constexpr int kFusedMaxEntries = 2048;
constexpr int kFusedMaxTokens = 512;

// Combine backward: one block per token, one wavefront per row slice, at most
// this many wavefronts (fewer above eight slots, which need more registers).
constexpr int bwd_max_waves(int k) { return k > 8 ? 4 : 16; }

// Bits of the sticky device error word.
constexpr uint32_t kErrBadTopk = 1u;
constexpr uint32_t kErrBounds = 2u;
constexpr uint32_t kErrCapacity = 4u;   // a low-latency slot window overflowed (row not placed)
constexpr uint32_t kErrStale = 8u;      // a reused layout no longer matches topk_idx (token dropped)
constexpr uint32_t kErrNonFinite = 16u; // fp8 dispatch met Inf or NaN in a 128-channel block

// Layout mode, chosen on the host from the tile count and passed to both the
// layout and the dispatch kernels (never re-derived on the device).
constexpr int kLayoutOneTile = 0;   // a single tile: no per-tile counts at all
constexpr int kLayoutWalk = 1;      // per-tile counts column by column, summed by the dispatch
constexpr int kLayoutPrefix = 2;    // per-tile exclusive prefixes, tile by tile
inline int layout_mode(int ntiles) {
    return ntiles <= 1 ? kLayoutOneTile : (ntiles <= kWalkTiles ? kLayoutWalk : kLayoutPrefix);
}

// In-tile expert rank of a (token, slot) entry, with the entry's expert id in
// the high half so that a dispatch reusing the layout can check that topk_idx
// has not changed since (0xFFFF = empty or invalid slot).
__host__ __device__ inline uint32_t erank_pack(int e, int rank) {
    return e >= 0 ? ((uint32_t)e << 16) | (uint32_t)rank : 0xFFFF0000u;
}

struct LayoutArgs {
    const int64_t* topk_idx;   // [T, k]
    int32_t T, k, E, R, El;
    uint32_t k_magic;          // ceil(2^20 / k):  entry -> token division
    uint32_t el_magic;         // ceil(2^20 / El): expert -> rank division
    int32_t max_tokens;        // row stride of srank
    int32_t mode;              // kLayoutOneTile / kLayoutWalk / kLayoutPrefix (must match the grid)
    int32_t in_rank_vec4;      // out_in_rank is 4-byte aligned and R % 4 == 0: 32-bit stores
    int32_t* tile_cnt;         // up to kWalkTiles tiles: [E + R, tile_stride] per-tile counts;
                               // beyond: [tiles, cnt_stride], rewritten by the last block as
                               // exclusive prefixes over the tiles
    int32_t tile_stride;       // >= number of tiles, multiple of 4
    int32_t cnt_stride;        // >= E + R, multiple of 64
    int32_t* grand_tot;        // [E + R]  totals over tiles (atomics; zero between launches)
    uint32_t* erank;           // [T, k]       erank_pack(expert, rank of slot (t, j) among the
                               //              expert's rows in the tile)
    uint16_t* srank;           // [R, max_tokens] rank of token t among the tile's tokens sent to r
    int32_t* cnt_e;            // [E]   workspace copies of the results
    int32_t* cnt_r;            // [R]
    int32_t* eoff;             // [E+1]
    int32_t* roff;             // [R+1]
    int32_t* out_cnt_e;        // nullable user outputs
    int32_t* out_cnt_r;
    uint8_t* out_in_rank;      // [T, R]
    uint32_t* err;
    uint32_t* done;            // arrival counter of the tile blocks (reset by the last one)
    int32_t ntiles;            // workgroups 0 .. ntiles-1 are the layout's tiles
    // workgroups ntiles .. gridDim.x-1 read these bytes (the token rows of the
    // dispatch that follows) so that they sit in the Infinity Cache when it runs
    const void* warm;
    int64_t warm_chunks;       // 16-byte chunks at `warm`
    uint32_t* warm_sink;       // written only if the loaded bits hit one value (keeps the loads)
};

struct PackArgs {
    const uint16_t* x;         // bf16 [T, H]
    const int64_t* topk_idx;   // [T, k]
    int32_t T, k, E, R, El, H;
    int32_t rbits;
    int32_t nslices;           // work items per token (row split)
    int32_t ll_bpt;            // fused low-latency dispatch: blocks per token
    int32_t max_tokens;
    int32_t s0;
    int64_t cap;               // low-latency slots per expert (M * R)
    const int32_t* tile_cnt;   // per-tile counts or prefixes over the tiles (see LayoutArgs)
    int32_t tile_stride;
    int32_t cnt_stride;
    int32_t mode;              // the layout mode the layout kernel ran with
    const uint32_t* erank;
    const uint16_t* srank;
    const int32_t* cnt_e;
    const int32_t* eoff;
    const int32_t* roff;
    void* send_rows;
    float* send_scales;
    void* recv_rows;
    float* recv_scales;
    int64_t send_cap_rows;     // rows the send buffer holds
    int64_t recv_cap_rows;     // rows the receive buffer holds
    int64_t pairs_cap;         // entries of recv_src_idx (max_tokens * k)
    int32_t* h_pos;
    int32_t* h_eoff;
    int32_t* h_roff;
    int32_t* h_send_src;
    int32_t* h_recv_src;
    int32_t* h_recv_counts;
    uint32_t* err;
};

struct CombineArgs {
    const uint16_t* y;         // bf16 expert outputs in the receive layout
    const float* w;            // [T, k]; nullptr = every weight 1 (dispatch backward)
    const int32_t* pos;        // [T, k]
    uint16_t* out;             // bf16 [T, H]
    int32_t T, k, H;
    int32_t nslices;
    int64_t rows_cap;          // rows of y the caller's buffer holds
    uint32_t* err;
};

struct CombineBwdArgs {
    const uint16_t* go;        // bf16 [T, H] gradient of the combine output
    const float* w;            // [T, k]
    const uint16_t* y;         // bf16 expert outputs in the receive layout
    const int32_t* pos;        // [T, k]
    uint16_t* gy;              // bf16 gradient of the expert outputs (rows at pos)
    float* gw;                 // [T, k] gradient of the weights
    int32_t T, k, H;
    int32_t nslices;           // wavefronts per block (one block per token), <= bwd_max_waves(k)
    int64_t rows_cap;
    uint32_t* err;
};

// Launchers (moe_kernels.hip).  Each returns the hipError_t of the launch.
// ntiles layout workgroups plus warm_blocks workgroups reading a.warm.
hipError_t launch_layout(const LayoutArgs& a, int ntiles, int warm_blocks, hipStream_t s);
// chunks: 16-byte input chunks each lane handles per work item (1,2,4,8,16).
// max_blocks > 0 caps the grid; the kernels then loop over their work items.
hipError_t launch_pack(const PackArgs& a, int chunks, bool fp8, bool ll, bool send, int max_blocks,
                       hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, int chunks, int kmax, int max_blocks, hipStream_t s);
hipError_t launch_combine_bwd(const CombineBwdArgs& a, int chunks, int kmax, int max_blocks, hipStream_t s);
// Low-latency dispatch without a separate layout launch (T * k <= kFusedMaxEntries,
// T <= kFusedMaxTokens); a summary block plus one block of `threads` (256 or
// 1024) per token.
hipError_t launch_ll_fused(const PackArgs& a, int chunks, int threads, bool fp8, hipStream_t s);
// Zero `words` 32-bit words at p (a kernel, so that it can sit in a captured graph).
hipError_t launch_zero_words(uint32_t* p, int64_t words, hipStream_t s);

}  // namespace moe
