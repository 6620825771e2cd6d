// A C-ABI consumer with no Python and no torch: it allocates device buffers
// with the HIP runtime, builds the inputs on the host, and runs
// moe_dispatch_layout, moe_dispatch and moe_combine through include/moe_ep.h.
// Checks only properties with a closed form (no oracle):
//  * the per-expert counts sum to the valid slots, and every rank count is the
//    number of tokens with at least one expert there;
//  * each receive row holds its source token's row (recv_src_idx);
//  * with the expert outputs equal to the received rows (an identity expert)
//    and weights that sum to exactly one (powers of two), combine returns x
//    bit for bit.
//  * backward, with the gradient rows equal to the received rows: dispatch
//    backward returns bf16(n_valid(t) * x[t]); combine backward with the output
//    gradient x and the identity expert outputs gives grad_w[t, j] = sum_h
//    x[t, h]^2 (exact in fp32 for these small integers) and grad_y rows
//    w * x[t] (exact: powers of two);
//  * a hook recorded after the backward and waited on another stream, and the
//    per-launch timing calls.
// Prints one line and exits 0 on success, 1 on a mismatch, 2 on an API error.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "moe_ep.h"

#define API(x)                                                                      \
    do {                                                                            \
        moe_status st_ = (x);                                                       \
        if (st_ != MOE_OK) {                                                        \
            std::printf("API error %s at line %d\n", moe_status_str(st_), __LINE__); \
            return 2;                                                               \
        }                                                                           \
    } while (0)
#define HIPCHK(x)                                                                            \
    do {                                                                                     \
        hipError_t e_ = (x);                                                                 \
        if (e_ != hipSuccess) {                                                              \
            std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);       \
            return 2;                                                                        \
        }                                                                                    \
    } while (0)

static uint16_t bf16_of_small_int(int v) {   // exact for |v| < 256
    float f = (float)v;
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static float f32_of_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

static uint16_t bf16_rne(float f) {   // round to nearest even (finite values)
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

int main() {
    const int T = 300, H = 1024, E = 64, R = 8, k = 4;
    moe_config cfg = {T, H, E, R, k, 0, MOE_QUANT_BF16, MOE_LAYOUT_CONTIGUOUS};
    moe_ctx* ctx = nullptr;
    API(moe_ctx_create(&cfg, &ctx));

    // inputs: x[t, h] = small integer pattern; slot j of token t -> expert (7t + 13j) mod E
    // (distinct within a row since 13j mod 64 differs for j < 4); slot 3 empty every 5th token
    std::vector<uint16_t> hx((size_t)T * H);
    for (int t = 0; t < T; ++t)
        for (int h = 0; h < H; ++h) hx[(size_t)t * H + h] = bf16_of_small_int(((t * 31 + h * 7) % 251) - 125);
    std::vector<int64_t> hidx((size_t)T * k);
    std::vector<float> hw((size_t)T * k);
    for (int t = 0; t < T; ++t) {
        const int nvalid = (t % 5 == 0) ? 3 : 4;
        for (int j = 0; j < k; ++j) {
            hidx[(size_t)t * k + j] = j < nvalid ? (7 * t + 13 * j) % E : -1;
            // weights summing to exactly one: 1/2, 1/4, 1/8, 1/8 (or 1/2, 1/4, 1/4)
            hw[(size_t)t * k + j] = j == 0 ? 0.5f : j == 1 ? 0.25f : (nvalid == 3 ? (j == 2 ? 0.25f : 0.0f) : 0.125f);
        }
    }

    auto hint = [&](int kind) {
        size_t b = 0;
        moe_size_hint(&cfg, kind, &b);
        return b;
    };
    void *x, *send, *recv, *out;
    int64_t* idx;
    float* w;
    int32_t *cnt_e, *cnt_r;
    uint8_t* in_rank;
    moe_handle h{};
    HIPCHK(hipMalloc(&x, hx.size() * 2));
    HIPCHK(hipMalloc(&idx, hidx.size() * 8));
    HIPCHK(hipMalloc(&w, hw.size() * 4));
    HIPCHK(hipMalloc(&send, hint(MOE_BUF_SEND_ROWS)));
    HIPCHK(hipMalloc(&recv, hint(MOE_BUF_RECV_ROWS)));
    HIPCHK(hipMalloc(&out, hint(MOE_BUF_COMBINE_OUT)));
    HIPCHK(hipMalloc(&cnt_e, hint(MOE_BUF_LAYOUT_EXPERT_COUNTS)));
    HIPCHK(hipMalloc(&cnt_r, hint(MOE_BUF_LAYOUT_RANK_COUNTS)));
    HIPCHK(hipMalloc(&in_rank, hint(MOE_BUF_LAYOUT_TOKEN_IN_RANK)));
    HIPCHK(hipMalloc(&h.pos, hint(MOE_BUF_HANDLE_POS)));
    HIPCHK(hipMalloc(&h.expert_offsets, hint(MOE_BUF_HANDLE_EXPERT_OFFSETS)));
    HIPCHK(hipMalloc(&h.rank_offsets, hint(MOE_BUF_HANDLE_RANK_OFFSETS)));
    HIPCHK(hipMalloc(&h.send_src_idx, hint(MOE_BUF_HANDLE_SEND_SRC)));
    HIPCHK(hipMalloc(&h.recv_src_idx, hint(MOE_BUF_HANDLE_RECV_SRC)));
    HIPCHK(hipMalloc(&h.recv_counts, hint(MOE_BUF_HANDLE_RECV_COUNTS)));
    HIPCHK(hipMemcpy(x, hx.data(), hx.size() * 2, hipMemcpyHostToDevice));
    HIPCHK(hipMemcpy(idx, hidx.data(), hidx.size() * 8, hipMemcpyHostToDevice));
    HIPCHK(hipMemcpy(w, hw.data(), hw.size() * 4, hipMemcpyHostToDevice));

    hipStream_t s;
    HIPCHK(hipStreamCreate(&s));
    // the layout with the token rows read into the Infinity Cache meanwhile (same outputs)
    API(moe_dispatch_layout_prefetch(ctx, idx, T, x, cnt_e, cnt_r, in_rank, s));
    moe_dispatch_buffers bufs = {send, nullptr, recv, nullptr};
    API(moe_dispatch(ctx, x, idx, T, 1, &bufs, &h, s));
    // identity expert: the expert outputs are the received rows themselves
    API(moe_combine(ctx, recv, w, &h, out, s));
    uint32_t flags = 0;
    API(moe_poll_error(ctx, s, &flags));

    std::vector<int32_t> he(E), hr(R), eoff(E + 1), rsrc((size_t)T * k);
    std::vector<uint8_t> hin((size_t)T * R);
    std::vector<uint16_t> hout((size_t)T * H);
    HIPCHK(hipMemcpy(he.data(), cnt_e, E * 4, hipMemcpyDeviceToHost));
    HIPCHK(hipMemcpy(hr.data(), cnt_r, R * 4, hipMemcpyDeviceToHost));
    HIPCHK(hipMemcpy(hin.data(), in_rank, hin.size(), hipMemcpyDeviceToHost));
    HIPCHK(hipMemcpy(eoff.data(), h.expert_offsets, (E + 1) * 4, hipMemcpyDeviceToHost));
    HIPCHK(hipMemcpy(rsrc.data(), h.recv_src_idx, rsrc.size() * 4, hipMemcpyDeviceToHost));
    HIPCHK(hipMemcpy(hout.data(), out, hout.size() * 2, hipMemcpyDeviceToHost));

    long valid = 0, sum_e = 0;
    for (int64_t v : hidx) valid += v >= 0;
    for (int c : he) sum_e += c;
    int bad = 0;
    if (sum_e != valid || eoff[E] != valid) bad |= 1;
    for (int r = 0; r < R; ++r) {
        int n = 0;
        for (int t = 0; t < T; ++t) n += hin[(size_t)t * R + r];
        if (n != hr[r]) bad |= 2;
    }
    std::vector<uint16_t> hrecv((size_t)valid * H);
    HIPCHK(hipMemcpy(hrecv.data(), recv, hrecv.size() * 2, hipMemcpyDeviceToHost));
    for (long i = 0; i < valid; ++i)
        if (std::memcmp(&hrecv[(size_t)i * H], &hx[(size_t)rsrc[i] * H], (size_t)H * 2) != 0) bad |= 4;
    for (size_t i = 0; i < hout.size(); ++i) {
        const uint16_t want = hx[i] == 0x8000 ? 0 : hx[i];   // -0 comes back as +0
        if (hout[i] != want) bad |= 8;
    }
    // ---- backward (timed, completed on a second stream through a hook)
    void *gx, *gy;
    float* gw;
    HIPCHK(hipMalloc(&gx, hout.size() * 2));
    HIPCHK(hipMalloc(&gy, hint(MOE_BUF_EXPERT_OUT)));
    HIPCHK(hipMalloc(&gw, hw.size() * 4));
    API(moe_timing_begin(ctx, 4));
    API(moe_dispatch_backward(ctx, recv, &h, gx, s));          // gradient rows = the received rows
    API(moe_combine_backward(ctx, x, w, recv, &h, gy, gw, s));  // output gradient = x, identity experts
    moe_hook* hook = nullptr;
    API(moe_hook_create(&hook));
    API(moe_hook_record(hook, s));
    hipStream_t s2;
    HIPCHK(hipStreamCreate(&s2));
    API(moe_hook_wait(hook, s2));
    HIPCHK(hipStreamSynchronize(s2));
    int32_t kids[4] = {-1, -1, -1, -1}, nl = 0;
    float ms[4] = {};
    API(moe_timing_launches(ctx, kids, ms, 4, &nl));
    double tot[MOE_KERNEL_COUNT];
    int64_t cnt[MOE_KERNEL_COUNT];
    API(moe_timing_end(ctx, tot, cnt));
    if (nl != 2 || kids[0] != MOE_KERNEL_DISPATCH_BWD || kids[1] != MOE_KERNEL_COMBINE_BWD || !(ms[0] > 0.f) ||
        cnt[MOE_KERNEL_COMBINE_BWD] != 1)
        bad |= 16;
    API(moe_poll_error(ctx, s, &flags));
    std::vector<uint16_t> hgx(hout.size()), hgy((size_t)valid * H);
    std::vector<float> hgw(hw.size());
    HIPCHK(hipMemcpy(hgx.data(), gx, hgx.size() * 2, hipMemcpyDeviceToHost));
    HIPCHK(hipMemcpy(hgw.data(), gw, hgw.size() * 4, hipMemcpyDeviceToHost));
    HIPCHK(hipMemcpy(hgy.data(), gy, hgy.size() * 2, hipMemcpyDeviceToHost));
    std::vector<int32_t> hpos((size_t)T * k);
    HIPCHK(hipMemcpy(hpos.data(), h.pos, hpos.size() * 4, hipMemcpyDeviceToHost));
    for (int t = 0; t < T; ++t) {
        int nv = 0;
        double sq = 0.0;
        for (int j = 0; j < k; ++j) nv += hidx[(size_t)t * k + j] >= 0;
        for (int hh = 0; hh < H; ++hh) {
            const float v = f32_of_bf16(hx[(size_t)t * H + hh]);
            sq += (double)v * v;
            const uint16_t want = bf16_rne((float)nv * v);
            const uint16_t got = hgx[(size_t)t * H + hh];
            if (got != want && !(got == 0 && want == 0x8000)) bad |= 32;   // -0 sums to +0
        }
        for (int j = 0; j < k; ++j) {
            const int p = hpos[(size_t)t * k + j];
            const float gwv = hgw[(size_t)t * k + j];
            if (p < 0) {
                if (gwv != 0.f) bad |= 64;
                continue;
            }
            if ((double)gwv != sq) bad |= 64;
            const float wt = hw[(size_t)t * k + j];
            for (int hh = 0; hh < H; ++hh) {
                const uint16_t want = bf16_rne(wt * f32_of_bf16(hx[(size_t)t * H + hh]));
                if (hgy[(size_t)p * H + hh] != want) bad |= 128;
            }
        }
    }
    std::printf("c_abi_check: T=%d H=%d E=%d R=%d k=%d valid slots %ld, flags %u, result %s (%d)\n", T, H, E, R, k,
                valid, flags, bad ? "MISMATCH" : "ok", bad);

    API(moe_hook_destroy(hook));
    HIPCHK(hipStreamDestroy(s2));
    void* bufs_to_free[] = {x, idx, w, send, recv, out, cnt_e, cnt_r, in_rank, h.pos, h.expert_offsets,
                            h.rank_offsets, h.send_src_idx, h.recv_src_idx, h.recv_counts, gx, gy, gw};
    for (void* p : bufs_to_free) HIPCHK(hipFree(p));
    HIPCHK(hipStreamDestroy(s));
    API(moe_ctx_destroy(ctx));
    return bad ? 1 : 0;
}
