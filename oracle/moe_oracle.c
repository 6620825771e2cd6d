/*
 * moe_oracle.c -- plain, slow, obviously correct CPU oracle for MoE token
 * dispatch-layout / dispatch / combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or constant
 * generator with the HIP path.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (scalar code, no SIMD
 * intrinsics, no OpenMP).  -ffp-contract=off keeps every float multiply and add
 * separately rounded to IEEE binary32, which is what the combine definition
 * below asks for.
 *
 * Sources (the method's definition):
 *  - "DeepEP cross-node optimisation guide" (cyqw.cn), opening paragraph: the
 *    library's all-to-all GPU kernels are MoE dispatch and combine, with FP8
 *    support.  Same page, "Core API example": dispatch takes hidden_states,
 *    topk_idx, num_max_dispatch_tokens_per_rank and num_experts; combine takes
 *    expert outputs, topk_idx, topk_weights, the dispatch handle and
 *    num_experts.  Same page, "Core advantages / low-latency kernels": the
 *    production setting is 128 tokens per batch, hidden 7168, top-8 experts,
 *    FP8 dispatch and BF16 combine.  Same page, figure caption under
 *    "Technical analysis": layout information is computed once and reused.
 *    Same page, "Performance tuning": fixed-size buffers instead of queues.
 *  - "DeepTech: DeepSeek open-sources DeepEP" (010bt.com), feature list: expert
 *    parallelism places different experts on different nodes; dispatch and
 *    combine are the all-to-all kernels; native FP8 dispatch.
 *  The pages give no formulas.  Where they are silent the readings used are the
 *  plainest ones (expert e lives on rank e / (E/R); rows are ordered stably by
 *  token index then top-k slot; FP8 is OCP E4M3FN with one fp32 scale per 128
 *  channels of a token row; combine accumulates in fp32 over slots in
 *  ascending order and rounds once to bf16 with round-to-nearest-even).
 *
 * Parity pins: every function here is pinned by tests/test_oracle_pins.py
 * against closed forms, textbook library routines and brute force.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

/* ------------------------------------------------------------------------ */
/* bf16 codec.  bf16 is the top half of an IEEE binary32 (1 sign, 8 exponent,
 * 7 mantissa bits).  Decode is exact.  Encode rounds to nearest, ties to even
 * on the 16 dropped bits; NaN stays NaN (quiet bit forced on). */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

float orc_bf16_to_f32(uint16_t b) { return bits_f32((uint32_t)b << 16); }

uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u = f32_bits(f);
    if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t upper = u >> 16;          /* truncated result */
    uint32_t lower = u & 0xFFFFu;      /* dropped bits */
    /* above the halfway point, or exactly halfway with an odd kept part: round up.
       A carry out of the mantissa correctly bumps the exponent (max -> Inf). */
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
    return (uint16_t)upper;
}

/* ------------------------------------------------------------------------ */
/* OCP FP8 E4M3FN codec: 1 sign, 4 exponent (bias 7), 3 mantissa bits.
 *   exponent field 0       : subnormal, value = m/8 * 2^-6
 *   exponent field 1..15   : normal,    value = (1 + m/8) * 2^(e-7)
 *   0x7F and 0xFF          : NaN (the only non-finite codes; no infinities)
 * Largest finite magnitude is 0x7E = 1.75 * 2^8 = 448. */

float orc_e4m3_to_f32(uint8_t q)
{
    int s = (q >> 7) & 1, e = (q >> 3) & 15, m = q & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp((double)m / 8.0, -6)
                          : ldexp(1.0 + (double)m / 8.0, e - 7);
    return (float)(s ? -mag : mag);
}

/* Encode a binary32 value: round to the nearest E4M3 value, ties to the even
 * mantissa, saturating to +-448 (a value that would round past 448 -- i.e.
 * |v| >= 464, the midpoint to the next binade -- becomes 448).  NaN -> 0x7F
 * with the input's sign bit.  The sign of zero (and of values that round to
 * zero) is kept. */
uint8_t orc_f32_to_e4m3(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v)) return (uint8_t)(sign | 0x7F);
    double a = fabs((double)v);
    if (a >= 464.0) return (uint8_t)(sign | 0x7E);

    /* spacing of representable values around a: 2^-9 in the subnormal range
       (below 2^-6), else 2^(floor(log2 a) - 3) */
    double quantum;
    if (a < ldexp(1.0, -6)) {
        quantum = ldexp(1.0, -9);
    } else {
        int ex;
        frexp(a, &ex);                   /* a = f * 2^ex, f in [0.5, 1) */
        quantum = ldexp(1.0, (ex - 1) - 3);
    }
    double n = a / quantum;              /* exact: power-of-two division */
    double r = nearbyint(n);             /* default mode: nearest, ties to even */
    double q = r * quantum;              /* the rounded magnitude, exactly */

    if (q == 0.0) return sign;
    if (q < ldexp(1.0, -6)) {            /* subnormal code: m = q / 2^-9 in 1..7 */
        int m = (int)(q / ldexp(1.0, -9));
        return (uint8_t)(sign | m);
    }
    int ex;
    double f = frexp(q, &ex);            /* q = f * 2^ex, f in [0.5, 1) */
    int e = (ex - 1) + 7;                /* biased exponent field */
    int m = (int)((2.0 * f - 1.0) * 8.0);
    return (uint8_t)(sign | (e << 3) | m);
}

/* vector helpers for the tests */
void orc_f32_to_e4m3_n(const float* v, int64_t n, uint8_t* out)
{ for (int64_t i = 0; i < n; i++) out[i] = orc_f32_to_e4m3(v[i]); }
void orc_e4m3_to_f32_n(const uint8_t* q, int64_t n, float* out)
{ for (int64_t i = 0; i < n; i++) out[i] = orc_e4m3_to_f32(q[i]); }
void orc_f32_to_bf16_n(const float* v, int64_t n, uint16_t* out)
{ for (int64_t i = 0; i < n; i++) out[i] = orc_f32_to_bf16(v[i]); }
void orc_bf16_to_f32_n(const uint16_t* b, int64_t n, float* out)
{ for (int64_t i = 0; i < n; i++) out[i] = orc_bf16_to_f32(b[i]); }

/* ------------------------------------------------------------------------ */
/* Step 1, dispatch layout.  Expert parallelism puts expert e on virtual rank
 * e / (E/R) (DeepTech release article, the paragraph defining EP).  For every
 * token t and slot j with a valid expert id e = topk_idx[t, j]:
 *   num_tokens_per_expert[e]   += 1
 *   is_token_in_rank[t, e/El]   = 1
 * and num_tokens_per_virtual_rank[r] is the number of tokens with
 * is_token_in_rank[t, r] = 1.  id -1 marks an empty slot; any other id outside
 * [0, E) is counted as an error and otherwise treated like -1.
 * Returns the number of such bad ids. */
int64_t orc_layout(const int64_t* topk_idx, int64_t T, int k, int E, int R,
                   int32_t* num_tokens_per_expert, int32_t* num_tokens_per_rank,
                   uint8_t* is_token_in_rank)
{
    int El = E / R;
    int64_t bad = 0;
    for (int e = 0; e < E; e++) num_tokens_per_expert[e] = 0;
    for (int r = 0; r < R; r++) num_tokens_per_rank[r] = 0;
    for (int64_t t = 0; t < T; t++)
        for (int r = 0; r < R; r++) is_token_in_rank[t * R + r] = 0;

    for (int64_t t = 0; t < T; t++) {
        for (int j = 0; j < k; j++) {
            int64_t e = topk_idx[t * k + j];
            if (e == -1) continue;
            if (e < -1 || e >= E) { bad++; continue; }
            num_tokens_per_expert[e] += 1;
            is_token_in_rank[t * R + e / El] = 1;
        }
    }
    for (int64_t t = 0; t < T; t++)
        for (int r = 0; r < R; r++)
            num_tokens_per_rank[r] += is_token_in_rank[t * R + r];
    return bad;
}

/* ------------------------------------------------------------------------ */
/* Step 2, offsets and stable positions.
 *   expert_offsets = exclusive prefix sum of num_tokens_per_expert (E+1)
 *   rank_offsets   = exclusive prefix sum of num_tokens_per_virtual_rank (R+1)
 * Walking tokens in index order, and within a token its slots in order:
 *   pos[t, j]  = expert_offsets[e] + (number of earlier (t', j') routed to e)
 *   spos[t, r] = rank_offsets[r] + (number of earlier tokens sent to rank r)
 *   recv_src[pos[t, j]] = t,  send_src[spos[t, r]] = t
 * pos / spos are -1 where the slot is empty or the token does not go to r.
 * Low-latency (padded) layout, when M > 0: the receiving rank keeps, per local
 * expert, cap = M * R fixed slots; this GPU, as source rank s0, owns slots
 * [s0*M, s0*M + M) ("fixed-size buffers instead of queues", guide's
 * "Performance tuning").  The slot of (t, j) is s0*M + (its rank among the
 * rows for expert e), and pos_ll[t, j] = e * cap + slot indexes the padded
 * buffer viewed as [E, cap, row] (rank-major then local-expert, because
 * e = r * El + local).  The caller ensures T <= M; a row whose rank among
 * expert e's rows is M or more (only possible when a token repeats an
 * expert) has no slot: pos_ll = -1 (it is not placed), and *ll_overflow
 * counts such rows.  The other outputs describe the routing and do not change.
 * Returns N_send (the number of send rows), or -1 if out of host memory;
 * *n_pairs gets N_pairs. */
int64_t orc_positions(const int64_t* topk_idx, int64_t T, int k, int E, int R,
                      const int32_t* num_tokens_per_expert,
                      const int32_t* num_tokens_per_rank,
                      const uint8_t* is_token_in_rank,
                      int32_t* expert_offsets, int32_t* rank_offsets,
                      int32_t* pos, int32_t* spos,
                      int32_t* send_src, int32_t* recv_src,
                      int64_t M, int s0, int32_t* pos_ll, int64_t* n_pairs,
                      int64_t* ll_overflow)
{
    expert_offsets[0] = 0;
    for (int e = 0; e < E; e++) expert_offsets[e + 1] = expert_offsets[e] + num_tokens_per_expert[e];
    rank_offsets[0] = 0;
    for (int r = 0; r < R; r++) rank_offsets[r + 1] = rank_offsets[r] + num_tokens_per_rank[r];

    int32_t* ce = (int32_t*)calloc((size_t)E, sizeof(int32_t));   /* running per-expert counters */
    int32_t* cr = (int32_t*)calloc((size_t)R, sizeof(int32_t));   /* running per-rank counters */
    if (ce == NULL || cr == NULL) { free(ce); free(cr); return -1; }
    int64_t cap = M * (int64_t)R;
    int64_t overflow = 0;

    for (int64_t t = 0; t < T; t++) {
        for (int j = 0; j < k; j++) {
            int64_t e = topk_idx[t * k + j];
            int32_t p = -1, pl = -1;
            if (e >= 0 && e < E) {
                int32_t rank_in_expert = ce[e]++;
                p = expert_offsets[e] + rank_in_expert;
                recv_src[p] = (int32_t)t;
                /* low latency: this source's window of expert e holds M slots
                   (fixed-size buffers of num_max_dispatch_tokens_per_rank rows);
                   a row past it is not placed.  With distinct experts per token
                   and T <= M this cannot happen; a token that repeats an expert
                   can make it happen. */
                if (M > 0) {
                    if (rank_in_expert < M) pl = (int32_t)(e * cap + (int64_t)s0 * M + rank_in_expert);
                    else overflow++;
                }
            }
            pos[t * k + j] = p;
            if (M > 0) pos_ll[t * k + j] = pl;
        }
        for (int r = 0; r < R; r++) {
            int32_t sp = -1;
            if (is_token_in_rank[t * R + r]) {
                sp = rank_offsets[r] + cr[r]++;
                send_src[sp] = (int32_t)t;
            }
            spos[t * R + r] = sp;
        }
    }
    free(ce);
    free(cr);
    *n_pairs = expert_offsets[E];
    if (ll_overflow) *ll_overflow = overflow;
    return rank_offsets[R];
}

/* ------------------------------------------------------------------------ */
/* FP8 quantisation of one token row (kdjingpai tutorial, "Function 3: FP8
 * operation optimisation"; guide's production setting "FP8 dispatch").  For
 * each block of 128 consecutive channels:
 *   a    = max |x_i|                       (x_i decoded from bf16 exactly)
 *   a'   = max(a, 1e-4)                    (floor: an all-zero block stays finite)
 *   s    = 448 / a'        (binary32, correctly rounded)
 *   sinv = a' / 448        (binary32, correctly rounded; stored dequant scale)
 *   q_i  = E4M3(x_i * s)   (binary32 product, then RNE saturating encode)
 * H must be a multiple of 128. */
void orc_quant_row(const uint16_t* x, int H, uint8_t* q, float* scales)
{
    for (int b = 0; b < H / 128; b++) {
        float a = 0.0f;
        for (int i = 0; i < 128; i++) {
            float v = fabsf(orc_bf16_to_f32(x[b * 128 + i]));
            if (v > a) a = v;
        }
        float ap = a > 1e-4f ? a : 1e-4f;
        float s = 448.0f / ap;
        float sinv = ap / 448.0f;
        for (int i = 0; i < 128; i++) {
            float prod = orc_bf16_to_f32(x[b * 128 + i]) * s;
            q[b * 128 + i] = orc_f32_to_e4m3(prod);
        }
        scales[b] = sinv;
    }
}

void orc_quant_rows(const uint16_t* x, int64_t nrows, int H, uint8_t* q, float* scales)
{
    for (int64_t r = 0; r < nrows; r++)
        orc_quant_row(x + r * H, H, q + r * H, scales + r * (H / 128));
}

/* ------------------------------------------------------------------------ */
/* Step 3, dispatch payload.  Every destination row is a copy of its source
 * token's payload: the bf16 row itself, or its FP8 codes plus per-block
 * scales.  The send buffer is rank-major (rows [rank_offsets[r],
 * rank_offsets[r+1]) go to rank r), the receive buffer expert-major; row i
 * of each holds token send_src[i] / recv_src[i].  With one GPU the transfer
 * to peer ranks is this local copy.
 * quant = 0: bf16 rows of H uint16 (scales unused, may be NULL).
 * quant = 1: fp8 rows of H bytes plus H/128 fp32 scales.
 * send_rows may be NULL (low-latency mode writes only the receive side). */
void orc_dispatch_rows(const uint16_t* x, int H, int quant,
                       const int32_t* send_src, int64_t n_send,
                       const int32_t* recv_src, int64_t n_pairs,
                       void* send_rows, float* send_scales,
                       void* recv_rows, float* recv_scales)
{
    int nb = H / 128;
    for (int pass = 0; pass < 2; pass++) {
        const int32_t* src = pass == 0 ? send_src : recv_src;
        int64_t n = pass == 0 ? n_send : n_pairs;
        void* rows = pass == 0 ? send_rows : recv_rows;
        float* scales = pass == 0 ? send_scales : recv_scales;
        if (rows == NULL) continue;
        for (int64_t i = 0; i < n; i++) {
            const uint16_t* xr = x + (int64_t)src[i] * H;
            if (quant == 0) {
                uint16_t* out = (uint16_t*)rows + i * H;
                for (int h = 0; h < H; h++) out[h] = xr[h];
            } else {
                orc_quant_row(xr, H, (uint8_t*)rows + i * H, scales + i * nb);
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Step 4, combine (guide's "Core API example": combine takes expert outputs,
 * topk_weights and the dispatch handle; production setting "BF16 combine").
 *   out[t, h] = bf16_rne( sum over valid j, in ascending j, of
 *                         w[t, j] * y[pos[t, j], h] )
 * Accumulation starts at +0.0f; each product and each sum is rounded to
 * binary32 separately (no fused multiply-add).  Empty slots (pos = -1)
 * contribute nothing; a token with no valid slot gets +0. */
void orc_combine(const uint16_t* y, int H, const float* w, const int32_t* pos,
                 int64_t T, int k, uint16_t* out)
{
    for (int64_t t = 0; t < T; t++) {
        for (int h = 0; h < H; h++) {
            float acc = 0.0f;
            for (int j = 0; j < k; j++) {
                int32_t p = pos[t * k + j];
                if (p < 0) continue;
                float prod = w[t * k + j] * orc_bf16_to_f32(y[(int64_t)p * H + h]);
                acc = acc + prod;
            }
            out[t * H + h] = orc_f32_to_bf16(acc);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Backward pass.  The DeepTech release article's feature list names
 * high-throughput kernels for training; training needs the gradients of
 * dispatch and combine.  The pages give no formulas for them, so these are the
 * derivatives of the forward definitions above:
 *  - dispatch copies x[t] into receive row pos[t, j] for every valid slot j;
 *    the adjoint of that copy adds the gradients of those rows back into
 *    token t.  FP8 quantisation is passed through as the identity (its codes
 *    times the stored scale reproduce x up to rounding).
 *  - combine is linear in the expert outputs and in the weights:
 *    d out[t] / d y[pos[t, j]] = w[t, j] and d out[t] / d w[t, j] =
 *    y[pos[t, j]].  Its final bf16 rounding is passed through as the identity.
 * Gradients travel in bf16 like the forward combine's inputs and outputs. */

/* Dispatch backward:
 *   grad_x[t, h] = bf16_rne( sum over valid j, ascending, of g[pos[t, j], h] )
 * summed in binary32 from +0, one addition at a time (the forward combine's
 * accumulation with every weight equal to one).  Empty slots contribute
 * nothing; a token with no valid slot gets +0. */
void orc_dispatch_backward(const uint16_t* g, int H, const int32_t* pos,
                           int64_t T, int k, uint16_t* grad_x)
{
    for (int64_t t = 0; t < T; t++) {
        for (int h = 0; h < H; h++) {
            float acc = 0.0f;
            for (int j = 0; j < k; j++) {
                int32_t p = pos[t * k + j];
                if (p >= 0) acc = acc + orc_bf16_to_f32(g[(int64_t)p * H + h]);
            }
            grad_x[t * H + h] = orc_f32_to_bf16(acc);
        }
    }
}

/* Combine backward, with go = the gradient of combine's output [T, H]:
 *   grad_y[pos[t, j], h] = bf16_rne( w[t, j] * go[t, h] ) for every valid slot,
 *       the product rounded to binary32 first, as in the forward combine;
 *       rows of grad_y that no slot points at are not written.
 *   grad_w[t, j] = sum over h of go[t, h] * y[pos[t, j], h], 0 for an empty
 *       slot.  Each product of two bf16 values is exact in binary64 and the
 *       sum is taken in binary64, so the result is the exact dot product to
 *       within H * 2^-53 of the sum of |terms|. */
void orc_combine_backward(const uint16_t* go, const float* w, const uint16_t* y,
                          const int32_t* pos, int64_t T, int k, int H,
                          uint16_t* grad_y, double* grad_w)
{
    for (int64_t t = 0; t < T; t++) {
        for (int j = 0; j < k; j++) {
            int32_t p = pos[t * k + j];
            if (p < 0) {
                grad_w[t * k + j] = 0.0;
                continue;
            }
            double dot = 0.0;
            for (int h = 0; h < H; h++) {
                float gv = orc_bf16_to_f32(go[t * H + h]);
                float prod = w[t * k + j] * gv;
                grad_y[(int64_t)p * H + h] = orc_f32_to_bf16(prod);
                dot += (double)gv * (double)orc_bf16_to_f32(y[(int64_t)p * H + h]);
            }
            grad_w[t * k + j] = dot;
        }
    }
}
