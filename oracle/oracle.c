/*
 * oracle.c -- plain sequential CPU definition of the single-GPU share of
 * DeepEP-style MoE dispatch / combine.
 *
 * TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's CPU
 * baseline load this; the product path never does. Written from the pages'
 * descriptions, step by step in the order they give, with no blocking,
 * fusion or reordering: the pack reads x, the permute reads the packed send
 * buffer (the pages' two-stage dataflow), the combine walks tokens and
 * columns with one fp32 accumulator.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off -fno-fast-math
 * (no contraction: the only fused multiply-adds are explicit fmaf calls, and
 * fp32 divisions are IEEE single-precision SSE divisions).
 *
 * Page titles are abbreviated as in oracle.h: [P1] event-driven EP kernel
 * scheduling / zero-copy; [P2] DeepEP study notes; [P3] DeepEP low-latency
 * dispatch.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Number formats                                                      */
/* ------------------------------------------------------------------ */

/* bf16 keeps the top 16 bits of an fp32 pattern. Round to nearest, ties to
 * the even kept pattern: add 0x7FFF plus the lowest kept bit, then truncate.
 * A NaN becomes the canonical quiet NaN 0x7FC0. */
uint16_t orc_bf16_rne(float v)
{
    uint32_t u;
    memcpy(&u, &v, sizeof u);
    if (isnan(v))
        return 0x7FC0;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

float orc_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float v;
    memcpy(&v, &u, sizeof v);
    return v;
}

/* OCP E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; no
 * infinities; S.1111.111 is NaN, so the largest finite magnitude is
 * 1.75 * 2^8 = 448. Normal numbers cover [2^-6, 448]; below 2^-6 the codes
 * are subnormal multiples of 2^-9 (code = value / 2^-9).
 * Rounding is to nearest, ties to even, done exactly in double precision
 * (rint in the default rounding mode is round-half-even). Magnitudes above
 * 464 -- the midpoint between 448 and the NaN pattern's value 480 --
 * saturate to 448; 464 itself ties to the even mantissa, i.e. 448.
 * The sign is kept (so -0 and negative underflow give 0x80); NaN gives 0x7F. */
uint8_t orc_e4m3_rne(float v)
{
    if (isnan(v))
        return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a > 464.0)
        return sign | 0x7E;
    if (a < 0x1p-6) {
        /* subnormal grid: q * 2^-9, q in 0..8; q == 8 is the smallest normal,
         * whose code 0x08 (exponent field 1, mantissa 0) equals q itself. */
        double q = rint(a * 512.0);
        return sign | (uint8_t)q;
    }
    int e2;
    double f = frexp(a, &e2);       /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;                 /* a = m * 2^E, m = 2f in [1, 2) */
    double m8 = rint(f * 16.0);     /* m with 3 fraction bits, times 8: 8..16 */
    if (m8 == 16.0) {               /* mantissa overflow carries into the exponent */
        m8 = 8.0;
        E += 1;
    }
    /* E is now in [-6, 8]; E == 8 with m8 == 15 cannot occur since a <= 464. */
    return sign | (uint8_t)(((E + 7) << 3) | ((int)m8 - 8));
}

/* Array forms of the two encoders (plain loops over the scalar definitions;
 * they exist so the tests can sweep millions of bit patterns quickly). */
void orc_bf16_rne_n(const float *v, uint16_t *out, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = orc_bf16_rne(v[i]);
}

void orc_e4m3_rne_n(const float *v, uint8_t *out, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = orc_e4m3_rne(v[i]);
}

float orc_e4m3_to_f32(uint8_t q)
{
    int s = q >> 7, ex = (q >> 3) & 0xF, m = q & 7;
    double v;
    if (ex == 0xF && m == 7)
        return NAN;
    if (ex == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, ex - 7);
    return (float)(s ? -v : v);
}

/* FP8 dispatch ([P1] "低延迟模式：固定缓冲区与信号槽机制": the payload is
 * quantised to FP8 before it is sent, combine stays in BF16; [P2] "内存布局":
 * the scales travel inside each token's payload). Granularity: one scale per
 * token per 128 contiguous channels. For group g:
 *   amax = max |x_i| (exact), a = max(amax, 1e-4f), s = a / 448 (IEEE fp32),
 *   q_i = e4m3_rne(x_i / s)  (one IEEE fp32 division per element),
 * and s is stored as the dequantisation multiplier (x_i ~ e4m3(q_i) * s). */
void orc_quantize_row(const uint16_t *x_row, int h, uint8_t *q_row, float *scales)
{
    for (int g = 0; g < h / 128; ++g) {
        const uint16_t *xg = x_row + (size_t)g * 128;
        float amax = 0.0f;
        for (int i = 0; i < 128; ++i) {
            float a = fabsf(orc_bf16_to_f32(xg[i]));
            if (a > amax)
                amax = a;
        }
        float a = fmaxf(amax, 1e-4f);
        float s = a / 448.0f;
        for (int i = 0; i < 128; ++i)
            q_row[(size_t)g * 128 + i] = orc_e4m3_rne(orc_bf16_to_f32(xg[i]) / s);
        scales[g] = s;
    }
}

/* ------------------------------------------------------------------ */
/* Layout and offsets                                                  */
/* ------------------------------------------------------------------ */

static int check_shape(int T, int K, int E, int R)
{
    if (T < 0 || K < 1 || E < 1 || R < 1 || E % R != 0)
        return ORC_EINVAL;
    return ORC_OK;
}

/* [P2] "dispatch 前：全局布局与通知": get_dispatch_layout yields how many
 * tokens each expert and each rank will receive and which ranks each token
 * goes to; notify_dispatch then turns counts into prefix offsets
 * (channel_prefix_matrix). [P1] "事件驱动调度的本质": count locally, then
 * prefix-sum the receive offsets. [P2] "DeepEP v2": one copy per destination
 * rank, so a token counts at most once per rank.
 *
 * Step order:
 *   1. scan t = 0..T-1, k = 0..K-1 (row-major): skip -1, reject e outside
 *      [0, E); count the entry for expert e; mark rank e/L for token t and
 *      count the token for that rank the first time only;
 *   2. exclusive prefix sums of the rank and expert counts;
 *   3. a second row-major scan hands out running per-rank and per-expert
 *      counters: pos_in_rank[t,r] = tokens before t in rank r, and
 *      slot_in_expert[t,k] = entries before (t,k) in expert e. With distinct
 *      experts per row this is "tokens before t routed to e";
 *   4. channel c owns tokens [c*ceil(T/C), min((c+1)*ceil(T/C), T)) ([P2]
 *      "dispatch 过程": channels split the tokens into contiguous ranges);
 *      channel_prefix[r,c] = tokens of rank r before the end of channel c. */
int orc_layout(const int64_t *topk_idx, int T, int K, int E, int R, int C,
               int32_t *num_tokens_per_expert, int32_t *num_tokens_per_rank,
               uint8_t *is_token_in_rank, int32_t *rank_off, int32_t *exp_off,
               int32_t *pos_in_rank, int32_t *slot_in_expert,
               int32_t *channel_prefix, int32_t *totals)
{
    int rc = check_shape(T, K, E, R);
    if (rc != ORC_OK)
        return rc;
    if (channel_prefix != NULL && C < 1)
        return ORC_EINVAL;
    const int L = E / R;

    /* 1. counts and the rank-membership table */
    for (int e = 0; e < E; ++e)
        num_tokens_per_expert[e] = 0;
    for (int r = 0; r < R; ++r)
        num_tokens_per_rank[r] = 0;
    memset(is_token_in_rank, 0, (size_t)T * R);
    for (int t = 0; t < T; ++t) {
        for (int k = 0; k < K; ++k) {
            int64_t e = topk_idx[(size_t)t * K + k];
            if (e == -1)
                continue;
            if (e < 0 || e >= E)
                return ORC_EROUTE;
            num_tokens_per_expert[e] += 1;
            int r = (int)(e / L);
            if (!is_token_in_rank[(size_t)t * R + r]) {
                is_token_in_rank[(size_t)t * R + r] = 1;
                num_tokens_per_rank[r] += 1;
            }
        }
    }

    /* 2. exclusive prefix sums (kept in 64 bits, then range-checked) */
    int64_t acc = 0;
    rank_off[0] = 0;
    for (int r = 0; r < R; ++r) {
        acc += num_tokens_per_rank[r];
        if (acc > INT32_MAX)
            return ORC_EINVAL;
        rank_off[r + 1] = (int32_t)acc;
    }
    const int64_t n_rank_rows = acc;
    acc = 0;
    exp_off[0] = 0;
    for (int e = 0; e < E; ++e) {
        acc += num_tokens_per_expert[e];
        if (acc > INT32_MAX)
            return ORC_EINVAL;
        exp_off[e + 1] = (int32_t)acc;
    }
    const int64_t n_exp_rows = acc;

    /* 3. running counters in scan order */
    int32_t *run_r = calloc((size_t)R, sizeof *run_r);
    int32_t *run_e = calloc((size_t)E, sizeof *run_e);
    if (!run_r || !run_e) {
        free(run_r);
        free(run_e);
        return ORC_EINVAL;
    }
    for (int t = 0; t < T; ++t) {
        for (int r = 0; r < R; ++r)
            pos_in_rank[(size_t)t * R + r] =
                is_token_in_rank[(size_t)t * R + r] ? run_r[r]++ : -1;
        for (int k = 0; k < K; ++k) {
            int64_t e = topk_idx[(size_t)t * K + k];
            slot_in_expert[(size_t)t * K + k] = (e == -1) ? -1 : run_e[e]++;
        }
    }
    free(run_r);
    free(run_e);

    /* 4. channel prefix matrix: inclusive per-rank counts at channel ends */
    if (channel_prefix != NULL) {
        const int64_t span = ((int64_t)T + C - 1) / C;
        for (int r = 0; r < R; ++r) {
            int64_t seen = 0, t = 0;
            for (int c = 0; c < C; ++c) {
                int64_t end = (c + 1) * span;
                if (end > T)
                    end = T;
                for (; t < end; ++t)
                    seen += is_token_in_rank[(size_t)t * R + r];
                channel_prefix[(size_t)r * C + c] = (int32_t)seen;
            }
        }
    }

    totals[0] = (int32_t)n_rank_rows;
    totals[1] = (int32_t)n_exp_rows;
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Row payloads                                                        */
/* ------------------------------------------------------------------ */

/* Bytes of one row's data part: bf16 = 2h, fp8 = h (scales kept apart). */
static size_t row_bytes(int h, int fp8) { return fp8 ? (size_t)h : (size_t)h * 2; }

/* Token t's payload: its bf16 row, or (fp8) its row quantised once into the
 * caller's scratch (q_tmp [h], s_tmp [h/128]); every destination gets a copy. */
static void token_payload(const uint16_t *x, int h, int fp8, int t, uint8_t *q_tmp,
                          float *s_tmp, const void **row, const float **scales)
{
    const uint16_t *xr = x + (size_t)t * h;
    if (fp8) {
        orc_quantize_row(xr, h, q_tmp, s_tmp);
        *row = q_tmp;
        *scales = s_tmp;
    } else {
        *row = xr;
        *scales = NULL;
    }
}

/* Copy row `src_row` of (src, src_scales) to row `dst_row` of (dst, dst_scales). */
static void copy_row(const void *src, const float *src_scales, int64_t src_row,
                     void *dst, float *dst_scales, int64_t dst_row, int h, int fp8)
{
    size_t rb = row_bytes(h, fp8);
    memcpy((uint8_t *)dst + (size_t)dst_row * rb,
           (const uint8_t *)src + (size_t)src_row * rb, rb);
    if (fp8)
        memcpy(dst_scales + (size_t)dst_row * (h / 128),
               src_scales + (size_t)src_row * (h / 128), sizeof(float) * (size_t)(h / 128));
}

/* ------------------------------------------------------------------ */
/* High-throughput dispatch                                            */
/* ------------------------------------------------------------------ */

/* Pack ([P2] "dispatch 过程": a channel's sender walks its tokens in order and
 * enqueues a token for a destination rank when is_token_in_rank hits; the
 * receiver places it at the prefix offset in recv_x; the payload carries x,
 * the source index, topk_idx and topk_weights. [P2] "DeepEP v2": one full
 * activation per destination rank, not one per expert.) Rank segment r holds
 * its tokens in ascending t at rows rank_off[r] + pos_in_rank[t,r]. Per-row
 * metadata: the source token, and the token's top-k list seen from rank r
 * (local expert index e - r*L and its weight for experts on r; -1 and 0.0f
 * for the others).
 *
 * Permute ([P1] "高吞吐量模式：协调阶段与紧凑缓冲区": the received data is
 * grouped by source rank and is rearranged locally into contiguous
 * per-expert blocks for the grouped GEMM; the receive buffer holds exactly
 * the received rows.) Expert e's block starts at exp_off[e]; entry (t,k) goes
 * to row exp_off[e] + slot_in_expert[t,k], copied from the packed row of
 * (t, rank of e). pos_exp[t,k] records that row (the handle combine reads);
 * -1 for a -1 entry. */
int orc_dispatch(const uint16_t *x, int h, const int64_t *topk_idx, const float *topk_w,
                 int T, int K, int E, int R,
                 const uint8_t *is_token_in_rank, const int32_t *rank_off,
                 const int32_t *exp_off, const int32_t *pos_in_rank,
                 const int32_t *slot_in_expert, int fp8,
                 void *send_x, float *send_scales, int32_t *send_src,
                 int64_t *send_topk_idx, float *send_topk_w, int64_t send_cap_rows,
                 void *recv_x, float *recv_scales, int32_t *recv_src,
                 int64_t recv_cap_rows, int32_t *pos_exp)
{
    return orc_dispatch_tokens(x, h, topk_idx, topk_w, T, K, E, R, is_token_in_rank, rank_off,
                               exp_off, pos_in_rank, slot_in_expert, fp8, send_x, send_scales,
                               send_src, send_topk_idx, send_topk_w, send_cap_rows, recv_x,
                               recv_scales, recv_src, recv_cap_rows, pos_exp, 0, T);
}

/* The same for the tokens [t_begin, t_end) only: their pack rows, then their
 * permute rows. Every row a token writes is fixed by the layout, and its
 * permute reads only rows its own pack wrote, so disjoint token ranges can
 * run side by side (the benchmark's threaded timing of the oracle does);
 * orc_dispatch is the range [0, T). */
int orc_dispatch_tokens(const uint16_t *x, int h, const int64_t *topk_idx, const float *topk_w,
                        int T, int K, int E, int R,
                        const uint8_t *is_token_in_rank, const int32_t *rank_off,
                        const int32_t *exp_off, const int32_t *pos_in_rank,
                        const int32_t *slot_in_expert, int fp8,
                        void *send_x, float *send_scales, int32_t *send_src,
                        int64_t *send_topk_idx, float *send_topk_w, int64_t send_cap_rows,
                        void *recv_x, float *recv_scales, int32_t *recv_src,
                        int64_t recv_cap_rows, int32_t *pos_exp, int t_begin, int t_end)
{
    int rc = check_shape(T, K, E, R);
    if (rc != ORC_OK)
        return rc;
    if (h < 1 || t_begin < 0 || t_end > T || t_begin > t_end)
        return ORC_EINVAL;
    if (fp8 && h % 128 != 0)
        return ORC_EUNSUPPORTED;
    if (rank_off[R] > send_cap_rows || exp_off[E] > recv_cap_rows)
        return ORC_ECAPACITY;
    const int L = E / R;

    uint8_t *q_tmp = fp8 ? malloc((size_t)h) : NULL;
    float *s_tmp = fp8 ? malloc(sizeof(float) * (size_t)(h / 128)) : NULL;
    if (fp8 && (!q_tmp || !s_tmp)) {
        free(q_tmp);
        free(s_tmp);
        return ORC_EINVAL;
    }

    /* pack: t ascending, then r ascending; an FP8 row is quantised once per token */
    for (int t = t_begin; t < t_end; ++t) {
        const void *payload;
        const float *pscales;
        token_payload(x, h, fp8, t, q_tmp, s_tmp, &payload, &pscales);
        for (int r = 0; r < R; ++r) {
            if (!is_token_in_rank[(size_t)t * R + r])
                continue;
            int64_t row = (int64_t)rank_off[r] + pos_in_rank[(size_t)t * R + r];
            copy_row(payload, pscales, 0, send_x, send_scales, row, h, fp8);
            send_src[row] = t;
            for (int k = 0; k < K; ++k) {
                int64_t e = topk_idx[(size_t)t * K + k];
                int on_r = (e != -1) && (e / L == r);
                send_topk_idx[(size_t)row * K + k] = on_r ? e - (int64_t)r * L : -1;
                send_topk_w[(size_t)row * K + k] = on_r ? topk_w[(size_t)t * K + k] : 0.0f;
            }
        }
    }

    /* permute: t ascending, then k ascending, reading the packed buffer */
    for (int t = t_begin; t < t_end; ++t) {
        for (int k = 0; k < K; ++k) {
            int64_t e = topk_idx[(size_t)t * K + k];
            if (e == -1) {
                pos_exp[(size_t)t * K + k] = -1;
                continue;
            }
            int r = (int)(e / L);
            int64_t src_row = (int64_t)rank_off[r] + pos_in_rank[(size_t)t * R + r];
            int64_t row = (int64_t)exp_off[e] + slot_in_expert[(size_t)t * K + k];
            copy_row(send_x, send_scales, src_row, recv_x, recv_scales, row, h, fp8);
            recv_src[row] = t;
            pos_exp[(size_t)t * K + k] = (int32_t)row;
        }
    }
    free(q_tmp);
    free(s_tmp);
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Low-latency fixed-slot dispatch                                     */
/* ------------------------------------------------------------------ */

/* [P1] "低延迟模式：固定缓冲区与信号槽机制": every (source rank, expert) pair
 * owns a fixed private region, so the sender computes the destination
 * address directly: region (expert * num_ranks + src_rank), times the region
 * capacity, plus the slot. After the data, the sender stores the number of
 * tokens it sent into the region's count slot, whose initial "empty" value
 * differs from every valid count. [P2] "Buffer 与内存视角": counters start
 * at -1, meaning nothing received. [P3] 4.2: the receiver reads the count at
 * index local_expert * num_ranks + src_rank -- the same region index inside
 * one destination, so concatenating all destinations' buffers gives the
 * global-expert form used here. [P3] 2.2: the receive side is sized for the
 * worst case, every token of a source reaching one expert, so T <= cap.
 *
 * Slots are handed out in scan order (t ascending, then k), exactly like
 * slot_in_expert. Counts are written for every expert, zeros included,
 * after all rows. */
int orc_ll_dispatch(const uint16_t *x, int h, const int64_t *topk_idx,
                    int T, int K, int E, int R, int src_rank, int cap, int R_buf,
                    int fp8, void *ll_x, float *ll_scales, int32_t *ll_src,
                    int32_t *ll_count, int32_t *pos_ll)
{
    int rc = check_shape(T, K, E, R);
    if (rc != ORC_OK)
        return rc;
    if (h < 1 || cap < 1 || src_rank < 0 || src_rank >= R || (R_buf != R && R_buf != 1))
        return ORC_EINVAL;
    if ((int64_t)E * R_buf * cap > INT32_MAX)
        return ORC_EINVAL;
    if (fp8 && h % 128 != 0)
        return ORC_EUNSUPPORTED;
    if (T > cap)
        return ORC_ECAPACITY;
    for (size_t i = 0; i < (size_t)T * K; ++i)
        if (topk_idx[i] < -1 || topk_idx[i] >= E)
            return ORC_EROUTE;

    /* with distinct experts per row a region gets at most T <= cap rows; a row
     * that repeats an expert could exceed that, which is a capacity error */
    int32_t *count = calloc((size_t)E, sizeof *count);
    if (!count)
        return ORC_EINVAL;
    for (size_t i = 0; i < (size_t)T * K; ++i)
        if (topk_idx[i] >= 0 && ++count[topk_idx[i]] > cap) {
            free(count);
            return ORC_ECAPACITY;
        }
    memset(count, 0, sizeof *count * (size_t)E);
    uint8_t *q_tmp = fp8 ? malloc((size_t)h) : NULL;
    float *s_tmp = fp8 ? malloc(sizeof(float) * (size_t)(h / 128)) : NULL;
    if (fp8 && (!q_tmp || !s_tmp)) {
        free(count);
        free(q_tmp);
        free(s_tmp);
        return ORC_EINVAL;
    }
    for (int t = 0; t < T; ++t) {
        const void *payload;
        const float *pscales;
        token_payload(x, h, fp8, t, q_tmp, s_tmp, &payload, &pscales);
        for (int k = 0; k < K; ++k) {
            int64_t e = topk_idx[(size_t)t * K + k];
            if (e == -1) {
                pos_ll[(size_t)t * K + k] = -1;
                continue;
            }
            int64_t region = (R_buf == 1) ? e : e * R + src_rank;
            int64_t slot = count[e]++;
            int64_t row = region * cap + slot;
            copy_row(payload, pscales, 0, ll_x, ll_scales, row, h, fp8);
            ll_src[row] = t;
            pos_ll[(size_t)t * K + k] = (int32_t)row;
        }
    }
    free(q_tmp);
    free(s_tmp);
    for (int e = 0; e < E; ++e) {
        int64_t region = (R_buf == 1) ? e : (int64_t)e * R + src_rank;
        ll_count[region] = count[e];
    }
    free(count);
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Combine                                                             */
/* ------------------------------------------------------------------ */

/* [P2] "combine 过程": the handle saved at dispatch routes each expert output
 * back to its source token, where the results are reduced; [P1] low-latency
 * section: combine stays in BF16. Reading used here: for token t and column
 * c, acc starts at +0.0f and takes acc = fmaf(w[t,k], y[pos[t,k], c], acc)
 * for k = 0..K-1 over entries whose handle row is valid (>= 0); the result
 * is rounded to bf16 to nearest even. */
int orc_combine(const uint16_t *expert_out, int64_t n_rows, int h,
                const float *topk_w, const int32_t *pos, int T, int K,
                uint16_t *out)
{
    if (T < 0 || K < 1 || h < 1 || n_rows < 0)
        return ORC_EINVAL;
    for (size_t i = 0; i < (size_t)T * K; ++i)
        if (pos[i] >= n_rows)
            return ORC_EROUTE;
    for (int t = 0; t < T; ++t) {
        for (int c = 0; c < h; ++c) {
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                int32_t p = pos[(size_t)t * K + k];
                if (p < 0)
                    continue;
                float y = orc_bf16_to_f32(expert_out[(size_t)p * h + c]);
                acc = fmaf(topk_w[(size_t)t * K + k], y, acc);
            }
            out[(size_t)t * h + c] = orc_bf16_rne(acc);
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Two-stage combine                                                   */
/* ------------------------------------------------------------------ */

/* [P2] "DeepEP v2": combine sends a rank-level partial result back to the
 * source, because one source token may get outputs from several experts of
 * the same rank; the rank reduces them first, and the source's epilogue
 * reduces over the destination ranks. Readings: the partial travels in
 * bf16 (combine stays BF16, [P1] "低延迟模式"), made by the same fp32 fma
 * chain as the one-stage combine (k ascending, from +0.0f) over the entries
 * of the row's rank; the final sum adds a token's partials in ascending
 * rank order in fp32 from +0.0f (the weights are already applied) and
 * rounds to bf16 nearest even.
 *
 * Stage 1, per rank-major row i (the send-buffer layout, token send_src[i]):
 * partial[i,c] = bf16_rne(fma chain over k with send_topk_idx[i,k] >= 0 of
 * send_topk_w[i,k] * expert_out[pos_exp[t,k], c]). */
int orc_combine_partial(const uint16_t *expert_out, int64_t n_rows, int h,
                        const int32_t *send_src, const int64_t *send_topk_idx,
                        const float *send_topk_w, int64_t n_send,
                        const int32_t *pos_exp, int T, int K, uint16_t *partial)
{
    if (T < 0 || K < 1 || h < 1 || n_rows < 0 || n_send < 0)
        return ORC_EINVAL;
    for (int64_t i = 0; i < n_send; ++i) {
        const int32_t t = send_src[i];
        if (t < 0 || t >= T)
            return ORC_EROUTE;
        for (int k = 0; k < K; ++k) {
            if (send_topk_idx[(size_t)i * K + k] < 0)
                continue;
            const int32_t p = pos_exp[(size_t)t * K + k];
            if (p < 0 || p >= n_rows)
                return ORC_EROUTE;
        }
    }
    for (int64_t i = 0; i < n_send; ++i) {
        const int32_t t = send_src[i];
        for (int c = 0; c < h; ++c) {
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                if (send_topk_idx[(size_t)i * K + k] < 0)
                    continue;
                const int32_t p = pos_exp[(size_t)t * K + k];
                const float y = orc_bf16_to_f32(expert_out[(size_t)p * h + c]);
                acc = fmaf(send_topk_w[(size_t)i * K + k], y, acc);
            }
            partial[(size_t)i * h + c] = orc_bf16_rne(acc);
        }
    }
    return ORC_OK;
}

/* Stage 2, per source token t: out[t,c] = bf16_rne(sum over ranks r
 * ascending with pos_in_rank[t,r] >= 0 of partial[rank_off[r] +
 * pos_in_rank[t,r], c]), fp32 adds from +0.0f. */
int orc_combine_final(const uint16_t *partial, int64_t n_send, int h,
                      const int32_t *rank_off, const int32_t *pos_in_rank, int T, int R,
                      uint16_t *out)
{
    if (T < 0 || R < 1 || h < 1 || n_send < 0)
        return ORC_EINVAL;
    for (size_t i = 0; i < (size_t)T * R; ++i) {
        if (pos_in_rank[i] < 0)
            continue;
        const int64_t row = (int64_t)rank_off[i % R] + pos_in_rank[i];
        if (row >= n_send)
            return ORC_EROUTE;
    }
    for (int t = 0; t < T; ++t) {
        for (int c = 0; c < h; ++c) {
            float acc = 0.0f;
            for (int r = 0; r < R; ++r) {
                const int32_t p = pos_in_rank[(size_t)t * R + r];
                if (p < 0)
                    continue;
                const int64_t row = (int64_t)rank_off[r] + p;
                acc = acc + orc_bf16_to_f32(partial[(size_t)row * h + c]);
            }
            out[(size_t)t * h + c] = orc_bf16_rne(acc);
        }
    }
    return ORC_OK;
}

