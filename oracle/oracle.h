/*
 * oracle.h -- plain, sequential CPU definition of what one GPU computes in
 * DeepEP-style MoE expert-parallel dispatch / combine.
 *
 * TEST INFRASTRUCTURE. This library is the yardstick that the HIP kernels
 * are checked against. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load it; the product path never does. It shares no
 * code, header, table or helper with the HIP path.
 *
 * Sources (the three web pages this work follows):
 *   [P1] "事件驱动 EP 内核的调度策略与零拷贝通信：从 DeepEP 看高性能并发架构设计"
 *        (event-driven EP kernel scheduling and zero-copy communication)
 *   [P2] "DeepEP 学习笔记：MoE 场景下的专家并行通信" (DeepEP study notes)
 *   [P3] "DeepSeek DeepEP探索：低延迟分发（low latency dispatch）的架构设计与实现"
 *        (DeepEP low-latency dispatch)
 *
 * Conventions: every array is dense row-major; bf16 values travel as their
 * uint16 bit patterns; e4m3 values as uint8 (OCP E4M3FN). Integer results
 * are defined exactly; the only floating-point results are the FP8 scales
 * and codes (one IEEE fp32 division each) and the combine output (an fp32
 * fused-multiply-add chain in top-k order, rounded to bf16 to nearest even).
 *
 * Parity pins: every function here is pinned by the CPU tests (library
 * routines, closed forms, invariants, a hand-worked example, brute force).
 * No function is "parity unpinned".
 */
#ifndef EPX_ORACLE_H
#define EPX_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes; the numbering matches the product library's so tests can
 * compare error behaviour, but nothing is shared with it. */
#define ORC_OK 0
#define ORC_EINVAL (-1)      /* bad shape or parameter */
#define ORC_ECAPACITY (-2)   /* an output buffer is too small / T > cap */
#define ORC_EUNSUPPORTED (-3) /* FP8 with h % 128 != 0 */
#define ORC_EROUTE (-5)      /* a top-k entry outside [-1, E), or a handle row
                                outside the expert-output buffer */

/* Number conversions written from the format definitions. */
uint16_t orc_bf16_rne(float v);  /* fp32 -> bf16, nearest-even; NaN -> 0x7FC0 */
float orc_bf16_to_f32(uint16_t b);
uint8_t orc_e4m3_rne(float v);   /* fp32 -> OCP E4M3FN, nearest-even, saturating */
float orc_e4m3_to_f32(uint8_t q);
void orc_bf16_rne_n(const float *v, uint16_t *out, size_t n);
void orc_e4m3_rne_n(const float *v, uint8_t *out, size_t n);

/* Per-token FP8 quantisation of one bf16 row of h channels (h % 128 == 0):
 * q_row[h] codes and scales[h/128] dequantisation multipliers. */
void orc_quantize_row(const uint16_t *x_row, int h, uint8_t *q_row, float *scales);

/* get_dispatch_layout plus the receive-offset prefix sums ([P2] "dispatch
 * 前：全局布局与通知"; [P1] "事件驱动调度的本质", the coordination pass).
 * Inputs: topk_idx [T,K] (−1 = no route). L = E/R experts per rank; expert e
 * lives on rank e / L. Outputs (all required except channel_prefix):
 *   num_tokens_per_expert [E], num_tokens_per_rank [R],
 *   is_token_in_rank [T,R] (0/1), rank_off [R+1], exp_off [E+1],
 *   pos_in_rank [T,R] (−1 where the token does not go to the rank),
 *   slot_in_expert [T,K] (−1 for a −1 entry),
 *   channel_prefix [R,C] (may be NULL; C ignored then), totals [2]. */
int orc_layout(const int64_t *topk_idx, int T, int K, int E, int R, int C,
               int32_t *num_tokens_per_expert, int32_t *num_tokens_per_rank,
               uint8_t *is_token_in_rank, int32_t *rank_off, int32_t *exp_off,
               int32_t *pos_in_rank, int32_t *slot_in_expert,
               int32_t *channel_prefix, int32_t *totals);

/* High-throughput dispatch: rank-deduplicated pack, then the local permute
 * into expert-contiguous blocks. Layout inputs are orc_layout's outputs.
 * Row payload: bf16 (send_x / recv_x are uint16 [rows,h]) or, with fp8,
 * uint8 [rows,h] codes plus float [rows,h/128] scales.
 * send_cap_rows / recv_cap_rows: rows the caller provided. */
int orc_dispatch(const uint16_t *x, int h, const int64_t *topk_idx, const float *topk_w,
                 int T, int K, int E, int R,
                 const uint8_t *is_token_in_rank, const int32_t *rank_off,
                 const int32_t *exp_off, const int32_t *pos_in_rank,
                 const int32_t *slot_in_expert, int fp8,
                 void *send_x, float *send_scales, int32_t *send_src,
                 int64_t *send_topk_idx, float *send_topk_w, int64_t send_cap_rows,
                 void *recv_x, float *recv_scales, int32_t *recv_src,
                 int64_t recv_cap_rows, int32_t *pos_exp);

/* orc_dispatch for the tokens [t_begin, t_end) only (see oracle.c). */
int orc_dispatch_tokens(const uint16_t *x, int h, const int64_t *topk_idx, const float *topk_w,
                        int T, int K, int E, int R,
                        const uint8_t *is_token_in_rank, const int32_t *rank_off,
                        const int32_t *exp_off, const int32_t *pos_in_rank,
                        const int32_t *slot_in_expert, int fp8,
                        void *send_x, float *send_scales, int32_t *send_src,
                        int64_t *send_topk_idx, float *send_topk_w, int64_t send_cap_rows,
                        void *recv_x, float *recv_scales, int32_t *recv_src,
                        int64_t recv_cap_rows, int32_t *pos_exp, int t_begin, int t_end);

/* Low-latency fixed-slot dispatch ([P1] "低延迟模式：固定缓冲区与信号槽机制";
 * [P3] 4.2). Region rho = e*R + src_rank (R_buf == R, all destinations'
 * buffers side by side) or rho = e (R_buf == 1, this source's slice only);
 * row = rho*cap + slot. ll_count [E*R_buf] must be pre-filled with −1 by the
 * caller; this writes count[rho(e)] for every expert e (zeros included).
 * Rows the call does not address are left untouched. */
int orc_ll_dispatch(const uint16_t *x, int h, const int64_t *topk_idx,
                    int T, int K, int E, int R, int src_rank, int cap, int R_buf,
                    int fp8, void *ll_x, float *ll_scales, int32_t *ll_src,
                    int32_t *ll_count, int32_t *pos_ll);

/* Combine ([P2] "combine 过程"): out[t,c] = bf16_rne(fma chain over k of
 * topk_w[t,k] * expert_out[pos[t,k], c], from +0.0f, k ascending), skipping
 * entries with pos[t,k] < 0. */
int orc_combine(const uint16_t *expert_out, int64_t n_rows, int h,
                const float *topk_w, const int32_t *pos, int T, int K,
                uint16_t *out);

/* Two-stage combine ([P2] "DeepEP v2": a rank-level partial reduce, then a
 * final reduce over destination ranks at the source).
 * Stage 1: partial[i,c] = bf16_rne(fma chain, k ascending from +0.0f, over
 * k with send_topk_idx[i,k] >= 0, of send_topk_w[i,k] *
 * expert_out[pos_exp[send_src[i],k], c]) for each rank-major row i.
 * Stage 2: out[t,c] = bf16_rne(fp32 sum from +0.0f, ranks ascending, over r
 * with pos_in_rank[t,r] >= 0, of partial[rank_off[r] + pos_in_rank[t,r], c]). */
int orc_combine_partial(const uint16_t *expert_out, int64_t n_rows, int h,
                        const int32_t *send_src, const int64_t *send_topk_idx,
                        const float *send_topk_w, int64_t n_send,
                        const int32_t *pos_exp, int T, int K, uint16_t *partial);
int orc_combine_final(const uint16_t *partial, int64_t n_send, int h,
                      const int32_t *rank_off, const int32_t *pos_in_rank, int T, int R,
                      uint16_t *out);

#ifdef __cplusplus
}
#endif

#endif /* EPX_ORACLE_H */
