/*
 * epx.h -- C ABI of libepx: the single-GPU hot path of DeepEP-style MoE
 * expert-parallel dispatch / combine, written for AMD MI355X (gfx950).
 *
 * Sources (the three web pages the method is taken from):
 *   [P1] "事件驱动 EP 内核的调度策略与零拷贝通信：从 DeepEP 看高性能并发架构设计"
 *        (event-driven EP kernel scheduling and zero-copy communication)
 *   [P2] "DeepEP 学习笔记：MoE 场景下的专家并行通信" (DeepEP study notes)
 *   [P3] "DeepSeek DeepEP探索：低延迟分发（low latency dispatch）的架构设计与实现"
 *        (DeepEP low-latency dispatch)
 *
 * One GPU owns T tokens. Destination "ranks" are logical partitions of the
 * expert set: rank r holds experts [r*L, (r+1)*L) with L = E / R. Nothing
 * here talks to another GPU.
 *
 * Conventions shared by every call
 *   - Pointers are device memory unless a comment says "host". Every array is
 *     dense row-major. The caller allocates and owns every buffer; no call
 *     allocates device memory (epx_create allocates the context's error word
 *     and a 512-byte ring of launch stamps).
 *   - bf16 data is passed as uint16 bit patterns; FP8 data as uint8 codes in
 *     OCP E4M3FN (max 448, no infinities).
 *   - Hidden-state buffers (x, send_x, recv_x, ll_x, expert_out, out) and the
 *     per-token layout tables (is_token_in_rank, pos_in_rank, slot_in_expert)
 *     must be 16-byte aligned; h must be a multiple of 8 (of 128 with FP8).
 *   - Every call only enqueues work on `stream` and returns; none waits for
 *     the GPU, except epx_get_error. Work is ordered by the stream alone.
 *   - Host-detectable errors are returned at once and nothing is launched.
 *     Errors only the kernels can see (a top-k entry outside [-1, E), a row
 *     beyond the caller's capacity, a handle row outside the expert-output
 *     buffer) set bits in the context's device error word; read and clear
 *     them with epx_get_error. After such an error the outputs of that call
 *     are unspecified, but no write lands outside a buffer's stated size.
 *   - Results are deterministic: no atomics decide an order, so two runs on
 *     the same inputs give identical bytes.
 */
#ifndef EPX_H
#define EPX_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes */
#define EPX_OK 0
#define EPX_EINVAL (-1)       /* bad shape, parameter, null or misaligned pointer */
#define EPX_ECAPACITY (-2)    /* T > cap (low-latency), or workspace too small */
#define EPX_EUNSUPPORTED (-3) /* FP8 requested with h % 128 != 0 */
#define EPX_EHIP (-4)         /* a HIP runtime call or kernel launch failed */
#define EPX_EDEVICE (-5)      /* epx_get_error: the device error word was set */

/* Bits of the device error word */
#define EPX_DEV_BAD_ROUTE 1   /* a top-k entry outside [-1, E) */
#define EPX_DEV_OVERFLOW 2    /* a row index reached the caller's capacity */
#define EPX_DEV_BAD_HANDLE 4  /* a combine handle row >= n_rows */
#define EPX_DEV_WORKSPACE 8   /* the layout workspace was not zeroed before its
                                 first use, or is shared by overlapping calls */

/* Limits of this implementation */
#define EPX_MAX_TOPK 32
#define EPX_MAX_EXPERTS 512
#define EPX_MAX_RANKS 64
#define EPX_MAX_SWEEP_GBPS 100000
#define EPX_NOALLOC_SCRATCH_BYTES (1u << 20) /* see epx_get_dispatch_layout_noalloc */

typedef struct epx_ctx epx_ctx;

/* Context: binds a device and owns its device error word and the stamps of
 * its paced launches (epx_set_sweep_rate). [P2] "Buffer 与内存视角" /
 * "内存生命周期": a Buffer is built once, used by every call and destroyed at
 * the end; here it holds no communication state (there is no peer).
 * `device` is a HIP device ordinal; the calls below must be issued with that
 * device current. Returns EPX_EINVAL for a bad ordinal, EPX_EHIP if the
 * context's device memory cannot be allocated. */
int epx_create(epx_ctx **out, int device);
int epx_destroy(epx_ctx *ctx);
const char *epx_strerror(int code);

/* Rate of the paced store sweep of the high-throughput dispatch
 * (epx_dispatch, epx_dispatch_fused), in GB/s of destination rows, for bf16
 * rows and for FP8 rows (codes plus scale row); 0 turns pacing off. Pacing
 * changes when each row is stored, never what is stored: outputs are
 * identical at every rate. When every token's wave is on the device at once
 * (the fused call's one-launch shapes; epx_dispatch while T fits the device),
 * each wave stores its token's rows in ascending order of their place in
 * the output -- send rows, then receive rows -- and holds a row back until
 * its byte offset in that order, at this rate, has elapsed since the start
 * of the wave's schedule (below). The waves' stores then move through the
 * output as one front, which HBM absorbs at sequential-write speed, where
 * the same rows in routing order arrive as random writes. A larger epx_dispatch is launched
 * as chunks of consecutive tokens that each fit, each sweeping its own rows
 * at 93% of the rate. Left unpaced: the permute alone (epx_dispatch with
 * send_x = NULL), which reads as many rows as it writes; a call whose row
 * bound (T*(K + min(K,R)) rows) is at most 320 MiB for bf16 or 128 MiB for
 * FP8 (such rows mostly stay in the memory-side cache during the launch, and
 * the pacing delay would cost more than the ordering saves); rows of more
 * than 8192 channels (stored one register pass at a time). A rate above
 * what the memory sustains lets the front spread back toward random order
 * (in one launch measured no slower than unpaced); a lower one leaves
 * bandwidth idle. Late waves: a paced launch's first block stamps its start,
 * and a wave that starts more than an eighth of the launch's longest sweep
 * (at least 4, at most 16 microseconds) after it -- a wave that found no
 * place until others ended, e.g. beside kernels of other streams, or when
 * the device holds fewer waves than its occupancy query reported -- stores
 * its rows unpaced instead of waiting for times already past, so such a
 * wave costs at most that much plus its own unpaced stores (outputs are
 * unaffected either way). A wave's schedule starts when it is ready but no
 * earlier than a fixed time after its entry -- 1 us (bf16 dispatch), 3 us
 * (FP8 dispatch) or 9 us (the fused launch, whose waves first wait for the
 * layout hand-over) plus the time the launch's x rows take at its rate --
 * so the launch's front starts sharp. Defaults, measured on MI355X: 6450
 * (bf16) and 6400 (FP8);
 * epx_calibrate_sweep_rate derives them from the device instead. The
 * setting is per context and read at each call. EPX_EINVAL for a NULL
 * context or a rate outside [0, EPX_MAX_SWEEP_GBPS]. */
int epx_set_sweep_rate(epx_ctx *ctx, int bf16_gbps, int fp8_gbps);

/* The context's current sweep rates (host out), as epx_set_sweep_rate or
 * epx_calibrate_sweep_rate left them. EPX_EINVAL for a NULL argument. */
int epx_get_sweep_rate(epx_ctx *ctx, int *bf16_gbps, int *fp8_gbps);

/* Set the sweep rates from this device's own memory: times a sequential
 * fill of `scratch` (device memory of `bytes` >= 512 MiB, larger than the
 * memory-side cache, 16-byte aligned; its contents are overwritten) on
 * `stream` -- three untimed fills, then the median of nine -- and sets the
 * bf16 and FP8 rates to 93.3% and 90.4% of that fill rate (the ratios of
 * the defaults above to the fill rate of the GPU they were measured on).
 * *fill_gbps (host, may be NULL) receives the measured fill rate in GB/s.
 * Unlike every other call, this one waits for the stream; call it once,
 * outside any graph capture. EPX_EINVAL for a bad scratch, EPX_EHIP if a
 * launch or event fails (the rates are then left as they were). */
int epx_calibrate_sweep_rate(epx_ctx *ctx, void *scratch, size_t bytes, int *fill_gbps,
                             hipStream_t stream);

/* Workspace bytes epx_get_dispatch_layout needs for (T, K, E, R) (host out):
 * a 128-byte head plus 8 bytes per (256-token tile, expert or rank).
 * [P2] "Buffer 与内存视角": the workspace is allocated up front, once. */
int epx_workspace_size(int T, int K, int E, int R, size_t *bytes);

/* fp32 entries per row of every FP8 scale array (send_scales, recv_scales,
 * ll_scales) for hidden size h: the h/128 group scales rounded up to a
 * multiple of 32, so each row fills whole 128-byte lines; the kernels write
 * the padding entries as +0.0f. Row i's scales start at i * stride. Returns
 * 0 if h is not a positive multiple of 128. (Rows that end inside a line
 * would leave each line shared by two rows written at different times.) */
int epx_scale_stride(int h);

/* Bytes of a low-latency receive buffer for max_tokens_per_rank tokens per
 * source: E*R regions of max_tokens_per_rank rows (bf16: 2h bytes; fp8: h
 * bytes + epx_scale_stride(h) fp32 scales) plus one int32 source index per row and one
 * int32 count per region, each array rounded up to 128 bytes, the total
 * rounded up to a multiple of 128. [P3] 2.2: the size hint of the worst-case
 * layout, rounded to the buffer alignment. Returns 0 for bad arguments. */
size_t epx_ll_size_hint(int max_tokens_per_rank, int h, int R, int E, int fp8);

/* get_dispatch_layout + receive offsets. [P2] "dispatch 前：全局布局与通知"
 * (per-expert and per-rank token counts, is_token_in_rank, then prefix sums
 * into channel_prefix_matrix); [P1] "事件驱动调度的本质" (count locally,
 * prefix-sum the offsets); [P2] "DeepEP v2" (one copy per destination rank).
 *
 * In:  topk_idx [T,K] int64, each entry in [-1, E) (-1 = no route).
 *      1 <= K <= 32, 1 <= E <= 512, 1 <= R <= 64, E % R == 0, T >= 0.
 *      C >= 1 channels when channel_prefix != NULL (ignored otherwise).
 * Out: num_tokens_per_expert [E]   entries routed to each expert
 *      num_tokens_per_rank [R]     distinct tokens routed to each rank
 *      is_token_in_rank [T,R]      1 if token t goes to rank r, else 0
 *      rank_off [R+1], exp_off [E+1]   exclusive prefix sums of the counts
 *      pos_in_rank [T,R]           tokens before t in rank r, or -1
 *      slot_in_expert [T,K]        entries before (t,k) routed to the same
 *                                  expert in row-major (t,k) order, or -1
 *      channel_prefix [R,C]        optional: channel c owns tokens
 *                                  [c*ceil(T/C), min((c+1)*ceil(T/C), T));
 *                                  entry = tokens of rank r before its end
 *      totals [2]                  (rows of the rank-major send buffer,
 *                                   rows of the expert-major receive buffer)
 *      totals_host_mapped          optional host-pinned int32[2]
 *                                  (hipHostMalloc) that also receives totals;
 *                                  valid once the stream has been synchronised
 * ws:  device workspace of epx_workspace_size bytes (0 when T = 0): a
 *      call number and a block counter, then the per-tile counts that
 *      later tiles read for their prefix (tagged with the call number). Zero-fill it before its first use; every call leaves it
 *      ready for the next one (also across graph replays), so it is
 *      allocated and cleared once. Calls that share a workspace must not
 *      overlap. A workspace found in another state sets EPX_DEV_WORKSPACE,
 *      the call's outputs are not valid and the workspace must be
 *      zero-filled again; no wait inside the kernel is unbounded. */
int epx_get_dispatch_layout(epx_ctx *ctx, const int64_t *topk_idx, int T, int K, int E,
                            int R, int C, int32_t *num_tokens_per_expert,
                            int32_t *num_tokens_per_rank, uint8_t *is_token_in_rank,
                            int32_t *rank_off, int32_t *exp_off, int32_t *pos_in_rank,
                            int32_t *slot_in_expert, int32_t *channel_prefix,
                            int32_t *totals, int32_t *totals_host_mapped, void *ws,
                            size_t ws_bytes, hipStream_t stream);

/* epx_get_dispatch_layout with no workspace argument, for callers that
 * cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Arguments and outputs are those of
 * epx_get_dispatch_layout without ws / ws_bytes; nothing is allocated: the
 * workspace is a fixed array of EPX_NOALLOC_SCRATCH_BYTES bytes in device
 * memory that each GPU holds from the library's load until the process
 * ends, its address found once per device by epx_create. Each call first
 * clears the part it uses (a fill kernel on `stream`, so the pair may be
 * captured in a graph), so an earlier call's state, even one that set
 * EPX_DEV_WORKSPACE, never carries over. A shape whose workspace
 * (epx_workspace_size) exceeds the array returns EPX_ECAPACITY with nothing
 * launched: 1 MiB covers about 116 000 tokens at E = 256, R = 32. Every call
 * on one GPU shares the array: calls that overlap on one GPU (other
 * streams, other threads, other contexts) race and their outputs are not
 * valid. */
int epx_get_dispatch_layout_noalloc(epx_ctx *ctx, const int64_t *topk_idx, int T, int K, int E,
                                    int R, int C, int32_t *num_tokens_per_expert,
                                    int32_t *num_tokens_per_rank, uint8_t *is_token_in_rank,
                                    int32_t *rank_off, int32_t *exp_off, int32_t *pos_in_rank,
                                    int32_t *slot_in_expert, int32_t *channel_prefix,
                                    int32_t *totals, int32_t *totals_host_mapped,
                                    hipStream_t stream);

/* High-throughput dispatch: the rank-deduplicated pack and the local permute
 * into expert-contiguous blocks, reading x once. [P2] "dispatch 过程" (each
 * token is sent, in token order, to every rank is_token_in_rank marks, with
 * its source index, top-k indices and weights; the receiver writes at the
 * prefix offset); [P2] "DeepEP v2" (one full activation per destination
 * rank); [P1] "高吞吐量模式：协调阶段与紧凑缓冲区" (exact-size ragged
 * receive buffer, then a local permute into the per-expert blocks a grouped
 * GEMM reads); [P1] "低延迟模式" and [P2] "内存布局" (optional FP8 payload
 * with its scales).
 *
 * In:  x [T,h] bf16; topk_idx [T,K]; topk_w [T,K] fp32; the layout outputs
 *      rank_off, exp_off, pos_in_rank, slot_in_expert of the same topk_idx.
 *      fp8 = 0: rows are bf16 (2h bytes). fp8 = 1: rows are e4m3 codes
 *      (h bytes) plus fp32 scales [rows, epx_scale_stride(h)], of which the
 *      first h/128 are used: per token and per 128 channels, s = max(amax,
 *      1e-4) / 448 and q = e4m3(x / s), both IEEE fp32 divisions, rounded to
 *      nearest even (OCP E4M3FN, saturating to 448). amax is the largest
 *      magnitude that compares (a NaN never wins); a NaN quotient (x NaN,
 *      or +-Inf over an Inf scale) is coded 0x7F.
 * Out: send_x [send_cap_rows, h(*2)] rank-major: row rank_off[r] +
 *        pos_in_rank[t,r] holds token t for each rank r it goes to;
 *      send_scales [send_cap_rows, epx_scale_stride(h)] (fp8 only, else
 *        may be NULL; 16-byte aligned);
 *      send_src [rows] source token; send_topk_idx [rows,K] int64 local
 *        expert index (e - r*L) where expert e is on the row's rank, else -1;
 *      send_topk_w [rows,K] the weight there, else 0;
 *      recv_x [recv_cap_rows, ...] expert-major: row exp_off[e] +
 *        slot_in_expert[t,k] holds token t for each entry (t,k) with expert e;
 *      recv_scales (fp8, as send_scales), recv_src [rows] source token;
 *      pos_exp [T,K] the recv row of (t,k), or -1: the handle for combine.
 *      A row index >= its capacity is not written and sets
 *      EPX_DEV_OVERFLOW; totals from the layout call say what is needed.
 * send_x = NULL: the permute alone, no send buffer (send_*, topk_w,
 *      rank_off and pos_in_rank may then be NULL). This is the receiver's
 *      side of [P1] "高吞吐量模式": given its received rows as x and their
 *      local expert indices as topk_idx (E = local experts, R = 1, with a
 *      layout of those indices), it arranges them into per-expert blocks in
 *      row order. The rows are copied bit for bit, so FP8 payloads (codes,
 *      scales) can be passed as bf16 rows of half the width. */
int epx_dispatch(epx_ctx *ctx, const uint16_t *x, int h, const int64_t *topk_idx,
                 const float *topk_w, int T, int K, int E, int R, const int32_t *rank_off,
                 const int32_t *exp_off, const int32_t *pos_in_rank,
                 const int32_t *slot_in_expert, int fp8, void *send_x, float *send_scales,
                 int32_t *send_src, int64_t *send_topk_idx, float *send_topk_w,
                 int64_t send_cap_rows, void *recv_x, float *recv_scales,
                 int32_t *recv_src, int64_t recv_cap_rows, int32_t *pos_exp,
                 hipStream_t stream);

/* The receiver's local permute, in one launch. [P1] "高吞吐量模式：协调阶段
 * 与紧凑缓冲区": a destination receives exact-size rows from its sources
 * and arranges them locally into contiguous per-expert blocks for the
 * grouped GEMM. N received rows (row n: the token's payload, copied bit for
 * bit -- bf16 or FP8 codes alike) go, for each entry k of local_topk_idx
 * [N,K] (local expert index in [0, L), or -1 = the entry belongs to another
 * rank), to row exp_off[e] + slot_in_expert[n,k] of out_rows, where
 * exp_off / slot_in_expert come from epx_get_dispatch_layout over
 * local_topk_idx with E = L, R = 1 (rows in received order inside each
 * expert's block); a side row per received row (e.g. its FP8 scale row, 0
 * to 1024 bytes) travels with it to out_side.
 * In:  rows [N, row_bytes] (row_bytes a multiple of 16, at most 1 MiB),
 *      side [N, side_bytes] (side_bytes a multiple of 16, or 0: side and
 *      out_side may be NULL), both 16-byte aligned; 1 <= K <= 32,
 *      1 <= L <= 512.
 * Out: out_rows [cap_rows, row_bytes], out_side [cap_rows, side_bytes],
 *      src_row [cap_rows] (the received row each output row holds),
 *      pos [N,K] (the output row of (n,k), or -1). A row index outside
 *      [0, cap_rows) is not written and sets EPX_DEV_OVERFLOW; an entry
 *      outside [-1, L) sets EPX_DEV_BAD_ROUTE and is skipped. */
int epx_permute(epx_ctx *ctx, const void *rows, int row_bytes, const void *side, int side_bytes,
                const int64_t *local_topk_idx, int N, int K, int L, const int32_t *exp_off,
                const int32_t *slot_in_expert, void *out_rows, void *out_side,
                int32_t *src_row, int64_t cap_rows, int32_t *pos, hipStream_t stream);

/* Workspace bytes epx_dispatch_fused needs for (T, K, E, R) (host out): the
 * same as the layout's (epx_workspace_size), whose head and per-tile words
 * it uses. Zero-filled before its first use, like the layout's. */
int epx_fused_workspace_size(int T, int K, int E, int R, size_t *bytes);

/* get_dispatch_layout and the high-throughput dispatch in one launch. [P2]
 * "DeepEP v2": the v2 dispatch kernel computes is_token_in_rank itself
 * (notify warps in place of get_dispatch_layout) while its dispatch warps
 * move the data. Arguments and outputs are those of epx_get_dispatch_layout
 * (topk_idx, C, the counts, is_token_in_rank, offsets, pos_in_rank,
 * slot_in_expert, channel_prefix, totals, totals_host_mapped) followed by
 * those of epx_dispatch (x, h, topk_w, fp8 and every send / recv output;
 * send_x must not be NULL), with the same meaning, layout and errors; the
 * results are bit-identical to the two calls in sequence. ws: a workspace
 * of epx_fused_workspace_size bytes, zero-filled before its first use and
 * left ready by every call (after an EPX_DEV_WORKSPACE flag, zero it
 * again); calls that share it must not overlap, and it may be shared with
 * epx_get_dispatch_layout calls of any shape. The
 * capacities must be known up front (no host wait happens): T*min(K,R) send
 * rows and T*K receive rows always suffice. One launch for T <= 1024
 * (every block then computes the whole batch's layout itself and leaves the
 * workspace untouched), and for larger T while the tiled grid (ceil(T/8)
 * blocks of 512 threads) covers every compute unit and fits on the device
 * at once (at h = 7168 and 256 units: 2048 <= T <= 4096); else the layout
 * and the dispatch are launched one after the other (epx_fused_launches says
 * which; T = 0 is one launch). In the tiled one-launch form every block
 * waits for the per-tile counts that the first ceil(T/256) blocks publish:
 * work on other streams that holds the device for longer than the bounded
 * wait (a fraction of a second) makes the call set EPX_DEV_WORKSPACE
 * instead of hanging, and its outputs are then not valid. */
int epx_dispatch_fused(epx_ctx *ctx, const uint16_t *x, int h, const int64_t *topk_idx,
                       const float *topk_w, int T, int K, int E, int R, int C,
                       int32_t *num_tokens_per_expert, int32_t *num_tokens_per_rank,
                       uint8_t *is_token_in_rank, int32_t *rank_off, int32_t *exp_off,
                       int32_t *pos_in_rank, int32_t *slot_in_expert, int32_t *channel_prefix,
                       int32_t *totals, int32_t *totals_host_mapped, void *ws, size_t ws_bytes,
                       int fp8, void *send_x, float *send_scales, int32_t *send_src,
                       int64_t *send_topk_idx, float *send_topk_w, int64_t send_cap_rows,
                       void *recv_x, float *recv_scales, int32_t *recv_src,
                       int64_t recv_cap_rows, int32_t *pos_exp, hipStream_t stream);

/* How many launches epx_dispatch_fused takes for this shape on the
 * context's device (host out: 1 or 2, see above); arguments as there.
 * Nothing is launched. */
int epx_fused_launches(epx_ctx *ctx, int T, int h, int K, int E, int R, int fp8, int *launches);

/* Combine: reduce expert outputs back to source-token order. [P2] "combine
 * 过程" (route back through the handle, reduce per source token); [P1]
 * "低延迟模式" (combine stays BF16).
 * In:  expert_out [n_rows, h] bf16 (expert-major, or the low-latency layout);
 *      topk_w [T,K] fp32; pos [T,K] handle rows (pos_exp or pos_ll; < 0 =
 *      skip; >= n_rows sets EPX_DEV_BAD_HANDLE and is skipped).
 * Out: out [T,h] bf16: per column, acc = +0.0f, then for k = 0..K-1 over
 *      valid entries acc = fmaf(topk_w[t,k], expert_out[pos[t,k]], acc);
 *      the result is rounded to bf16, nearest even (NaN -> 0x7FC0). */
int epx_combine(epx_ctx *ctx, const uint16_t *expert_out, int64_t n_rows, int h,
                const float *topk_w, const int32_t *pos, int T, int K, uint16_t *out,
                hipStream_t stream);

/* Two-stage combine, stage 1: a rank-level partial result per rank-major
 * row. [P2] "DeepEP v2": combine returns a rank-level partial result -- a
 * token may get outputs from several experts of one rank, which that rank
 * reduces first -- and the source's epilogue reduces over the destination
 * ranks (stage 2, epx_combine_final).
 * In:  expert_out [n_rows, h] bf16, expert-major (the rows recv_x held);
 *      from epx_dispatch: send_src [send_cap_rows], send_topk_idx
 *      [send_cap_rows, K] (local expert index, or -1 for an entry on
 *      another rank), send_topk_w [send_cap_rows, K], pos_exp [T, K];
 *      num_send_rows: device int32 with the number of rank-major rows (the
 *      layout's totals[0]), or NULL if all send_cap_rows rows are in use.
 * Out: partial [send_cap_rows, h] bf16: row i < rows holds, per column, the
 *      fp32 chain acc = fmaf(send_topk_w[i,k], expert_out[pos_exp[t,k]],
 *      acc) over k ascending with send_topk_idx[i,k] >= 0, from +0.0f,
 *      t = send_src[i], rounded to bf16 nearest even (the bf16 a rank would
 *      send back). Rows past the count are not written. A send_src outside
 *      [0, T) (its row becomes +0) or a handle row >= n_rows (the entry is
 *      skipped) sets EPX_DEV_BAD_HANDLE. */
int epx_combine_partial(epx_ctx *ctx, const uint16_t *expert_out, int64_t n_rows, int h,
                        const int32_t *send_src, const int64_t *send_topk_idx,
                        const float *send_topk_w, const int32_t *pos_exp, int T, int K,
                        int64_t send_cap_rows, const int32_t *num_send_rows,
                        uint16_t *partial, hipStream_t stream);

/* Two-stage combine, stage 2 at the source. [P2] "DeepEP v2" (the epilogue
 * reduces over the destination ranks).
 * In:  partial [n_partial_rows, h] bf16 from epx_combine_partial; the
 *      layout outputs rank_off [R+1] and pos_in_rank [T, R].
 * Out: out [T, h] bf16: per column, acc = +0.0f, then acc = acc +
 *      partial[rank_off[r] + pos_in_rank[t,r]] for r ascending with
 *      pos_in_rank[t,r] >= 0 (fp32), rounded to bf16 nearest even. A row
 *      index >= n_partial_rows sets EPX_DEV_BAD_HANDLE and is skipped. */
int epx_combine_final(epx_ctx *ctx, const uint16_t *partial, int64_t n_partial_rows, int h,
                      const int32_t *rank_off, const int32_t *pos_in_rank, int T, int R,
                      uint16_t *out, hipStream_t stream);

/* Set n int32 counts to -1, the "nothing arrived" value. [P2] "Buffer 与内存
 * 视角" (counters start at -1); [P1] "低延迟模式" (the count slot starts
 * empty). A fill kernel, so it is safe inside a captured graph. */
int epx_ll_reset(epx_ctx *ctx, int32_t *ll_count, int64_t n, hipStream_t stream);

/* Low-latency fixed-slot dispatch in one launch, with no layout call and no
 * host round trip. [P1] "低延迟模式：固定缓冲区与信号槽机制" (each (source
 * rank, expert) pair owns a private region of `cap` rows at region index
 * expert * num_ranks + src_rank; the count slot is written after the data);
 * [P3] 4.2 (count index local_expert * num_ranks + src_rank); [P3] 2.2
 * (receive regions sized for the worst case, every token to one expert).
 *
 * In:  x [T,h] bf16; topk_idx [T,K]; this GPU's source rank src_rank in
 *      [0, R); cap >= T rows per region (else EPX_ECAPACITY, nothing
 *      launched); R_buf = R (all destinations' buffers side by side: region
 *      e*R + src_rank) or 1 (this source's slice only: region e);
 *      E * R_buf * cap must fit in int32. fp8 as in epx_dispatch.
 * Out: ll_x [E*R_buf*cap, h(*2)], ll_scales (fp8: [E*R_buf*cap,
 *      epx_scale_stride(h)], 16-byte aligned), ll_src [E*R_buf*cap]:
 *      entry (t,k) with expert e fills row region(e)*cap + slot, where slot
 *      counts entries before (t,k) routed to e (row-major order); other
 *      rows are not touched.
 *      ll_count [E*R_buf]: count[region(e)] = entries routed to e, for every
 *      e (0 included); counts of other sources' regions are not touched, so
 *      they keep what epx_ll_reset put there.
 *      pos_ll [T,K]: the row of (t,k), or -1: the handle for combine.
 * Ping-pong ([P2] "三个方法概览", low-latency mode: two buffers flipped by
 * XOR, reused with no allocation and no host wait):
 *      next_ll_count [n_next], if n_next > 0, is the other buffer's count
 *      array; this launch sets it to -1 so the next step can use that buffer
 *      without an epx_ll_reset. It must not overlap ll_count (EPX_EINVAL)
 *      and no reader of it may still be running.
 * Buffer fill ([P1] "工程实践：模式选择与监控要点": buffer utilisation, slots
 * used over slots available, in low-latency mode): ll_stats, if not
 *      NULL, is a device int32[2] that receives the entries routed by this
 *      source (the sum of its counts) and the largest count of any of its
 *      regions; utilisation = ll_stats[0] / (E * cap), peak region fill =
 *      ll_stats[1] / cap. */
int epx_ll_dispatch(epx_ctx *ctx, const uint16_t *x, int h, const int64_t *topk_idx,
                    int T, int K, int E, int R, int src_rank, int cap, int R_buf, int fp8,
                    void *ll_x, float *ll_scales, int32_t *ll_src, int32_t *ll_count,
                    int32_t *pos_ll, int32_t *next_ll_count, int64_t n_next,
                    int32_t *ll_stats, hipStream_t stream);

/* Synchronise `stream`, return the device error word in *device_flags (host)
 * and clear it. Returns EPX_EDEVICE if any bit was set, EPX_OK otherwise. */
int epx_get_error(epx_ctx *ctx, int *device_flags, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* EPX_H */
