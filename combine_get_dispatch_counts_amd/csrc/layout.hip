// layout.hip -- the get_dispatch_layout kernel.
//
// [P2] "DeepEP 学习笔记" (DeepEP study notes), "dispatch 前：全局布局与通知":
// per-expert and per-rank counts and is_token_in_rank from topk_idx, then
// prefix sums into channel_prefix_matrix. [P1] "事件驱动 EP 内核的调度策略与
// 零拷贝通信", "事件驱动调度的本质": count locally, prefix-sum the offsets.
// [P2] "DeepEP v2": a token counts once per destination rank.
//
// One launch, deterministic results, one hand-over between blocks. The
// kernel is latency-bound (a few hundred KB of input), so it is built to
// keep every phase short rather than to save work:
//   - The tokens are cut into tiles of 256 (512 for large batches) and each
//     tile into `subs` parts; block (tile, part) writes the output rows of
//     its part, so the row writes are spread over many compute units. Each
//     block loads and counts its whole tile, one thread per token.
//   - Counting is one non-returning LDS OR per entry and per rank: each
//     wave ORs its lanes into per-expert and per-rank bitmaps (the OR over a
//     token's entries deduplicates ranks; an expert repeated in a row adds
//     to a separate per-wave count instead). A count is a popcount of a
//     bitmap, a token's rank in its wave a popcount of the bits below it,
//     and the earlier waves' counts give the rest of the tile's prefix.
//   - Part 0 of each tile publishes the tile's E + R counts; every block
//     writes its is_token_in_rank rows (they need only the rank bits), then
//     loads the words of all earlier tiles at once, spread over all of its
//     threads (tile-major, so the loads are coalesced; words still stale are
//     loaded again together), and adds them into LDS; one more block does
//     the same over all tiles for the totals,
//     and writes the counts, offsets and totals while the tiles write rows.
//     A batch of one tile needs no hand-over: its part 0 writes the totals
//     from its own counts and the workspace is not touched.
// A wave in which some token lists one expert twice counts earlier entries
// one by one instead, so a slot stays "entries before (t,k)" exactly.
#include "layout_device.h"

namespace epx {
namespace {

constexpr int kLThreads = 512;     // threads per block
constexpr int kMaxTileWaves = 8;   // counting waves of the largest tile (512 tokens)
// published words in flight per thread (fewer with the long top-k rows,
// whose registers are needed elsewhere)
template <int KMAX>
constexpr int kReadBatch = KMAX <= 8 ? 24 : 8;

// LDS of a block whose tile has cw counting waves: rank bits per token,
// per-wave expert bitmaps, rank masks and expert counts, per-wave exclusive
// prefixes, and per column (E + R) the tile's counts, the earlier tiles'
// counts and the offsets.
__host__ __device__ inline size_t layout_lds_bytes(int E, int R, int cw)
{
    const size_t ER = (size_t)E + R;
    return sizeof(uint64_t) * ((size_t)cw * kWave + (size_t)cw * E + (size_t)cw * R) +
           sizeof(int) * ((size_t)cw * E + (size_t)cw * ER + 3 * ER + 2);
}

// Entries before (tile token tt, slot k) inside tt's wave that route to e,
// counted one by one: the path for a wave in which some row repeats an
// expert (kept out of line so the common path stays small).
__device__ __noinline__ int wave_rank_slow(const LayoutArgs &a, int tile_base, int tt, int k,
                                           int e)
{
    const int64_t *base = a.topk_idx + (int64_t)(tile_base + (tt & ~63)) * a.K;
    const int upto = (tt & 63) * a.K + k;
    int n = 0;
    for (int i = 0; i < upto; ++i)
        n += (base[i] == e);
    return n;
}

// Add the published words of tiles [0, ntiles) into acc[0..ER) (LDS, zeroed
// before), every thread of the block loading its share of the ntiles * ER
// words in tile-major order, B at a time; the words that do not yet carry
// the tag are loaded again together until they all do. Returns false if a
// word stayed unpublished too long.
template <int B>
__device__ bool add_tile_words(const uint64_t *pub, int ER, int ntiles, uint32_t tag, int *acc)
{
    const int n = ntiles * ER, step = (int)blockDim.x;
    // column of word i0 + q * step: c0 + q * sr, wrapped into [0, ER)
    const int sr = step % ER;
    for (int i0 = threadIdx.x; i0 < n; i0 += B * step) {
        const int c0 = i0 % ER;
        uint32_t pending = 0;  // this batch's words still to add
#pragma unroll
        for (int q = 0; q < B; ++q)
            pending |= (i0 + q * step < n) ? 1u << q : 0u;
        for (int polls = 0;; ++polls) {
            uint64_t wv[B];
#pragma unroll
            for (int q = 0; q < B; ++q)
                wv[q] = i0 + q * step < n ? pub_load(pub + i0 + q * step) : 0;
            int c = c0;
#pragma unroll
            for (int q = 0; q < B; ++q) {
                if ((uint32_t)(wv[q] >> 32) == tag && ((pending >> q) & 1u)) {
                    atomicAdd(&acc[c], (int)(uint32_t)wv[q]);
                    pending &= ~(1u << q);
                }
                c += sr;
                c = c >= ER ? c - ER : c;
            }
            if (!pending)
                break;
            if (polls >= kSpinLimit)
                return false;
            __builtin_amdgcn_s_sleep(2);
        }
    }
    return true;
}

template <int KMAX>
__global__ __launch_bounds__(kLThreads) void layout_kernel(LayoutArgs a)
{
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int E = a.E, R = a.R, ER = E + R;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int tt_n = a.tile_tokens, cw = tt_n / kWave;  // tile tokens, counting waves
    uint64_t *rb = reinterpret_cast<uint64_t *>(lds);   // [tt_n]
    uint64_t *emask = rb + tt_n;                         // [cw][E]
    uint64_t *rmask = emask + (size_t)cw * E;            // [cw][R]
    int *ecnt = reinterpret_cast<int *>(rmask + (size_t)cw * R);  // [cw][E]
    int *wpre = ecnt + (size_t)cw * E;  // [cw][E + R] counts of the tile's earlier waves
    int *agg = wpre + (size_t)cw * ER;  // [E + R] this tile's counts (totals block: all)
    int *pre = agg + ER;                // [E + R] counts of the earlier tiles
    int *off = pre + ER;                // [E + R + 2] offsets
    __shared__ uint32_t s_tag;
    __shared__ int s_go, s_dup[kMaxTileWaves];

    if (a.ntiles == 0) {  // T = 0: zero counts and offsets, no tiles
        for (int i = tid; i < ER; i += blockDim.x)
            agg[i] = 0;
        __syncthreads();
        write_totals(a, agg, off);
        if (a.channel_prefix)
            for (int i = tid; i < R * a.C; i += blockDim.x)
                a.channel_prefix[i] = 0;
        return;
    }
    const bool handover = a.ntiles > 1;
    unsigned long long head = 0;
    unsigned int arrival = 0;
    if (handover && tid == 0)
        head = load_call(a.hdr);

    // the totals block (there is one only with a hand-over): every tile's
    // published counts
    if ((int)blockIdx.x == a.ntiles * a.subs) {
        if (tid == 0) {
            uint32_t tag;
            s_go = enter_call(a.hdr, head, &tag, &arrival);
            s_tag = tag;
        }
        for (int c = tid; c < ER; c += blockDim.x)
            agg[c] = 0;
        __syncthreads();
        const bool ok = s_go && add_tile_words<kReadBatch<KMAX>>(a.pub, ER, a.ntiles, s_tag, agg);
        if (__syncthreads_or(!ok)) {
            if (tid == 0)
                flag_error(a.err, EPX_DEV_WORKSPACE);
        } else {
            write_totals(a, agg, off);
        }
        if (tid == 0)
            close_call(a.hdr, arrival);
        return;
    }

    const int tile = (int)blockIdx.x / a.subs, part = (int)blockIdx.x - tile * a.subs;
    const int tile_base = tile * tt_n;
    const int ntok = min(tt_n, a.T - tile_base);
    const int per = tt_n / a.subs;
    const int p_lo = part * per, p_hi = min(p_lo + per, ntok);  // this block's tile tokens
    const bool counter = tid < tt_n;
    int ek[KMAX];
    load_row_experts<KMAX>(a, counter ? tile_base + tid : a.T, ek);  // -1 past the last token
    if (handover && tid == 0) {  // after the tile's loads are out
        uint32_t tag;
        s_go = enter_call(a.hdr, head, &tag, &arrival);
        s_tag = tag;
    }

    for (int i = tid; i < cw * E; i += blockDim.x) {
        emask[i] = 0;
        ecnt[i] = 0;
    }
    for (int i = tid; i < cw * R; i += blockDim.x)
        rmask[i] = 0;
    for (int c = tid; c < ER; c += blockDim.x) {
        agg[c] = 0;
        pre[c] = 0;
    }
    __syncthreads();

    // count the tile: per expert every entry (bitmap of lanes and count),
    // per rank every token once (a ballot per rank)
    uint64_t rbits = 0;
    if (counter) {
        const uint64_t bit = 1ull << lane;
        int dup = 0, bad = 0;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const int e = ek[k];
            bad |= (e == -2);
            int rep = 0;  // e already listed earlier in the row
#pragma unroll
            for (int k2 = 0; k2 < k; ++k2)
                rep |= (e >= 0 && ek[k2] == e);
            dup |= rep;
            if (e >= 0) {
                if (rep)  // the lane's bit is already set: the repeat is counted apart
                    __hip_atomic_fetch_add(&ecnt[w * E + e], 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_WORKGROUP);
                else
                    __hip_atomic_fetch_or(reinterpret_cast<unsigned long long *>(&emask[w * E + e]),
                                          bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                rbits |= 1ull << div_by_magic(e, a.L_mul);
            }
        }
        rb[tid] = rbits;
        if (bad && part == 0)
            flag_error(a.err, EPX_DEV_BAD_ROUTE);
        for (uint64_t m = rbits; m; m &= m - 1) {
            const int r = __builtin_ctzll(m);
            __hip_atomic_fetch_or(reinterpret_cast<unsigned long long *>(&rmask[w * R + r]), bit,
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        const uint64_t anydup = uniform64(__ballot(dup));
        if (lane == 0)
            s_dup[w] = anydup != 0;
    }
    __syncthreads();

    // per column the earlier waves' prefixes and the tile's count (a wave's
    // count: its lanes' bits plus the repeats), which part 0 publishes at once
    const uint32_t tag = s_tag;
    const bool go = !handover || s_go;
    const bool publish = handover && go && part == 0;
    const uint64_t hi = (uint64_t)tag << 32;
    uint64_t *prow = a.pub + (int64_t)tile * ER;
    for (int c = tid; c < ER; c += blockDim.x) {
        int run = 0;
        for (int w2 = 0; w2 < cw; ++w2) {
            wpre[w2 * ER + c] = run;
            run += c < E ? __popcll(emask[w2 * E + c]) + ecnt[w2 * E + c]
                         : __popcll(rmask[w2 * R + (c - E)]);
        }
        agg[c] = run;
        if (publish)
            pub_store(prow + c, hi | (uint32_t)run);
    }

    // is_token_in_rank rows of this block's tokens (contiguous: written as
    // blocks, 16 bytes per thread per step where R allows); they need only
    // the rank bits, so they go out before the wait for the earlier tiles
    const int nt = p_hi - p_lo;
    const int64_t row0 = (int64_t)(tile_base + p_lo) * R;
    if ((R & 15) == 0) {
        const int nq = R >> 4;
        Walk it(tid, blockDim.x, nq);
        for (int q = tid; q < nt * nq; q += blockDim.x, it.next())
            *reinterpret_cast<u32x4 *>(a.is_token_in_rank + row0 + (int64_t)q * 16) =
                rank_bytes16(rb[p_lo + it.row] >> (it.col * 16));
    } else {
        Walk it(tid, blockDim.x, R);
        for (int i = tid; i < nt * R; i += blockDim.x, it.next())
            a.is_token_in_rank[row0 + i] = (uint8_t)((rb[p_lo + it.row] >> it.col) & 1ull);
    }

    // the earlier tiles' counts (a batch of one tile: its own are the totals)
    bool ok = go;
    if (!handover) {
        if (part == 0) {
            __syncthreads();
            write_totals(a, agg, off);
        }
    } else if (ok && tile > 0) {
        ok = add_tile_words<kReadBatch<KMAX>>(a.pub, ER, tile, tag, pre);
    }
    if (__syncthreads_or(!ok)) {
        if (tid == 0)
            flag_error(a.err, EPX_DEV_WORKSPACE);
    } else {
        // slot_in_expert of this block's tokens: their own counting threads
        if (counter && tid >= p_lo && tid < p_hi) {
            const int t = tile_base + tid;
            int32_t *sie = a.slot_in_expert + (int64_t)t * a.K;
            const uint64_t below = lanes_below(lane);
            const bool slow = s_dup[w];
            int v[KMAX];
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                const int e = ek[k];
                v[k] = -1;
                if (e >= 0)
                    v[k] = pre[e] + wpre[w * ER + e] +
                           (slow ? wave_rank_slow(a, tile_base, tid, k, e)
                                 : __popcll(emask[w * E + e] & below));
            }
            if ((a.K & 3) == 0) {
#pragma unroll
                for (int k0 = 0; k0 < KMAX; k0 += 4)
                    if (k0 < a.K)
                        *reinterpret_cast<u32x4 *>(sie + k0) =
                            u32x4{(uint32_t)v[k0], (uint32_t)v[k0 + 1], (uint32_t)v[k0 + 2],
                                  (uint32_t)v[k0 + 3]};
            } else {
#pragma unroll
                for (int k = 0; k < KMAX; ++k)
                    if (k < a.K)
                        sie[k] = v[k];
            }
        }

        // pos_in_rank rows of this block's tokens are contiguous: written
        // as blocks, 16 bytes per thread per step where R allows
        if ((R & 3) == 0) {
            const int nq = R >> 2;
            Walk it(tid, blockDim.x, nq);
            for (int q = tid; q < nt * nq; q += blockDim.x, it.next()) {
                const int r0 = it.col * 4, tt = p_lo + it.row;
                const int ww = tt >> 6;
                const uint64_t rbt = rb[tt], below = lanes_below(tt & 63);
                int v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = r0 + j;
                    v[j] = ((rbt >> r) & 1ull) ? pre[E + r] + wpre[ww * ER + E + r] +
                                                     __popcll(rmask[ww * R + r] & below)
                                               : -1;
                }
                *reinterpret_cast<u32x4 *>(a.pos_in_rank + row0 + (int64_t)q * 4) =
                    u32x4{(uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]};
            }
        } else {
            Walk it(tid, blockDim.x, R);
            for (int i = tid; i < nt * R; i += blockDim.x, it.next()) {
                const int r = it.col, tt = p_lo + it.row, ww = tt >> 6;
                a.pos_in_rank[row0 + i] =
                    ((rb[tt] >> r) & 1ull)
                        ? pre[E + r] + wpre[ww * ER + E + r] +
                              __popcll(rmask[ww * R + r] & lanes_below(tt & 63))
                        : -1;
            }
        }

        // channel_prefix columns whose channel ends in this block's tokens
        if (a.channel_prefix && nt > 0) {
            const int64_t span = ((int64_t)a.T + a.C - 1) / a.C;
            const int64_t lo = tile_base + p_lo, hi_t = tile_base + p_hi;
            const int c0 = (int)(lo / span);
            const int c1 = hi_t == a.T ? a.C - 1 : (int)(hi_t / span) - 1;
            const int nc = c1 - c0 + 1;
            Walk it(tid, blockDim.x, nc > 0 ? nc : 1);
            for (int i = tid; i < R * nc && nc > 0; i += blockDim.x, it.next()) {
                const int r = it.row, c = c0 + it.col;
                const int n = (int)(channel_end(a, c) - tile_base);  // tile tokens before the end
                int v = pre[E + r];
                for (int w2 = 0; w2 < cw && n > w2 * kWave; ++w2) {
                    const uint64_t m = n >= (w2 + 1) * kWave ? ~0ull : lanes_below(n - w2 * kWave);
                    v += __popcll(rmask[w2 * R + r] & m);
                }
                a.channel_prefix[(int64_t)r * a.C + c] = v;
            }
        }
    }
    if (handover && tid == 0)
        close_call(a.hdr, arrival);
}

}  // namespace

// Tokens per tile: 256, or 512 for batches above 4096 tokens while the
// per-wave tables of a 512-token tile stay small (E <= 256), so that the
// number of tiles -- and of published words every block reads -- stays
// small.
int layout_tile_tokens(int T, int E)
{
    return (T > 4096 && E <= 256) ? 2 * kLayoutTile : kLayoutTile;
}

size_t layout_workspace_bytes(int T, int E, int R)
{
    // sized for 256-token tiles, which the fused kernel uses; the layout
    // kernel's tiles are never smaller
    const size_t ntiles = ((size_t)T + kLayoutTile - 1) / kLayoutTile;
    if (ntiles == 0)
        return 0;
    return sizeof(LayoutHdr) + ntiles * (size_t)(E + R) * sizeof(uint64_t);
}

// Parts per tile: the row writes of a tile spread over several blocks
// (64-token parts of a 256-token tile, 128-token parts of a 512-token
// tile) while the tiles alone are few; beyond 32 tiles one block per tile
// (every block reads the earlier tiles' words, whose number grows with the
// blocks). Measured: T = 4096 / 16384 take 10.8 / 15.0 us in 4 parts
// against 11.6 / 17.5 in one; 29 811 received rows (59 tiles of 512, E = 8,
// R = 1) take 12.2 us in one part against 13.8 in 4.
int layout_parts(int T, int tile_tokens)
{
    const int ntiles = (T + tile_tokens - 1) / tile_tokens;
    if (ntiles <= 1)
        return T <= 0 ? 1 : (T + 63) / 64;
    return ntiles <= 32 ? 4 : 1;
}

template <int KMAX>
static void launch_layout_k(const LayoutArgs &a, hipStream_t stream)
{
    LayoutArgs b = a;
    b.tile_tokens = layout_tile_tokens(a.T, a.E);
    b.ntiles = (a.T + b.tile_tokens - 1) / b.tile_tokens;
    b.subs = layout_parts(a.T, b.tile_tokens);
    // the tiles' blocks, plus one block for the totals when tiles hand over
    const int blocks = b.ntiles == 0 ? 1 : b.ntiles * b.subs + (b.ntiles > 1 ? 1 : 0);
    hipLaunchKernelGGL((layout_kernel<KMAX>), dim3(blocks), dim3(kLThreads),
                       layout_lds_bytes(a.E, a.R, b.tile_tokens / kWave), stream, b);
}

// The per-token top-k loops are unrolled to KMAX; the common K <= 8 gets a
// small kernel (instruction fetch matters for a short, few-block kernel).
hipError_t launch_layout(const LayoutArgs &a, hipStream_t stream)
{
    if (a.K <= 8)
        launch_layout_k<8>(a, stream);
    else
        launch_layout_k<EPX_MAX_TOPK>(a, stream);
    return hipGetLastError();
}

}  // namespace epx
