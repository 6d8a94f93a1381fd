// layout_device.h -- device code of get_dispatch_layout, shared by the
// layout kernel and the fused layout + dispatch kernel.
//
// [P2] "DeepEP 学习笔记" (DeepEP study notes), "dispatch 前：全局布局与通知":
// per-expert and per-rank counts and is_token_in_rank from topk_idx, then
// prefix sums (channel_prefix_matrix). [P1] "事件驱动 EP 内核的调度策略与零拷贝
// 通信", "事件驱动调度的本质": count locally, prefix-sum the offsets.
// [P2] "DeepEP v2": a token counts once per destination rank.
//
// One launch, deterministic results:
//   Block b handles tile b of 256 tokens (8 waves; two threads per token:
//   the first 256 count, all share the writes).
//   Workgroups are dispatched in index order, so a tile waits only for
//   tiles that are running or done; with a few hundred tiles they are all
//   resident at once anyway. Each wave ORs its lanes into LDS bitmaps:
//   emask[w][e] has bit l set when token l of wave w routes an entry to
//   expert e, rmask likewise per rank (the OR deduplicates ranks for free).
//   A token's rank inside the tile is the earlier waves' count plus
//   popcount(mask & lanes below it).
//   The tile then publishes its per-expert and per-rank counts and looks
//   back over the earlier tiles' published words for its prefix (a
//   decoupled look-back: a word carries the call's tag, an "inclusive" bit
//   and the value, so one 64-bit load reads all three). With the prefix the
//   block writes is_token_in_rank, pos_in_rank, slot_in_expert and its
//   channel_prefix columns once, in final form. One more block looks back
//   from past the last tile: that prefix is the totals, from which it
//   writes the counts, offsets and totals while the tiles write rows.
//   A 64-bit counter in the workspace (call number << 32 | blocks arrived)
//   gives every layout block (tiles and the totals block) the call's tag in
//   one atomic, issued beside the topk loads; the last of them to arrive
//   moves it on to the next call. (The fused launch takes no arrivals: its
//   blocks read the call number, and its last block to finish moves it
//   on.) Waits are bounded: a tile that waits too long flags
//   EPX_DEV_WORKSPACE and goes on, so the kernel always ends.
// A wave in which some token lists one expert twice counts earlier entries
// directly instead, so a slot stays "entries before (t,k)" exactly.
#pragma once

#include "epx_device.h"
#include "epx_internal.h"

namespace epx {
namespace {


constexpr int W = kLayoutWaves;

struct CountLds {
    uint64_t *rb;     // [kLayoutTile] rank bits of each token of the tile
    uint64_t *emask;  // [W][E]
    uint64_t *rmask;  // [W][R]
    int *ecnt;        // [W][E] entries of wave w routed to e
    int *wpre_e;      // [W][E] entries of the tile's earlier waves routed to e
    int *wpre_r;      // [W][R] tokens of the tile's earlier waves going to r
    int *dupwave;     // [W] 1 if the wave has a row with a repeated expert
};

__host__ __device__ inline size_t count_lds_bytes(int E, int R)
{
    return sizeof(uint64_t) * (kLayoutTile + (size_t)W * E + (size_t)W * R) +
           sizeof(int) * (2 * (size_t)W * E + (size_t)W * R + W);
}

__device__ CountLds carve_count(char *base, int E, int R)
{
    CountLds s;
    s.rb = reinterpret_cast<uint64_t *>(base);
    s.emask = s.rb + kLayoutTile;
    s.rmask = s.emask + (size_t)W * E;
    s.ecnt = reinterpret_cast<int *>(s.rmask + (size_t)W * R);
    s.wpre_e = s.ecnt + (size_t)W * E;
    s.wpre_r = s.wpre_e + (size_t)W * E;
    s.dupwave = s.wpre_r + (size_t)W * R;
    return s;
}

// After the count scratch: the tile's counts, its prefix and (last tile)
// the offsets, each E + R (+ 2) ints.
__host__ __device__ inline size_t layout_lds_bytes(int E, int R)
{
    return count_lds_bytes(E, R) + sizeof(int) * (3 * (size_t)(E + R) + 2);
}

// Published words: (tag << 32) | inclusive bit 31 | value (< 2^31). A word
// from an earlier call carries an older tag and reads as "not yet".
constexpr uint64_t kInclusive = 0x80000000ull;
constexpr int kSpinLimit = 1 << 18;

__device__ __forceinline__ void pub_store(uint64_t *p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t pub_load(const uint64_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One round of the look-back: the words of tiles j, j-1, .., j-B+1 of
// column c, loaded together (a tile index below 0 loads the reader's own
// row instead, so surplus loads do not pile onto the lines every tile
// reads), then summed from j down until a word is unpublished or carries an
// inclusive prefix. Returns how many words were consumed; *done is set when
// an inclusive prefix ended the walk.
template <int B>
__device__ __forceinline__ int look_back_round(const uint64_t *pub, int ER, int self, int j, int c,
                                               uint32_t tag, uint32_t &acc, bool &done)
{
    uint64_t w[B];
#pragma unroll
    for (int u = 0; u < B; ++u)
        w[u] = pub_load(pub + (int64_t)(j - u >= 0 ? j - u : self) * ER + c);
    int u = 0;
    for (; u < B && j - u >= 0; ++u) {
        if ((uint32_t)(w[u] >> 32) != tag)
            break;
        acc += (uint32_t)w[u] & 0x7FFFFFFFu;
        if (w[u] & kInclusive) {
            done = true;
            return u + 1;
        }
    }
    return u;
}

// Sum over tiles before `tile` of column c: walk back from tile - 1, adding
// aggregates until a tile's inclusive prefix ends the walk (a decoupled
// look-back). `self` is a row of the workspace that surplus loads may read
// (the reader's own tile row). Returns false if a word stayed unpublished
// too long.
__device__ bool look_back(const uint64_t *pub, int ER, int tile, int self, int c, uint32_t tag,
                          int *out)
{
    uint32_t acc = 0;
    int j = tile - 1, polls = 0;
    while (j >= 0) {
        bool done = false;
        const int batch = j < 4 ? 4 : 16;
        const int u = j < 4 ? look_back_round<4>(pub, ER, self, j, c, tag, acc, done)
                            : look_back_round<16>(pub, ER, self, j, c, tag, acc, done);
        if (done)
            break;
        j -= u;
        if (j >= 0 && u < batch) {  // stopped at an unpublished word: poll again
            if (++polls > kSpinLimit) {
                *out = (int)acc;
                return false;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    *out = (int)acc;
    return true;
}

// Flat index walker over a [rows, cols] row-major block: thread tid starts
// at element tid and steps by blockDim, tracking (row, col) with one
// division up front instead of one per element.
struct Walk {
    int row, col, drow, dcol, cols;
    __device__ Walk(int tid, int step, int ncols)
    {
        cols = ncols;
        row = tid / ncols;
        col = tid - row * ncols;
        drow = step / ncols;
        dcol = step - drow * ncols;
    }
    __device__ void next()
    {
        row += drow;
        col += dcol;
        if (col >= cols) {
            col -= cols;
            ++row;
        }
    }
};

// Load a token's K expert ids into ek (-1 = no route or k >= K, -2 = out of
// range). Loads go out 8 at a time from clamped, always-valid addresses and
// are masked afterwards, so they are in flight together. Needs T >= 1.
template <int KMAX>
__device__ __forceinline__ void load_row_experts(const LayoutArgs &a, int t, int (&ek)[KMAX])
{
    const int64_t *row = a.topk_idx + (int64_t)min(t, a.T - 1) * a.K;
#pragma unroll
    for (int k0 = 0; k0 < KMAX; k0 += 8) {
        if (k0 < a.K) {
            int64_t v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                v[j] = row[min(k0 + j, a.K - 1)];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t e = v[j];
                ek[k0 + j] = (k0 + j >= a.K || t >= a.T) ? -1
                             : (e >= 0 && e < a.E)      ? (int)e
                             : (e == -1 ? -1 : -2);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                ek[k0 + j] = -1;
        }
    }
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

// Entries before (tile token tt, slot k) inside tt's wave that route to e.
__device__ __forceinline__ int wave_rank(const LayoutArgs &a, const CountLds &s, int tile_base,
                                         int tt, int k, int e)
{
    const int w = tt >> 6;
    if (!s.dupwave[w])
        return __popcll(s.emask[w * a.E + e] & lanes_below(tt & 63));
    return wave_rank_slow(a, tile_base, tt, k, e);
}

// Bytes (0/1) for the low 16 bits of `bits`, one byte per bit.
__device__ __forceinline__ u32x4 rank_bytes16(uint64_t bits)
{
    uint32_t wd[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t nib = (uint32_t)(bits >> (4 * j)) & 0xFu;
        wd[j] = (nib & 1u) | ((nib & 2u) << 7) | ((nib & 4u) << 14) | ((nib & 8u) << 21);
    }
    return u32x4{wd[0], wd[1], wd[2], wd[3]};
}

// Row of R bytes (0/1) for one token, byte by byte (R not a multiple of 16).
__device__ void write_rank_row(uint8_t *dst, uint64_t rbits, int R)
{
    for (int r = 0; r < R; ++r)
        dst[r] = (uint8_t)((rbits >> r) & 1ull);
}

// Exclusive scan of in[0..n) into out[0..n] by one wave.
__device__ void wave_exclusive_scan(const int *in, int n, int *out)
{
    const int lane = lane_id();
    const int per = (n + kWave - 1) / kWave;
    const int lo = min(n, lane * per), hi = min(n, lo + per);
    int sum = 0;
    for (int i = lo; i < hi; ++i)
        sum += in[i];
    const int incl = wave_inclusive_sum(sum);
    int run = incl - sum;
    for (int i = lo; i < hi; ++i) {
        out[i] = run;
        run += in[i];
    }
    if (lane == kWave - 1)
        out[n] = incl;
}

// Channel c covers tokens [c*ceil(T/C), min((c+1)*ceil(T/C), T)); the tile
// holding its last token owns column c of channel_prefix.
__device__ __forceinline__ int64_t channel_end(const LayoutArgs &a, int c)
{
    const int64_t span = ((int64_t)a.T + a.C - 1) / a.C;
    return min((int64_t)(c + 1) * span, (int64_t)a.T);
}

// Counts, offsets and totals from the totals in tot[0..E+R), using off as
// scratch; one block.
__device__ void write_totals(const LayoutArgs &a, const int *tot, int *off)
{
    const int tid = threadIdx.x;
    if (tid < kWave)
        wave_exclusive_scan(tot, a.E, off);
    else if (tid < 2 * kWave)
        wave_exclusive_scan(tot + a.E, a.R, off + a.E + 1);
    __syncthreads();
    for (int e = tid; e < a.E; e += blockDim.x)
        a.num_tokens_per_expert[e] = tot[e];
    for (int r = tid; r < a.R; r += blockDim.x)
        a.num_tokens_per_rank[r] = tot[a.E + r];
    for (int i = tid; i <= a.E; i += blockDim.x)
        a.exp_off[i] = off[i];
    for (int i = tid; i <= a.R; i += blockDim.x)
        a.rank_off[i] = off[a.E + 1 + i];
    if (tid == 0) {
        a.totals[0] = off[a.E + 1 + a.R];
        a.totals[1] = off[a.E];
        if (a.totals_host_mapped) {
            a.totals_host_mapped[0] = off[a.E + 1 + a.R];
            a.totals_host_mapped[1] = off[a.E];
        }
    }
}

// The work of one layout block: the totals for T = 0, the totals block
// (blockIdx == ntiles), or tile blockIdx. Every layout block of the launch
// takes one arrival on the workspace counter and the last to arrive opens
// the next call (see the header comment). A block that finds the workspace
// not left ready flags EPX_DEV_WORKSPACE and stops.
template <int KMAX>
__device__ __forceinline__ void layout_block(const LayoutArgs &a, char *lds)
{
    const CountLds s = carve_count(lds, a.E, a.R);
    const int ER = a.E + a.R;
    int *agg = reinterpret_cast<int *>(lds + count_lds_bytes(a.E, a.R));
    int *pre = agg + ER, *off = pre + ER;
    __shared__ int s_ok;
    __shared__ uint32_t s_tag;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;

    if (a.ntiles == 0) {  // T = 0: zero counts and offsets, no tiles
        for (int i = tid; i < ER; i += blockDim.x)
            agg[i] = 0;
        __syncthreads();
        write_totals(a, agg, off);
        if (a.channel_prefix)
            for (int i = tid; i < a.R * a.C; i += blockDim.x)
                a.channel_prefix[i] = 0;
        return;
    }

    // Threads tid and tid + 256 both hold token tid of the tile: the first
    // counts it, both share its slot writes; all share the look-back and the
    // row writes (more waves than tokens per SIMD, to hide latency).
    const int tile = blockIdx.x;
    const int tile_base = tile * kLayoutTile;
    const int ntok = min(kLayoutTile, a.T - tile_base);
    const int tt0 = tid & (kLayoutTile - 1);
    const bool counter = tid < kLayoutTile;
    const int t = tile_base + tt0;
    int ek[KMAX];
    if (tile < a.ntiles)
        load_row_experts<KMAX>(a, t, ek);
    if (tid == 0) {
        const uint32_t nblk = (uint32_t)a.ntiles + 1u;  // the layout blocks
        const unsigned long long v = atomicAdd(&a.hdr->calls, 1ull);
        const uint32_t arrived = (uint32_t)v;
        s_ok = arrived < nblk;
        s_tag = (uint32_t)(v >> 32) + 1u;
        if (arrived == nblk - 1)  // all layout blocks are in: open the next call
            atomicAdd(&a.hdr->calls, (1ull << 32) - (unsigned long long)nblk);
    }

    // The block after the last tile: the totals are the inclusive prefix
    // past the last tile, found by the same look-back a tile does.
    if (tile == a.ntiles) {
        __syncthreads();
        if (!s_ok) {
            if (tid == 0)
                flag_error(a.err, EPX_DEV_WORKSPACE);
            return;
        }
        for (int c = tid; c < ER; c += blockDim.x) {
            int p = 0;
            if (!look_back(a.pub, ER, a.ntiles, a.ntiles - 1, c, s_tag, &p))
                flag_error(a.err, EPX_DEV_WORKSPACE);
            agg[c] = p;
        }
        __syncthreads();
        write_totals(a, agg, off);
        return;
    }
    for (int i = tid; i < W * a.E; i += blockDim.x) {
        s.emask[i] = 0;
        s.ecnt[i] = 0;
    }
    for (int i = tid; i < W * a.R; i += blockDim.x)
        s.rmask[i] = 0;
    if (tid < W)
        s.dupwave[tid] = 0;
    __syncthreads();

    const uint64_t bit = 1ull << lane;
    uint64_t rbits = 0;
    int dup = 0, bad = 0;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        const int e = counter ? ek[k] : -1;
        bad |= (e == -2);
        if (e < 0)
            continue;
        const uint64_t old =
            atomicOr(reinterpret_cast<unsigned long long *>(&s.emask[w * a.E + e]), bit);
        dup |= (old & bit) != 0;
        atomicAdd(&s.ecnt[w * a.E + e], 1);
        rbits |= 1ull << (e / a.L);
    }
    if (counter)
        s.rb[tid] = rbits;
    if (bad)
        flag_error(a.err, EPX_DEV_BAD_ROUTE);
    for (uint64_t m = rbits; m; m &= m - 1) {
        const int r = __builtin_ctzll(m);
        atomicOr(reinterpret_cast<unsigned long long *>(&s.rmask[w * a.R + r]), bit);
    }
    if (counter && __any(dup) && lane == 0)
        s.dupwave[w] = 1;
    __syncthreads();
    const uint32_t tag = s_tag;
    if (!s_ok) {  // the counter was not left by a previous call: give up
        if (tid == 0)
            flag_error(a.err, EPX_DEV_WORKSPACE);
        return;
    }

    // wave prefixes inside the tile and the tile's counts, published at
    // once (tile 0's counts are already its inclusive prefix)
    uint64_t *pub_row = a.pub + (int64_t)tile * ER;
    const uint64_t hi = ((uint64_t)tag << 32) | (tile == 0 ? kInclusive : 0);
    for (int e = tid; e < a.E; e += blockDim.x) {
        int run = 0;
        for (int w2 = 0; w2 < W; ++w2) {
            s.wpre_e[w2 * a.E + e] = run;
            run += s.ecnt[w2 * a.E + e];
        }
        agg[e] = run;
        pub_store(pub_row + e, hi | (uint32_t)run);
    }
    for (int r = tid; r < a.R; r += blockDim.x) {
        int run = 0;
        for (int w2 = 0; w2 < W; ++w2) {
            s.wpre_r[w2 * a.R + r] = run;
            run += __popcll(s.rmask[w2 * a.R + r]);
        }
        agg[a.E + r] = run;
        pub_store(pub_row + a.E + r, hi | (uint32_t)run);
    }
    // this tile's prefix, then its inclusive prefix for the tiles after it
    for (int c = tid; c < ER; c += blockDim.x) {
        int p = 0;
        if (!look_back(a.pub, ER, tile, tile, c, tag, &p))
            flag_error(a.err, EPX_DEV_WORKSPACE);
        pre[c] = p;
        if (tile > 0)
            pub_store(pub_row + c, ((uint64_t)tag << 32) | kInclusive | (uint32_t)(p + agg[c]));
    }
    __syncthreads();

    if (t < a.T) {
        // slot of each entry among the entries of its expert, else -1; the
        // two threads of a token take half the entries each when K % 8 == 0
        const int wt = tt0 >> 6;
        const bool halves = (a.K & 7) == 0;
        const int k_lo = halves ? (tid >> 8) * (a.K >> 1) : 0;
        const int k_hi = halves ? k_lo + (a.K >> 1) : (counter ? a.K : 0);
        int32_t *sie = a.slot_in_expert + (int64_t)t * a.K;
        int v[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const int e = ek[k];
            v[k] = (e >= 0 && k >= k_lo && k < k_hi)
                       ? pre[e] + s.wpre_e[wt * a.E + e] + wave_rank(a, s, tile_base, tt0, k, e)
                       : -1;
        }
        if ((a.K & 3) == 0) {
#pragma unroll
            for (int k0 = 0; k0 < KMAX; k0 += 4)
                if (k0 >= k_lo && k0 < k_hi)
                    *reinterpret_cast<u32x4 *>(sie + k0) =
                        u32x4{(uint32_t)v[k0], (uint32_t)v[k0 + 1], (uint32_t)v[k0 + 2],
                              (uint32_t)v[k0 + 3]};
        } else {
#pragma unroll
            for (int k = 0; k < KMAX; ++k)
                if (k >= k_lo && k < k_hi)
                    sie[k] = v[k];
        }
    }

    // is_token_in_rank and pos_in_rank rows of the tile are contiguous:
    // write them as one block, 16 bytes per thread per step
    if ((a.R & 15) == 0) {
        uint8_t *dst = a.is_token_in_rank + (int64_t)tile_base * a.R;
        const int nq = a.R >> 4;
        for (int q = tid; q < ntok * nq; q += blockDim.x) {
            const int tt = q / nq, r0 = (q - tt * nq) * 16;
            *reinterpret_cast<u32x4 *>(dst + (int64_t)q * 16) = rank_bytes16(s.rb[tt] >> r0);
        }
    } else if (counter && t < a.T) {
        write_rank_row(a.is_token_in_rank + (int64_t)t * a.R, rbits, a.R);
    }
    if (a.R >= 4 && (a.R & (a.R - 1)) == 0) {
        // R/4 chunks per row, a power of two dividing the thread count, so a
        // thread's ranks r0..r0+3 stay fixed: their prefixes and masks for
        // each wave of tokens are read from LDS once
        int32_t *dst = a.pos_in_rank + (int64_t)tile_base * a.R;
        const int nq = a.R >> 2, qs = __builtin_ctz(nq);
        const int r0 = (tid & (nq - 1)) * 4;
#pragma unroll
        for (int ww = 0; ww < W; ++ww) {
            int base[4];
            uint64_t rm[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                base[j] = pre[a.E + r0 + j] + s.wpre_r[ww * a.R + r0 + j];
                rm[j] = s.rmask[ww * a.R + r0 + j];
            }
            const int qend = min((ww + 1) * kWave, ntok) * nq;
            for (int q = ww * kWave * nq + tid; q < qend; q += blockDim.x) {
                const int tt = q >> qs;
                const uint64_t rbt = s.rb[tt] >> r0, below = lanes_below(tt & 63);
                int v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    v[j] = ((rbt >> j) & 1ull) ? base[j] + __popcll(rm[j] & below) : -1;
                *reinterpret_cast<u32x4 *>(dst + (int64_t)q * 4) =
                    u32x4{(uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]};
            }
        }
    } else if ((a.R & 3) == 0) {
        int32_t *dst = a.pos_in_rank + (int64_t)tile_base * a.R;
        const int nq = a.R >> 2;
        for (int q = tid; q < ntok * nq; q += blockDim.x) {
            const int tt = q / nq, r0 = (q - tt * nq) * 4;
            const uint64_t rbt = s.rb[tt];
            const int ww = tt >> 6;
            const uint64_t below = lanes_below(tt & 63);
            int v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = r0 + j;
                v[j] = ((rbt >> r) & 1ull) ? pre[a.E + r] + s.wpre_r[ww * a.R + r] +
                                                 __popcll(s.rmask[ww * a.R + r] & below)
                                           : -1;
            }
            *reinterpret_cast<u32x4 *>(dst + (int64_t)q * 4) =
                u32x4{(uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]};
        }
    } else if (counter && t < a.T) {
        const uint64_t below = lanes_below(lane);
        int32_t *pir = a.pos_in_rank + (int64_t)t * a.R;
        for (int r = 0; r < a.R; ++r)
            pir[r] = ((rbits >> r) & 1ull) ? pre[a.E + r] + s.wpre_r[w * a.R + r] +
                                                 __popcll(s.rmask[w * a.R + r] & below)
                                           : -1;
    }

    // the channel columns whose last token lies in this tile
    if (a.channel_prefix) {
        Walk it(tid, blockDim.x, a.C);
        for (int i = tid; i < a.R * a.C; i += blockDim.x, it.next()) {
            const int r = it.row;
            const int64_t end = channel_end(a, it.col);
            if (end <= tile_base || end > tile_base + ntok)
                continue;
            const int n = (int)(end - tile_base);
            int v = pre[a.E + r];
            for (int w2 = 0; w2 < W; ++w2) {
                const int lo = w2 * kWave;
                if (n <= lo)
                    break;
                const uint64_t m = (n >= lo + kWave) ? ~0ull : lanes_below(n - lo);
                v += __popcll(s.rmask[w2 * a.R + r] & m);
            }
            a.channel_prefix[i] = v;
        }
    }
}

}  // namespace
}  // namespace epx
