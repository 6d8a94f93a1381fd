// layout_device.h -- device code of get_dispatch_layout, shared by the
// layout kernel (layout.hip) and the fused layout + dispatch kernel.
//
// [P2] "DeepEP 学习笔记" (DeepEP study notes), "dispatch 前：全局布局与通知":
// per-expert and per-rank counts and is_token_in_rank from topk_idx, then
// prefix sums (channel_prefix_matrix). [P1] "事件驱动 EP 内核的调度策略与零拷贝
// 通信", "事件驱动调度的本质": count locally, prefix-sum the offsets.
// [P2] "DeepEP v2": a token counts once per destination rank.
//
// The workspace protocol shared by both kernels. The tokens are cut into
// 256-token tiles; the block that counts a tile publishes its per-expert
// and per-rank counts as self-contained 64-bit words (call tag << 32 |
// count) in the workspace row of that tile, and readers poll a word until
// it carries the current call's tag, so a word left by an earlier call, of
// any shape, reads as "not yet". The call tag is the call number in the
// workspace head plus one; every block reads it with one plain load at its
// start, and a second counter in the head makes sure the number moves on
// only once every block of the launch holds it (two ways, below), so the
// next launch sees the new one. Every wait is bounded: a word that stays
// unpublished too long sets EPX_DEV_WORKSPACE and the kernel ends anyway.
#pragma once

#include "epx_device.h"
#include "epx_internal.h"

namespace epx {
namespace {

constexpr int kSpinLimit = 1 << 18;

__device__ __forceinline__ void pub_store(uint64_t *p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t pub_load(const uint64_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Two ways to move the call number on, which leave the head alike between
// calls (second counter 0, low half 0), so launches of either kind can
// share a workspace:
//  - count out (read_call_tag at the start, leave_call at the end): the
//    last block of the grid to finish moves the number on. Each block's
//    count goes out at its own end, spread over the launch; used by the
//    fused launch, whose hundreds of blocks counting at once would queue
//    on the word while their rows load.
//  - count in (load_call, enter_call once the block's loads are out,
//    close_call at the end): the last block to count in moves the number
//    on when it ends. No block ends waiting for a round trip on the word;
//    used by the layout kernel (a few dozen blocks), where that round trip
//    was on the critical path.

// The call's tag from the workspace head; false if the head was not left
// by a finished call (its low half is always 0 between calls).
__device__ __forceinline__ bool read_call_tag(const LayoutHdr *hdr, uint32_t *tag)
{
    const unsigned long long v =
        __hip_atomic_load(&hdr->calls, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *tag = (uint32_t)(v >> 32) + 1u;
    return (uint32_t)v == 0u;
}

// Counting out: called by one thread of every block when the block is done;
// the last one of the grid opens the next call.
__device__ __forceinline__ void leave_call(LayoutHdr *hdr)
{
    const unsigned int n = atomicAdd(&hdr->done, 1u);
    if (n == gridDim.x - 1) {
        __hip_atomic_store(&hdr->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        atomicAdd(&hdr->calls, 1ull << 32);
    }
}

// Counting in: the workspace head, loaded once by one thread of a block at
// its start.
__device__ __forceinline__ unsigned long long load_call(const LayoutHdr *hdr)
{
    return __hip_atomic_load(&hdr->calls, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The call's tag from the loaded head; false if the head was not left by a
// finished call (its low half is always 0 between calls). The block is then
// counted in: *arrival is how many blocks of the grid counted in before it.
// The increment is made from the loaded value (its low half, 0 in every
// state a finished call leaves), so it cannot go out before the head's load
// has returned: once the count reaches the grid, every block holds its tag.
__device__ __forceinline__ bool enter_call(LayoutHdr *hdr, unsigned long long head,
                                           uint32_t *tag, unsigned int *arrival)
{
    *tag = (uint32_t)(head >> 32) + 1u;
    *arrival = atomicAdd(&hdr->done, 1u + ((uint32_t)head & 1u));
    return (uint32_t)head == 0u;
}

// Called by the block's counting-in thread when the block is done: the last
// block to have counted in moves the call number on (every block of the grid
// read it before). The count's round trip has long completed by then, so no
// block ends waiting for it.
__device__ __forceinline__ void close_call(LayoutHdr *hdr, unsigned int arrival)
{
    if (arrival == gridDim.x - 1) {
        __hip_atomic_store(&hdr->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        atomicAdd(&hdr->calls, 1ull << 32);
    }
}

// Sum of column c of the published words of tiles [0, ntiles): in *all,
// and over tiles below `upto` in *before. 16 words are loaded together,
// then each is polled on its own until it carries the tag. Returns false
// if a word stayed unpublished past the spin limit.
__device__ __forceinline__ bool sum_tile_words(const uint64_t *pub, int ER, int ntiles, int c,
                                               int upto, uint32_t tag, int *all, int *before)
{
    bool ok = true;
    int s_all = 0, s_before = 0;
    for (int j0 = 0; j0 < ntiles; j0 += 16) {
        const int nq = min(16, ntiles - j0);
        const uint64_t *col = pub + (int64_t)j0 * ER + c;
        uint64_t wv[16];
#pragma unroll
        for (int q = 0; q < 16; ++q)
            wv[q] = q < nq ? pub_load(col + (int64_t)q * ER) : 0;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            if (q >= nq)
                break;
            for (int polls = 0; (uint32_t)(wv[q] >> 32) != tag && ok;) {
                if (++polls > kSpinLimit)
                    ok = false;
                __builtin_amdgcn_s_sleep(2);
                wv[q] = pub_load(col + (int64_t)q * ER);
            }
            const int v = (int)(uint32_t)wv[q];
            s_all += v;
            s_before += j0 + q < upto ? v : 0;
        }
    }
    *all = s_all;
    *before = s_before;
    return ok;
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

// Channel c covers tokens [c*ceil(T/C), min((c+1)*ceil(T/C), T)); the block
// holding its last token owns column c of channel_prefix.
__device__ __forceinline__ int64_t channel_end(const LayoutArgs &a, int c)
{
    const int64_t span = ((int64_t)a.T + a.C - 1) / a.C;
    return min((int64_t)(c + 1) * span, (int64_t)a.T);
}

// Counts, offsets and totals from the totals in tot[0..E+R), using off as
// scratch; one block of at least two waves.
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

}  // namespace
}  // namespace epx
