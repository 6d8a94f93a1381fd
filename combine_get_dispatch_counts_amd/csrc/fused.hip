// fused.hip -- get_dispatch_layout and the high-throughput dispatch in one
// launch.
//
// [P2] "DeepEP v2": the v2 dispatch kernel computes the layout itself (its
// notify warps take the place of get_dispatch_layout) while its dispatch
// warps move the data, in one launch. Here every block of kLayoutThreads
// threads owns kFusedTokens consecutive tokens (one per wave) and works out
// their layout rows itself, so the grid is the size the dispatch alone needs.
//
// One hand-over. A token's in-rank position (in-expert slot) is the count of
// earlier tokens (entries) of the same rank (expert): the sum over the
// 256-token tiles before its own, plus the count inside its tile before it.
// The first ntiles blocks each count one whole tile in LDS and publish its
// E + R counts as self-contained words (tag << 32 | value), before they wait
// for anything; every block then reads all tiles' words -- their sum is the
// totals, from which it scans the offsets, and the tiles before its own give
// its prefix -- while it counts its own tile's tokens before its first token
// in LDS, and the entries of its own earlier tokens from the rank bits and
// entries its waves leave in LDS. No ordering between different addresses is relied on, and words
// left in the workspace by earlier calls, of any shape, carry older tags.
// Blocks write their own tokens' rows of is_token_in_rank, pos_in_rank and
// slot_in_expert, and the channel_prefix columns whose channel ends in their
// tokens; block 0 writes the counts, offsets and totals.
//
// The call's tag. No block takes an arrival on the call counter (one
// word: every block of the grid hitting it at once would serialise for
// microseconds): the counter moves on to the next call only when the last
// block of the grid has finished (a second counter counts finished
// blocks), so the call number is fixed for the whole launch and every
// block reads it with one plain load, checking on the way that no layout
// call was left unfinished (arrivals 0).
//
// When it is used. Every block waits for the first ntiles blocks, which
// wait for nothing before they publish; and the dispatch work is all in
// flight at once only while the whole grid is: a block keeps its place until
// its slowest wave ends, so later rounds of blocks would each start behind a
// tail (a loop over several tokens per wave instead raised the register
// count at h = 7168 far enough to halve the resident waves). With fewer
// blocks than compute units, on the other hand, a token's eight waves share
// one unit's store path while other units idle. The host therefore launches
// this kernel when its grid covers every compute unit and, by the occupancy
// query, fits on the chip at once; small batches go to fused_small_kernel
// below, and everything else runs the layout and the dispatch as two
// launches, whose 64-thread dispatch blocks spread one wave per token over
// the chip and free their place wave by wave. A block loads its tokens'
// rows only once it has counted (and, if it publishes, published): rows
// loaded at entry went out ahead of the counting loads, and the publishers
// every block waits for finished counting 5 us later; loaded after the
// publish, they still overlap the hand-over. Every wait is bounded. Each
// wave then stores its token's rows on the paced sweep (dispatch_device.h),
// its schedule starting when its block's hand-over is complete but no
// earlier than a fixed offset after its own entry (kFusedStartUs plus the
// launch's x-row time): most blocks are ready by then, so the front starts
// sharp instead of spread over the hand-over's 12-20 us (a start shared by
// all blocks, from block 0's entry, was measured too: blocks ready after it
// find rows overdue, which go out as one random burst).
#include <atomic>

#include "dispatch_device.h"
#include "layout_device.h"

namespace epx {
namespace {

constexpr int kFusedTokens = kLayoutThreads / kWave;  // tokens per block

// LDS of fused_kernel: the rank bits and entries of the block's tokens,
// then per expert and rank (E + R ints each): the counts over the block's
// tile before its first token, the tile it publishes, the totals, the counts
// over the earlier tiles, and the offsets (E + R + 2).
__host__ __device__ inline size_t fused_lds_bytes(int E, int R, int kmax)
{
    return sizeof(uint64_t) * kFusedTokens + sizeof(int) * (size_t)kFusedTokens * kmax +
           sizeof(int) * (5 * (size_t)(E + R) + 2);
}

template <int KMAX, bool FP8, int NV>
__global__ __launch_bounds__(kLayoutThreads) void fused_kernel(FusedArgs f)
{
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const LayoutArgs &l = f.lay;
    const DispatchArgs &a = f.disp;
    const uint64_t t_entry = wall_clock64();
    const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid >> 6;
    const int E = a.E, R = a.R, K = a.K, T = a.T, ER = E + R;
    if (blockIdx.x == 0 && tid == 0)
        stamp_launch(a, t_entry);
    uint64_t *tmask = reinterpret_cast<uint64_t *>(lds);                // [kFusedTokens]
    int *tent = reinterpret_cast<int *>(tmask + kFusedTokens);          // [kFusedTokens][KMAX]
    int *bef = tent + kFusedTokens * KMAX;  // [E + R] the tile's tokens before t0
    int *agg = bef + ER;                    // [E + R] the tile this block publishes
    int *tot = agg + ER;                    // [E + R] all tiles
    int *pre = tot + ER;                    // [E + R] the tiles before this block's
    int *off = pre + ER;                    // [E + 1] expert offsets, [R + 1] rank offsets
    __shared__ int s_go;
    __shared__ uint32_t s_tag;

    if (l.ntiles == 0) {  // T = 0: one block, zero counts and offsets, no counters
        for (int i = tid; i < ER; i += blockDim.x)
            tot[i] = 0;
        __syncthreads();
        write_totals(l, tot, off);
        if (l.channel_prefix)
            for (int i = tid; i < R * l.C; i += blockDim.x)
                l.channel_prefix[i] = 0;
        return;
    }

    const int t0 = blockIdx.x * kFusedTokens;
    const int tile = t0 / kLayoutTile, tile_base = tile * kLayoutTile;
    const int t = t0 + w;
    const bool have = t < T;
    const bool publisher = (int)blockIdx.x < l.ntiles;

    // Loads first: the call number; threads below kLayoutTile take the
    // tokens of the block's own tile before t0, the others (publishers only)
    // the tokens of tile blockIdx; lane k < K the token's entry k.
    if (tid == 0) {
        uint32_t tg;
        s_go = read_call_tag(l.hdr, &tg);  // false: the workspace was not left ready
        s_tag = tg;
    }
    const bool pub_thread = tid >= kLayoutTile;
    const int u = pub_thread ? (int)blockIdx.x * kLayoutTile + (tid - kLayoutTile)
                             : tile_base + tid;
    const bool counting = pub_thread ? (publisher && u < T) : u < t0;
    int eu[KMAX];
    if (counting) {
        load_row_experts<KMAX>(l, u, eu);
    } else {
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            eu[k] = -1;
    }
    const int64_t e = (have && lane < K) ? a.topk_idx[(int64_t)t * K + lane] : -1;

    // the token's rank bits and entries, for the tokens after it in the block
    const bool valid = lane < K && e >= 0 && e < E;
    const uint64_t mt = uniform64(wave_or(valid ? 1ull << div_by_magic((int)e, l.L_mul) : 0ull));
    if (lane == 0)
        tmask[w] = have ? mt : 0ull;
    if (lane < K)
        tent[w * KMAX + lane] = valid ? (int)e : -1;
    for (int i = tid; i < 2 * ER; i += blockDim.x)
        bef[i] = 0;  // bef and agg
    __syncthreads();

    // counts: per expert every valid entry, per rank every token once
    {
        int *cnt = pub_thread ? agg : bef;
        uint64_t m = 0;
        int bad = 0;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const int ek = eu[k];
            bad |= (ek == -2);
            if (ek < 0)
                continue;
            atomicAdd(&cnt[ek], 1);
            m |= 1ull << div_by_magic(ek, l.L_mul);
        }
        for (; m; m &= m - 1)
            atomicAdd(&cnt[E + __builtin_ctzll(m)], 1);
        if (bad && pub_thread)
            flag_error(a.err, EPX_DEV_BAD_ROUTE);
    }
    __syncthreads();
    const uint32_t tag = s_tag;
    bool go = s_go;
    if (!go) {
        if (tid == 0)
            flag_error(a.err, EPX_DEV_WORKSPACE);
    } else if (publisher) {
        uint64_t *prow = l.pub + (int64_t)blockIdx.x * ER;
        for (int c = tid; c < ER; c += blockDim.x)
            pub_store(prow + c, ((uint64_t)tag << 32) | (uint32_t)agg[c]);
    }

    // the token's row, only now: rows loaded at entry filled the memory
    // queues ahead of the counting loads (first touches of topk_idx), and
    // the publishers, which every block waits for, counted behind them
    typename std::conditional<FP8, RowFp8<NV>, RowBf16<NV>>::type row;
    const uint16_t *xrow = a.x + (size_t)(have ? t : 0) * a.h;
    row.load(reinterpret_cast<const u32x4 *>(xrow), 0, have ? (FP8 ? a.h >> 4 : a.h >> 3) : 0);

    // every tile's counts: the totals and this tile's prefix (bounded waits)
    bool ok = true;
    if (go) {
        for (int c = tid; c < ER; c += blockDim.x) {
            int all = 0, before = 0;
            if (ok)
                ok = sum_tile_words(l.pub, ER, l.ntiles, c, tile, tag, &all, &before);
            tot[c] = all;
            pre[c] = before;
        }
    }
    if (__syncthreads_or(!ok)) {
        if (tid == 0)
            flag_error(a.err, EPX_DEV_WORKSPACE);
        go = false;
    }
    if (go) {
        if (blockIdx.x == 0) {
            write_totals(l, tot, off);  // scans into off, then the global outputs
        } else {
            if (tid < kWave)
                wave_exclusive_scan(tot, E, off);
            else if (tid < 2 * kWave)
                wave_exclusive_scan(tot + E, R, off + E + 1);
        }
    }
    __syncthreads();

    // channel_prefix columns whose last token is one of this block's
    if (go && l.channel_prefix) {
        const int tlast = min(t0 + kFusedTokens, T) - 1;
        for (int c = tid; c < l.C; c += blockDim.x) {
            const int end = (int)channel_end(l, c);
            if (end - 1 < t0 || end - 1 > tlast)
                continue;
            for (int r = 0; r < R; ++r) {
                int n = pre[E + r] + bef[E + r];
                for (int w2 = 0; w2 < end - t0; ++w2)
                    n += (int)((tmask[w2] >> r) & 1ull);
                l.channel_prefix[(int64_t)r * l.C + c] = n;
            }
        }
    }

    if (go && have) {
        // earlier tokens of the block: per rank lane, the tokens going to
        // it; per entry lane, the entries with the same expert, and the
        // earlier entries of the token's own row. Each token's entries are
        // read at once and counted without a branch per entry (a read and
        // a wait per entry cost the block's last wave ~3 us).
        int cr = 0, ce = 0, rep = 0;
        const int ev = valid ? (int)e : -3;  // stored entries are >= -1
        for (int w2 = 0; w2 <= w; ++w2) {
            const bool earlier = w2 < w;
            cr += earlier ? (int)((tmask[w2] >> lane) & 1ull) : 0;
            const int *row = tent + w2 * KMAX;
#pragma unroll
            for (int k2 = 0; k2 < KMAX; ++k2) {
                const int hit = (row[k2] == ev) & (k2 < K);
                ce += earlier ? hit : 0;
                rep += (!earlier && k2 < lane) ? hit : 0;
            }
        }
        const bool in_r = lane < R && ((mt >> lane) & 1ull);
        const int p = in_r ? pre[E + lane] + bef[E + lane] + cr : -1;
        const int slot = valid ? pre[(int)e] + bef[(int)e] + ce + rep : -1;
        const int64_t send_r = in_r ? (int64_t)off[E + 1 + lane] + p : -1;
        const int64_t recv_r = valid ? (int64_t)off[(int)e] + slot : -1;
        if (lane < R) {
            l.is_token_in_rank[(int64_t)t * R + lane] = in_r ? 1 : 0;
            l.pos_in_rank[(int64_t)t * R + lane] = p;
        }
        if (lane < K)
            l.slot_in_expert[(int64_t)t * K + lane] = slot;
        dispatch_token<FP8>(a, t, row, xrow, e, send_r, recv_r, off[E + 1 + R], t_entry);
    }

    // this block is done: the last block of the grid opens the next call
    __syncthreads();
    if (tid == 0)
        leave_call(l.hdr);
}

// Small batches (T <= kSmallMaxT): one block of kLayoutThreads per token,
// and every block computes the layout of the whole batch itself in LDS from
// all T*K entries (as the low-latency kernel does), so no block waits for
// another and no workspace is touched. Block t then writes token t's rows of
// is_token_in_rank / pos_in_rank / slot_in_expert (block 0 also the counts,
// offsets, totals and channel_prefix), and its waves move the token's row in
// 1024-channel slices w, w + 8, ... to every destination (wave 0 writes the
// handle and the metadata). The counts are the layout's definition: per
// expert every valid entry, per rank every token once; positions and slots
// count the tokens, or entries, before t.
constexpr int kSmallMaxT = 1024;

__host__ __device__ inline size_t small_lds_bytes(int T, int E, int R)
{
    // token rank masks [T], counts [E + R], counts before t [E + R], offsets [E + R + 2]
    return sizeof(uint64_t) * (size_t)T + sizeof(int) * (3 * (size_t)(E + R) + 2);
}

template <int KMAX, bool FP8>
__global__ __launch_bounds__(kLayoutThreads) void fused_small_kernel(FusedArgs f)
{
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const LayoutArgs &l = f.lay;
    const DispatchArgs &a = f.disp;
    const int t = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1), w = tid >> 6;
    const int E = a.E, R = a.R, K = a.K, T = a.T;
    uint64_t *mask = reinterpret_cast<uint64_t *>(lds);
    int *cnt = reinterpret_cast<int *>(mask + T);  // [E] per expert, then [R] per rank
    int *before = cnt + E + R;
    int *off = before + E + R;  // [E+1] expert offsets, then [R+1] rank offsets

    // the token's experts (lane k) and the wave's first slice go out first
    const int64_t ek = lane < K ? a.topk_idx[(int64_t)t * K + lane] : -1;
    typename std::conditional<FP8, RowFp8<1>, RowBf16<2>>::type row;
    constexpr int per = decltype(row)::kPerPass;  // 1024 channels
    const int nitems = FP8 ? a.h >> 4 : a.h >> 3;
    const int nslices = (nitems + per - 1) / per;
    const uint16_t *xrow = a.x + (size_t)t * a.h;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(xrow);
    row.load(src, w * per, nitems);  // zeros past the row

    for (int i = tid; i < 2 * (E + R); i += blockDim.x)
        cnt[i] = 0;  // cnt and before
    __syncthreads();
    // every token of the batch, one thread each
    int bad = 0;
    for (int u = tid; u < T; u += blockDim.x) {
        int eu[KMAX];
        load_row_experts<KMAX>(l, u, eu);
        uint64_t m = 0;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const int e = eu[k];
            bad |= (e == -2);
            if (e < 0)
                continue;
            atomicAdd(&cnt[e], 1);
            if (u < t)
                atomicAdd(&before[e], 1);
            m |= 1ull << div_by_magic(e, l.L_mul);
        }
        mask[u] = m;
        for (uint64_t mm = m; mm; mm &= mm - 1) {
            const int r = __builtin_ctzll(mm);
            atomicAdd(&cnt[E + r], 1);
            if (u < t)
                atomicAdd(&before[E + r], 1);
        }
    }
    if (bad && t == 0)
        flag_error(a.err, EPX_DEV_BAD_ROUTE);
    __syncthreads();
    if (t == 0) {
        write_totals(l, cnt, off);  // scans into off, then the global outputs
    } else {
        if (tid < kWave)
            wave_exclusive_scan(cnt, E, off);
        else if (tid < 2 * kWave)
            wave_exclusive_scan(cnt + E, R, off + E + 1);
    }
    __syncthreads();
    if (t == 0 && l.channel_prefix) {
        for (int i = tid; i < R * l.C; i += blockDim.x) {
            const int r = i / l.C, c = i - r * l.C;
            const int end = (int)channel_end(l, c);
            int n = 0;
            for (int u = 0; u < end; ++u)
                n += (int)((mask[u] >> r) & 1ull);
            l.channel_prefix[i] = n;
        }
    }

    // token t: its row of the layout (wave 0) and its destinations (every wave)
    const uint64_t mt = mask[t];
    const bool in_r = lane < R && ((mt >> lane) & 1ull);
    int64_t send_r = -1, recv_r = -1;
    if (in_r && a.send_x)
        send_r = (int64_t)off[E + 1 + lane] + before[E + lane];
    const bool valid = lane < K && ek >= 0 && ek < E;
    int slot = -1;
    {
        int rep = 0;  // earlier entries of this row with the same expert
        for (int k2 = 0; k2 < K; ++k2)
            rep += (k2 < lane && readlane64(ek, k2) == ek);
        if (valid) {
            slot = before[ek] + rep;
            recv_r = (int64_t)off[ek] + slot;
        }
    }
    if (w == 0) {
        if (lane < R) {
            l.is_token_in_rank[(int64_t)t * R + lane] = in_r ? 1 : 0;
            l.pos_in_rank[(int64_t)t * R + lane] = in_r ? before[E + lane] : -1;
        }
        if (lane < K)
            l.slot_in_expert[(int64_t)t * K + lane] = slot;
    }
    const Dests d = token_dests(a, t, ek, send_r, recv_r, w == 0);
    for (int sl = w; sl < nslices; sl += kLayoutThreads / kWave) {
        if (sl != w)
            row.load(src, sl * per, nitems);
        scatter_slice<FP8>(row, d, sl * per, a);
    }
}

// Blocks of this kernel one compute unit holds at once for a dynamic LDS
// size (the occupancy query, cached for the last size asked).
template <int KMAX, bool FP8, int NV>
int fused_blocks_per_cu(size_t lds)
{
    static std::atomic<uint64_t> cache{0};  // (lds + 1) << 8 | blocks
    const uint64_t c = cache.load(std::memory_order_relaxed);
    if ((c >> 8) == lds + 1)
        return (int)(c & 0xFF);
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fused_kernel<KMAX, FP8, NV>,
                                                     kLayoutThreads, lds) != hipSuccess)
        return 0;
    n = n < 0 ? 0 : (n > 255 ? 255 : n);
    cache.store(((uint64_t)(lds + 1) << 8) | (uint64_t)n, std::memory_order_relaxed);
    return n;
}

// The grid: one block per kFusedTokens tokens (one block for T = 0).
int64_t fused_grid(const FusedArgs &f)
{
    const int64_t disp_blocks = (f.disp.T + kFusedTokens - 1) / kFusedTokens;
    return disp_blocks > 0 ? disp_blocks : 1;
}

// With launch false, only say how many launches the call takes (1 or 2).
template <int KMAX, bool FP8, int NV>
hipError_t launch_fused_k(const FusedArgs &f, std::atomic<unsigned> *seq, hipStream_t stream,
                          bool launch, int *launches)
{
    const size_t lds = fused_lds_bytes(f.lay.E, f.lay.R, KMAX);
    const int64_t blocks = fused_grid(f);
    const bool small = f.disp.T >= 1 && f.disp.T <= kSmallMaxT;
    const bool one = small || f.lay.ntiles == 0 ||
                     (blocks >= f.cus &&
                      blocks <= (int64_t)fused_blocks_per_cu<KMAX, FP8, NV>(lds) * f.cus);
    if (launches)
        *launches = one ? 1 : 2;
    if (!launch)
        return hipSuccess;
    if (small) {
        hipLaunchKernelGGL((fused_small_kernel<KMAX, FP8>), dim3((unsigned)f.disp.T),
                           dim3(kLayoutThreads), small_lds_bytes(f.disp.T, f.disp.E, f.disp.R),
                           stream, f);
        return hipGetLastError();
    }
    if (!one) {
        const hipError_t e = launch_layout(f.lay, stream);
        return e != hipSuccess ? e : launch_dispatch(f.disp, FP8, f.cus, seq, stream);
    }
    FusedArgs g = f;
    g.disp.stamp_slot = next_stamp_slot(seq);
    if (g.disp.sweep_bpt)
        g.disp.start_ticks = (uint32_t)(kFusedStartUs * g.disp.wclk_per_us) +
                             load_ticks(g.disp.T, g.disp.h, g.disp.sweep_bpt);
    hipLaunchKernelGGL((fused_kernel<KMAX, FP8, NV>), dim3((unsigned)blocks),
                       dim3(kLayoutThreads), lds, stream, g);
    return hipGetLastError();
}

template <int KMAX>
hipError_t launch_fused_kmax(const FusedArgs &f, bool fp8, std::atomic<unsigned> *seq,
                             hipStream_t stream, bool launch, int *launches)
{
    switch (pick_nv(f.disp.h, fp8) + (fp8 ? 100 : 0)) {
    case 8: return launch_fused_k<KMAX, false, 8>(f, seq, stream, launch, launches);
    case 14: return launch_fused_k<KMAX, false, 14>(f, seq, stream, launch, launches);
    case 16: return launch_fused_k<KMAX, false, 16>(f, seq, stream, launch, launches);
    case 104: return launch_fused_k<KMAX, true, 4>(f, seq, stream, launch, launches);
    case 107: return launch_fused_k<KMAX, true, 7>(f, seq, stream, launch, launches);
    default: return launch_fused_k<KMAX, true, 8>(f, seq, stream, launch, launches);
    }
}

}  // namespace

size_t fused_workspace_bytes(int T, int K, int E, int R)
{
    (void)K;
    return layout_workspace_bytes(T, E, R);  // the head and the tiles' words
}

hipError_t launch_fused(const FusedArgs &f, bool fp8, std::atomic<unsigned> *seq,
                        hipStream_t stream)
{
    return f.lay.K <= 8 ? launch_fused_kmax<8>(f, fp8, seq, stream, true, nullptr)
                        : launch_fused_kmax<EPX_MAX_TOPK>(f, fp8, seq, stream, true, nullptr);
}

hipError_t fused_launches(const FusedArgs &f, bool fp8, int *launches)
{
    return f.lay.K <= 8 ? launch_fused_kmax<8>(f, fp8, nullptr, nullptr, false, launches)
                        : launch_fused_kmax<EPX_MAX_TOPK>(f, fp8, nullptr, nullptr, false, launches);
}

}  // namespace epx
