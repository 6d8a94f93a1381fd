// fused.hip -- get_dispatch_layout and the high-throughput dispatch in one
// launch.
//
// [P2] "DeepEP v2": the v2 dispatch kernel computes the layout itself (its
// notify warps take the place of get_dispatch_layout) while its dispatch
// warps move the data, in one launch. Here the first blocks of the grid are
// the layout's blocks (layout_device.h: one per 256-token tile, then the
// totals block), and every block of kLayoutThreads threads then dispatches
// one token per wave (dispatch_device.h), so the grid is no larger than
// the dispatch alone needs.
//
// Hand-over. The layout blocks publish, beside their usual outputs, the
// totals and each token's final in-rank positions and in-expert slots as
// self-contained words (tag << 32 | value, the scheme of the tiles'
// look-back), so no ordering between different addresses is relied on, and
// words left in the workspace by earlier calls, of any shape, carry older
// tags. A block, once the totals are out, scans them into the rank and
// expert offsets in LDS; each of its waves then waits for its token's
// R + K words and moves the row.
//
// The call's tag. No block takes an arrival on the call counter (one
// word: every block of the grid hitting it at once would serialise for
// microseconds): the counter moves on to the next call only when the last
// block of the grid has finished (a second counter counts finished
// blocks), so the call number is fixed for the whole launch and every
// block reads it with one plain load, checking on the way that no layout
// call was left unfinished (arrivals 0).
//
// When it is used. The layout blocks, once their layout part is done, wait
// for the totals block like the others, so all layout blocks must be on the
// chip together; and the dispatch work is all in flight at once only while
// the whole grid is: a block keeps its place until its slowest wave ends,
// so later rounds of blocks would each start behind a tail (a loop over
// several tokens per wave instead raised the register count at h = 7168 far
// enough to halve the resident waves). With fewer blocks than compute units, on the
// other hand, a token's eight waves share one unit's store path while other
// units idle. The host therefore launches this kernel when its grid covers
// every compute unit and, by the occupancy query, fits on the chip at once;
// small batches go to fused_small_kernel below, and everything else runs
// the layout and the dispatch as two launches, whose 64-thread dispatch
// blocks spread one wave per token over the chip and free their place wave
// by wave. Layout blocks come first in the grid;
// dispatch-only blocks issue their row loads before waiting, so the loads
// overlap the layout. Every wait is bounded.
#include <atomic>

#include "dispatch_device.h"
#include "layout_device.h"

namespace epx {
namespace {

constexpr int kFusedTokens = kLayoutThreads / kWave;  // tokens per block

// Wait until the word each needing lane reads carries the call's tag
// (bounded; false on time-out). Wave-uniform loop.
__device__ bool wait_tagged(const uint64_t *p, bool need, uint32_t tag, uint64_t &w)
{
    int polls = 0;
    w = need ? pub_load(p) : 0;
    while (__any(need && (uint32_t)(w >> 32) != tag)) {
        if (++polls > kSpinLimit)
            return false;
        __builtin_amdgcn_s_sleep(2);
        if (need && (uint32_t)(w >> 32) != tag)
            w = pub_load(p);
    }
    return true;
}

template <int KMAX, bool FP8, int NV>
__global__ __launch_bounds__(kLayoutThreads) void fused_kernel(FusedArgs f)
{
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const DispatchArgs &a = f.disp;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid >> 6;
    const int t = blockIdx.x * kFusedTokens + w;
    const bool have = t < a.T;
    const int ER = a.E + a.R;
    int *tot = reinterpret_cast<int *>(lds + count_lds_bytes(a.E, a.R));
    int *off = tot + ER;  // [E+1] expert offsets, then [R+1] rank offsets

    bool go = true;  // block-uniform: false once the layout part was refused
    uint32_t tag;
    typename std::conditional<FP8, RowFp8<NV>, RowBf16<NV>>::type row;
    const uint16_t *xrow = a.x + (size_t)(have ? t : 0) * a.h;
    if ((int)blockIdx.x <= f.lay.ntiles) {  // a layout block (or T = 0)
        go = layout_block<KMAX>(f.lay, lds, f.tok, f.tot, false, tag);  // flags if refused
        if (f.lay.ntiles == 0)  // T = 0: one block, no counters involved
            return;
        __syncthreads();  // the layout's LDS is reused below
        if (go && have)
            row.load(reinterpret_cast<const u32x4 *>(xrow), 0, FP8 ? a.h >> 4 : a.h >> 3);
    } else {
        if (have)
            row.load(reinterpret_cast<const u32x4 *>(xrow), 0, FP8 ? a.h >> 4 : a.h >> 3);
        __shared__ int s_go;
        const unsigned long long v =
            __hip_atomic_load(&f.lay.hdr->calls, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        tag = (uint32_t)(v >> 32) + 1u;
        if (tid == 0) {
            s_go = (uint32_t)v == 0u;
            if (!s_go)
                flag_error(a.err, EPX_DEV_WORKSPACE);
        }
        __syncthreads();
        go = s_go;
    }
    const int64_t e = (have && lane < a.K) ? a.topk_idx[(int64_t)t * a.K + lane] : -1;

    if (go) {
        // the totals, 64 words per wave, then the offsets scanned into LDS
        for (int c0 = w * kWave; c0 < ER; c0 += kFusedTokens * kWave) {
            const int c = c0 + lane;
            uint64_t word;
            if (!wait_tagged(f.tot + min(c, ER - 1), c < ER, tag, word) && lane == 0)
                flag_error(a.err, EPX_DEV_WORKSPACE);
            if (c < ER)
                tot[c] = (int)((uint32_t)word & 0x7FFFFFFFu);
        }
        __syncthreads();
        if (tid < kWave)
            wave_exclusive_scan(tot, a.E, off);
        else if (tid < 2 * kWave)
            wave_exclusive_scan(tot + a.E, a.R, off + a.E + 1);
        __syncthreads();
    }
    if (go && have) {
        // the token's final positions (lane r < R) and slots (lane k < K)
        const uint64_t *tw = f.tok + (int64_t)t * (a.R + a.K);
        uint64_t pw, sw;
        const bool ok_p = wait_tagged(tw + min(lane, a.R - 1), lane < a.R, tag, pw);
        const bool ok_s = wait_tagged(tw + a.R + min(lane, a.K - 1), lane < a.K, tag, sw);
        if (!(ok_p && ok_s) && lane == 0)
            flag_error(a.err, EPX_DEV_WORKSPACE);
        int64_t send_r = -1, recv_r = -1;
        if (ok_p && lane < a.R) {
            const int p = (int)(uint32_t)pw;
            if (p >= 0)
                send_r = (int64_t)off[a.E + 1 + lane] + p;
        }
        if (ok_s && e >= 0 && e < a.E) {
            const int sl = (int)(uint32_t)sw;
            recv_r = sl >= 0 ? (int64_t)off[(int)e] + sl : -1;
        }
        dispatch_token<FP8>(a, t, row, xrow, e, send_r, recv_r);
    }

    // this block is done: the last block of the grid opens the next call
    __syncthreads();
    if (tid == 0) {
        const unsigned int n = atomicAdd(&f.lay.hdr->done, 1u);
        if (n == gridDim.x - 1) {
            __hip_atomic_store(&f.lay.hdr->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            atomicAdd(&f.lay.hdr->calls, 1ull << 32);
        }
    }
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
    if (w < nslices)
        row.load(src, w * per, nitems);

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
            m |= 1ull << (e / l.L);
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

// The grid: the layout's blocks, or the dispatch's one block per
// kFusedTokens tokens if more (one block for T = 0).
int64_t fused_grid(const FusedArgs &f)
{
    const int64_t disp_blocks = (f.disp.T + kFusedTokens - 1) / kFusedTokens;
    const int64_t nlay = f.lay.ntiles + 1;
    return f.lay.ntiles == 0 ? 1 : (disp_blocks > nlay ? disp_blocks : nlay);
}

// With launch false, only say how many launches the call takes (1 or 2).
template <int KMAX, bool FP8, int NV>
hipError_t launch_fused_k(const FusedArgs &f, hipStream_t stream, bool launch, int *launches)
{
    const size_t lds = layout_tok_lds_bytes(f.lay.E, f.lay.R, f.lay.K);
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
        return e != hipSuccess ? e : launch_dispatch(f.disp, FP8, stream);
    }
    hipLaunchKernelGGL((fused_kernel<KMAX, FP8, NV>), dim3((unsigned)blocks),
                       dim3(kLayoutThreads), lds, stream, f);
    return hipGetLastError();
}

template <int KMAX>
hipError_t launch_fused_kmax(const FusedArgs &f, bool fp8, hipStream_t stream, bool launch,
                             int *launches)
{
    switch (pick_nv(f.disp.h, fp8) + (fp8 ? 100 : 0)) {
    case 8: return launch_fused_k<KMAX, false, 8>(f, stream, launch, launches);
    case 14: return launch_fused_k<KMAX, false, 14>(f, stream, launch, launches);
    case 16: return launch_fused_k<KMAX, false, 16>(f, stream, launch, launches);
    case 104: return launch_fused_k<KMAX, true, 4>(f, stream, launch, launches);
    case 107: return launch_fused_k<KMAX, true, 7>(f, stream, launch, launches);
    default: return launch_fused_k<KMAX, true, 8>(f, stream, launch, launches);
    }
}

}  // namespace

size_t fused_workspace_bytes(int T, int K, int E, int R)
{
    const size_t base = layout_workspace_bytes(T, E, R);
    if (base == 0)
        return 0;
    // the layout's, then the totals row, then the tokens' words
    return base + (size_t)(E + R) * sizeof(uint64_t) + (size_t)T * (R + K) * sizeof(uint64_t);
}

hipError_t launch_fused(const FusedArgs &f, bool fp8, hipStream_t stream)
{
    return f.lay.K <= 8 ? launch_fused_kmax<8>(f, fp8, stream, true, nullptr)
                        : launch_fused_kmax<EPX_MAX_TOPK>(f, fp8, stream, true, nullptr);
}

hipError_t fused_launches(const FusedArgs &f, bool fp8, int *launches)
{
    return f.lay.K <= 8 ? launch_fused_kmax<8>(f, fp8, nullptr, false, launches)
                        : launch_fused_kmax<EPX_MAX_TOPK>(f, fp8, nullptr, false, launches);
}

}  // namespace epx
