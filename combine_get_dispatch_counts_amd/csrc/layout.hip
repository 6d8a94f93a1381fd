// layout.hip -- get_dispatch_layout and the receive-offset prefix sums.
//
// [P2] "DeepEP 学习笔记" (DeepEP study notes), "dispatch 前：全局布局与通知":
// per-expert and per-rank counts and is_token_in_rank from topk_idx, then
// prefix sums (channel_prefix_matrix). [P1] "事件驱动 EP 内核的调度策略与零拷贝
// 通信", "事件驱动调度的本质": count locally, prefix-sum the offsets.
// [P2] "DeepEP v2": a token counts once per destination rank.
//
// Two launches, no global atomics, deterministic:
//   count    one block per tile of 256 tokens (4 waves, one token per lane).
//            Each wave ORs its lanes into LDS bitmaps: emask[w][e] has bit l
//            set when token l of wave w routes an entry to expert e, rmask
//            likewise per rank (OR deduplicates ranks for free). Tile counts
//            go to the workspace [tile, E + R]; is_token_in_rank is written.
//   finalize one block per tile again. Each block sums the counts of the
//            tiles before it (a few KB from L2), scans the totals into
//            exp_off / rank_off in LDS, rebuilds its bitmaps and writes the
//            final positions: rank(t) = tile prefix + earlier waves' counts +
//            popcount(mask & lanes below t). Block 0 writes the counts,
//            offsets and totals.
// A wave in which some token lists one expert twice falls back to counting
// earlier entries directly, so ranks stay "entries before (t,k)" exactly.
#include "epx_device.h"
#include "epx_internal.h"

namespace epx {
namespace {

constexpr int W = kLayoutWaves;

struct TileLds {
    uint64_t *emask;      // [W][E]
    uint64_t *rmask;      // [W][R]
    uint64_t *tok_rbits;  // [tile] rank bits per token
    int *ecnt;            // [W][E] entries per expert in the wave
    int *dupwave;         // [W] 1 if the wave has a row with a repeated expert
    int *pre;             // [E+R] counts in earlier tiles (finalize only)
    int *tot;             // [E+R] counts over all tiles (finalize only)
    int *off;             // [E+1 + R+1] exclusive offsets (finalize only)
};

__host__ __device__ inline size_t tile_lds_bytes(int E, int R)
{
    return sizeof(uint64_t) * ((size_t)W * E + (size_t)W * R + kLayoutTile) +
           sizeof(int) * ((size_t)W * E + W);
}

__host__ __device__ inline size_t finalize_lds_bytes(int E, int R)
{
    return tile_lds_bytes(E, R) + sizeof(int) * (2 * (size_t)(E + R) + (E + R + 2));
}

__device__ TileLds carve(char *base, int E, int R)
{
    TileLds s;
    s.emask = reinterpret_cast<uint64_t *>(base);
    s.rmask = s.emask + (size_t)W * E;
    s.tok_rbits = s.rmask + (size_t)W * R;
    s.ecnt = reinterpret_cast<int *>(s.tok_rbits + kLayoutTile);
    s.dupwave = s.ecnt + (size_t)W * E;
    s.pre = s.dupwave + W;
    s.tot = s.pre + (E + R);
    s.off = s.tot + (E + R);
    return s;
}

// Build the bitmaps and per-wave expert counts of one tile. Every thread of
// the block must call this (it holds barriers).
__device__ void build_tile(const LayoutArgs &a, int tile_base, const TileLds &s, bool report)
{
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    for (int i = tid; i < W * a.E; i += blockDim.x) {
        s.emask[i] = 0;
        s.ecnt[i] = 0;
    }
    for (int i = tid; i < W * a.R; i += blockDim.x)
        s.rmask[i] = 0;
    if (tid < W)
        s.dupwave[tid] = 0;
    __syncthreads();

    const int t = tile_base + tid;
    const uint64_t bit = 1ull << lane;
    uint64_t rbits = 0;
    int dup = 0;
    if (t < a.T) {
        const int64_t *row = a.topk_idx + (int64_t)t * a.K;
        for (int k = 0; k < a.K; ++k) {
            const int64_t e = row[k];
            if (e == -1)
                continue;
            if (e < 0 || e >= a.E) {
                if (report)
                    flag_error(a.err, EPX_DEV_BAD_ROUTE);
                continue;
            }
            const uint64_t old =
                atomicOr(reinterpret_cast<unsigned long long *>(&s.emask[w * a.E + e]), bit);
            dup |= (old & bit) != 0;
            atomicAdd(&s.ecnt[w * a.E + e], 1);
            rbits |= 1ull << (int)(e / a.L);
        }
    }
    s.tok_rbits[tid] = rbits;
    for (uint64_t m = rbits; m; m &= m - 1) {
        const int r = __builtin_ctzll(m);
        atomicOr(reinterpret_cast<unsigned long long *>(&s.rmask[w * a.R + r]), bit);
    }
    if (__any(dup) && lane == 0)
        s.dupwave[w] = 1;
    __syncthreads();
}

// Entries before (tile token tt, slot k) inside tt's wave that route to e.
__device__ int wave_rank(const LayoutArgs &a, const TileLds &s, int tile_base, int tt, int k,
                         int64_t e)
{
    const int w = tt >> 6, l = tt & 63;
    if (!s.dupwave[w])
        return __popcll(s.emask[w * a.E + e] & lanes_below(l));
    const int64_t *base = a.topk_idx + (int64_t)(tile_base + (w << 6)) * a.K;
    const int upto = l * a.K + k;
    int n = 0;
    for (int i = 0; i < upto; ++i)
        n += (base[i] == e);
    return n;
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

__global__ __launch_bounds__(kLayoutTile) void layout_count_kernel(LayoutArgs a)
{
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const TileLds s = carve(lds, a.E, a.R);
    const int tile_base = blockIdx.x * kLayoutTile;
    build_tile(a, tile_base, s, true);

    const int ntok = min(kLayoutTile, a.T - tile_base);
    uint8_t *itr = a.is_token_in_rank + (int64_t)tile_base * a.R;
    for (int i = threadIdx.x; i < ntok * a.R; i += blockDim.x) {
        const int tt = i / a.R, r = i - tt * a.R;
        itr[i] = (uint8_t)((s.tok_rbits[tt] >> r) & 1ull);
    }
    int32_t *cnt = a.tile_cnt + (int64_t)blockIdx.x * (a.E + a.R);
    for (int e = threadIdx.x; e < a.E; e += blockDim.x) {
        int c = 0;
        for (int w = 0; w < W; ++w)
            c += s.ecnt[w * a.E + e];
        cnt[e] = c;
    }
    for (int r = threadIdx.x; r < a.R; r += blockDim.x) {
        int c = 0;
        for (int w = 0; w < W; ++w)
            c += __popcll(s.rmask[w * a.R + r]);
        cnt[a.E + r] = c;
    }
}

__global__ __launch_bounds__(kLayoutTile) void layout_finalize_kernel(LayoutArgs a)
{
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const TileLds s = carve(lds, a.E, a.R);
    const int b = blockIdx.x, tid = threadIdx.x;
    const int tile_base = b * kLayoutTile;
    const int ER = a.E + a.R;
    if (a.ntiles > 0)
        build_tile(a, tile_base, s, false);

    // counts before this tile and over all tiles, per expert then per rank
    for (int i = tid; i < ER; i += blockDim.x) {
        int p = 0, q = 0;
        for (int j = 0; j < a.ntiles; ++j) {
            const int v = a.tile_cnt[(int64_t)j * ER + i];
            p += (j < b) ? v : 0;
            q += v;
        }
        s.pre[i] = p;
        s.tot[i] = q;
    }
    __syncthreads();
    if (tid < kWave)
        wave_exclusive_scan(s.tot, a.E, s.off);
    else if (tid < 2 * kWave)
        wave_exclusive_scan(s.tot + a.E, a.R, s.off + a.E + 1);
    __syncthreads();

    if (b == 0) {
        for (int e = tid; e < a.E; e += blockDim.x)
            a.num_tokens_per_expert[e] = s.tot[e];
        for (int r = tid; r < a.R; r += blockDim.x)
            a.num_tokens_per_rank[r] = s.tot[a.E + r];
        for (int i = tid; i <= a.E; i += blockDim.x)
            a.exp_off[i] = s.off[i];
        for (int i = tid; i <= a.R; i += blockDim.x)
            a.rank_off[i] = s.off[a.E + 1 + i];
        if (tid == 0) {
            a.totals[0] = s.off[a.E + 1 + a.R];
            a.totals[1] = s.off[a.E];
            if (a.totals_host_mapped) {
                a.totals_host_mapped[0] = s.off[a.E + 1 + a.R];
                a.totals_host_mapped[1] = s.off[a.E];
            }
        }
        if (a.ntiles == 0 && a.channel_prefix)
            for (int i = tid; i < a.R * a.C; i += blockDim.x)
                a.channel_prefix[i] = 0;
    }
    if (a.ntiles == 0)
        return;

    const int ntok = min(kLayoutTile, a.T - tile_base);
    // pos_in_rank rows of the tile are contiguous: write them flat
    int32_t *pir = a.pos_in_rank + (int64_t)tile_base * a.R;
    for (int i = tid; i < ntok * a.R; i += blockDim.x) {
        const int tt = i / a.R, r = i - tt * a.R;
        int v = -1;
        if ((s.tok_rbits[tt] >> r) & 1ull) {
            const int w = tt >> 6, l = tt & 63;
            v = s.pre[a.E + r] + __popcll(s.rmask[w * a.R + r] & lanes_below(l));
            for (int w2 = 0; w2 < w; ++w2)
                v += __popcll(s.rmask[w2 * a.R + r]);
        }
        pir[i] = v;
    }
    int32_t *sie = a.slot_in_expert + (int64_t)tile_base * a.K;
    const int64_t *tk = a.topk_idx + (int64_t)tile_base * a.K;
    for (int i = tid; i < ntok * a.K; i += blockDim.x) {
        const int tt = i / a.K, k = i - tt * a.K;
        const int64_t e = tk[i];
        int v = -1;
        if (e >= 0 && e < a.E) {
            const int w = tt >> 6;
            v = s.pre[e] + wave_rank(a, s, tile_base, tt, k, e);
            for (int w2 = 0; w2 < w; ++w2)
                v += s.ecnt[w2 * a.E + e];
        }
        sie[i] = v;
    }
    // channel c ends at min((c+1)*ceil(T/C), T); the tile holding token end-1
    // writes the channel's column
    if (a.channel_prefix) {
        const int64_t span = ((int64_t)a.T + a.C - 1) / a.C;
        for (int i = tid; i < a.R * a.C; i += blockDim.x) {
            const int r = i / a.C, c = i - r * a.C;
            const int64_t end = min((int64_t)(c + 1) * span, (int64_t)a.T);
            if (end <= tile_base || end > tile_base + ntok)
                continue;
            const int n = (int)(end - tile_base);
            int v = s.pre[a.E + r];
            for (int w = 0; w < W; ++w) {
                const int lo = w * kWave;
                if (n <= lo)
                    break;
                const uint64_t m = (n >= lo + kWave) ? ~0ull : lanes_below(n - lo);
                v += __popcll(s.rmask[w * a.R + r] & m);
            }
            a.channel_prefix[i] = v;
        }
    }
}

}  // namespace

size_t layout_workspace_bytes(int T, int E, int R)
{
    const size_t ntiles = ((size_t)T + kLayoutTile - 1) / kLayoutTile;
    return ntiles * (size_t)(E + R) * sizeof(int32_t);
}

hipError_t launch_layout(const LayoutArgs &a, hipStream_t stream)
{
    if (a.ntiles > 0)
        hipLaunchKernelGGL(layout_count_kernel, dim3(a.ntiles), dim3(kLayoutTile),
                           tile_lds_bytes(a.E, a.R), stream, a);
    hipLaunchKernelGGL(layout_finalize_kernel, dim3(a.ntiles > 0 ? a.ntiles : 1),
                       dim3(kLayoutTile), finalize_lds_bytes(a.E, a.R), stream, a);
    return hipGetLastError();
}

}  // namespace epx
