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

// Flat index walker over a [rows, cols] block of a row-major array: thread
// tid starts at element tid and advances by blockDim, tracking (row, col)
// with one division up front instead of one per element.
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

// Build the bitmaps and per-wave expert counts of one tile. Every thread of
// the block must call this (it holds barriers). The token's K entries are
// loaded first, so their latency overlaps the LDS clear; they are returned
// in ek (expert id, -1 = no route, -2 = out of range).
__device__ void build_tile(const LayoutArgs &a, int tile_base, const TileLds &s, bool report,
                           int (&ek)[EPX_MAX_TOPK])
{
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int t = tile_base + tid;
    // Loads go out 8 at a time from clamped (always valid) addresses and are
    // masked afterwards, so they are in flight together rather than one
    // branch and one wait each. A tile exists only when T >= 1.
    const int64_t *row = a.topk_idx + (int64_t)min(t, a.T - 1) * a.K;
#pragma unroll
    for (int k0 = 0; k0 < EPX_MAX_TOPK; k0 += 8) {
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
    for (int k = 0; k < EPX_MAX_TOPK; ++k) {
        const int e = ek[k];
        bad |= (e == -2);
        if (e < 0)
            continue;
        const uint64_t old =
            atomicOr(reinterpret_cast<unsigned long long *>(&s.emask[w * a.E + e]), bit);
        dup |= (old & bit) != 0;
        atomicAdd(&s.ecnt[w * a.E + e], 1);
        rbits |= 1ull << (e / a.L);
    }
    if (report && bad)
        flag_error(a.err, EPX_DEV_BAD_ROUTE);
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

// Row of R bytes (0/1) for one token; 16-byte stores when R allows it.
__device__ void write_rank_row(uint8_t *dst, uint64_t rbits, int R)
{
    if ((R & 15) == 0) {
        for (int r0 = 0; r0 < R; r0 += 16) {
            uint32_t wd[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t nib = (uint32_t)(rbits >> (r0 + 4 * j)) & 0xFu;
                wd[j] = (nib & 1u) | ((nib & 2u) << 7) | ((nib & 4u) << 14) | ((nib & 8u) << 21);
            }
            *reinterpret_cast<u32x4 *>(dst + r0) = u32x4{wd[0], wd[1], wd[2], wd[3]};
        }
    } else {
        for (int r = 0; r < R; ++r)
            dst[r] = (uint8_t)((rbits >> r) & 1ull);
    }
}

__global__ __launch_bounds__(kLayoutTile) void layout_count_kernel(LayoutArgs a)
{
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const TileLds s = carve(lds, a.E, a.R);
    const int tile_base = blockIdx.x * kLayoutTile;
    int ek[EPX_MAX_TOPK];
    build_tile(a, tile_base, s, true, ek);

    const int t = tile_base + (int)threadIdx.x;
    if (t < a.T)
        write_rank_row(a.is_token_in_rank + (int64_t)t * a.R, s.tok_rbits[threadIdx.x], a.R);
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
    int ek[EPX_MAX_TOPK];
    if (a.ntiles > 0)
        build_tile(a, tile_base, s, false, ek);

    // counts before this tile and over all tiles, per expert then per rank;
    // 16 independent loads in flight per thread
    for (int i = tid; i < ER; i += blockDim.x) {
        int p = 0, q = 0;
        for (int j0 = 0; j0 < a.ntiles; j0 += 16) {
            int v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u)  // clamped rows, masked below
                v[u] = a.tile_cnt[(int64_t)min(j0 + u, a.ntiles - 1) * ER + i];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int c = (j0 + u < a.ntiles) ? v[u] : 0;
                p += (j0 + u < b) ? c : 0;
                q += c;
            }
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
    const int tt = tid, t = tile_base + tid;
    if (t < a.T) {
        const int w = tt >> 6;
        const uint64_t below = lanes_below(tt & 63);
        const uint64_t rbits = s.tok_rbits[tt];
        // pos_in_rank row: tokens before t in each rank it goes to, else -1
        int32_t *pir = a.pos_in_rank + (int64_t)t * a.R;
        for (int r0 = 0; r0 < a.R; r0 += 4) {
            int v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = r0 + j;
                v[j] = -1;
                if (r < a.R && ((rbits >> r) & 1ull)) {
                    int p = s.pre[a.E + r] + __popcll(s.rmask[w * a.R + r] & below);
                    for (int w2 = 0; w2 < w; ++w2)
                        p += __popcll(s.rmask[w2 * a.R + r]);
                    v[j] = p;
                }
            }
            if ((a.R & 3) == 0) {
                *reinterpret_cast<u32x4 *>(pir + r0) =
                    u32x4{(uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]};
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (r0 + j < a.R)
                        pir[r0 + j] = v[j];
            }
        }
        // slot_in_expert row: entries before (t,k) routed to the same expert
        int32_t *sie = a.slot_in_expert + (int64_t)t * a.K;
        int v[EPX_MAX_TOPK];
#pragma unroll
        for (int k = 0; k < EPX_MAX_TOPK; ++k) {
            v[k] = -1;
            const int e = ek[k];
            if (k < a.K && e >= 0) {
                int p = s.pre[e] + wave_rank(a, s, tile_base, tt, k, e);
                for (int w2 = 0; w2 < w; ++w2)
                    p += s.ecnt[w2 * a.E + e];
                v[k] = p;
            }
        }
        if ((a.K & 3) == 0) {
#pragma unroll
            for (int k0 = 0; k0 < EPX_MAX_TOPK; k0 += 4)
                if (k0 < a.K)
                    *reinterpret_cast<u32x4 *>(sie + k0) = u32x4{
                        (uint32_t)v[k0], (uint32_t)v[k0 + 1], (uint32_t)v[k0 + 2], (uint32_t)v[k0 + 3]};
        } else {
#pragma unroll
            for (int k = 0; k < EPX_MAX_TOPK; ++k)
                if (k < a.K)
                    sie[k] = v[k];
        }
    }
    // channel c ends at min((c+1)*ceil(T/C), T); the tile holding token end-1
    // writes the channel's column
    if (a.channel_prefix) {
        const int64_t span = ((int64_t)a.T + a.C - 1) / a.C;
        Walk it(tid, blockDim.x, a.C);
        for (int i = tid; i < a.R * a.C; i += blockDim.x, it.next()) {
            const int r = it.row, c = it.col;
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
