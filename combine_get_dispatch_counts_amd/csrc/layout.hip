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
//            likewise per rank (the OR deduplicates ranks for free). A
//            token's rank inside the tile is then the earlier waves' count
//            plus popcount(mask & lanes below it). The block writes
//            is_token_in_rank and these tile-local ranks straight into
//            pos_in_rank / slot_in_expert / channel_prefix, and the tile's
//            counts into the workspace [tile, E + R].
//   finalize one block per tile again: sums the counts of the tiles before
//            it (a few KB from L2), scans all tiles' totals into exp_off /
//            rank_off in LDS and adds the tile's prefix to the tile-local
//            ranks. Block 0 writes the counts, offsets and totals.
// A wave in which some token lists one expert twice counts earlier entries
// directly instead, so a slot stays "entries before (t,k)" exactly.
#include "epx_device.h"
#include "epx_internal.h"

namespace epx {
namespace {

constexpr int W = kLayoutWaves;

struct CountLds {
    uint64_t *emask;  // [W][E]
    uint64_t *rmask;  // [W][R]
    int *ecnt;        // [W][E] entries of wave w routed to e
    int *wpre_e;      // [W][E] entries of the tile's earlier waves routed to e
    int *wpre_r;      // [W][R] tokens of the tile's earlier waves going to r
    int *dupwave;     // [W] 1 if the wave has a row with a repeated expert
};

__host__ __device__ inline size_t count_lds_bytes(int E, int R)
{
    return sizeof(uint64_t) * ((size_t)W * E + (size_t)W * R) +
           sizeof(int) * (2 * (size_t)W * E + (size_t)W * R + W);
}

__device__ CountLds carve_count(char *base, int E, int R)
{
    CountLds s;
    s.emask = reinterpret_cast<uint64_t *>(base);
    s.rmask = s.emask + (size_t)W * E;
    s.ecnt = reinterpret_cast<int *>(s.rmask + (size_t)W * R);
    s.wpre_e = s.ecnt + (size_t)W * E;
    s.wpre_r = s.wpre_e + (size_t)W * E;
    s.dupwave = s.wpre_r + (size_t)W * R;
    return s;
}

__host__ __device__ inline size_t finalize_lds_bytes(int E, int R)
{
    return sizeof(int) * (2 * (size_t)(E + R) + (E + R + 2));  // pre, tot, off
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

template <int KMAX>
__global__ __launch_bounds__(kLayoutTile) void layout_count_kernel(LayoutArgs a)
{
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const CountLds s = carve_count(lds, a.E, a.R);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int tile_base = blockIdx.x * kLayoutTile;
    const int ntok = min(kLayoutTile, a.T - tile_base);
    const int t = tile_base + tid;

    int ek[KMAX];
    load_row_experts<KMAX>(a, t, ek);
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
    if (bad)
        flag_error(a.err, EPX_DEV_BAD_ROUTE);
    for (uint64_t m = rbits; m; m &= m - 1) {
        const int r = __builtin_ctzll(m);
        atomicOr(reinterpret_cast<unsigned long long *>(&s.rmask[w * a.R + r]), bit);
    }
    if (__any(dup) && lane == 0)
        s.dupwave[w] = 1;
    __syncthreads();

    // wave prefixes inside the tile, and the tile's counts
    int32_t *cnt = a.tile_cnt + (int64_t)blockIdx.x * (a.E + a.R);
    for (int e = tid; e < a.E; e += blockDim.x) {
        int run = 0;
        for (int w2 = 0; w2 < W; ++w2) {
            s.wpre_e[w2 * a.E + e] = run;
            run += s.ecnt[w2 * a.E + e];
        }
        cnt[e] = run;
    }
    for (int r = tid; r < a.R; r += blockDim.x) {
        int run = 0;
        for (int w2 = 0; w2 < W; ++w2) {
            s.wpre_r[w2 * a.R + r] = run;
            run += __popcll(s.rmask[w2 * a.R + r]);
        }
        cnt[a.E + r] = run;
    }
    __syncthreads();

    if (t < a.T) {
        const uint64_t below = lanes_below(lane);
        write_rank_row(a.is_token_in_rank + (int64_t)t * a.R, rbits, a.R);
        // tile-local rank of t in each rank it goes to, else -1: the row is
        // cleared first, then only the (at most K) ranks t goes to are set
        int32_t *pir = a.pos_in_rank + (int64_t)t * a.R;
        if ((a.R & 3) == 0) {
            for (int r0 = 0; r0 < a.R; r0 += 4)
                *reinterpret_cast<u32x4 *>(pir + r0) = u32x4{~0u, ~0u, ~0u, ~0u};
        } else {
            for (int r = 0; r < a.R; ++r)
                pir[r] = -1;
        }
        uint64_t m = rbits;
#pragma unroll
        for (int i = 0; i < KMAX; ++i) {
            if (m) {
                const int r = __builtin_ctzll(m);
                m &= m - 1;
                pir[r] = s.wpre_r[w * a.R + r] + __popcll(s.rmask[w * a.R + r] & below);
            }
        }
        // tile-local slot of each entry, else -1
        int32_t *sie = a.slot_in_expert + (int64_t)t * a.K;
        int v[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const int e = ek[k];
            v[k] = e >= 0 ? s.wpre_e[w * a.E + e] + wave_rank(a, s, tile_base, tid, k, e) : -1;
        }
        if ((a.K & 3) == 0) {
#pragma unroll
            for (int k0 = 0; k0 < KMAX; k0 += 4)
                if (k0 < a.K)
                    *reinterpret_cast<u32x4 *>(sie + k0) = u32x4{
                        (uint32_t)v[k0], (uint32_t)v[k0 + 1], (uint32_t)v[k0 + 2], (uint32_t)v[k0 + 3]};
        } else {
#pragma unroll
            for (int k = 0; k < KMAX; ++k)
                if (k < a.K)
                    sie[k] = v[k];
        }
    }

    // tile-local part of the channel columns this tile owns
    if (a.channel_prefix) {
        Walk it(tid, blockDim.x, a.C);
        for (int i = tid; i < a.R * a.C; i += blockDim.x, it.next()) {
            const int r = it.row;
            const int64_t end = channel_end(a, it.col);
            if (end <= tile_base || end > tile_base + ntok)
                continue;
            const int n = (int)(end - tile_base);
            int v = 0;
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

template <int KMAX>
__global__ __launch_bounds__(kLayoutTile) void layout_finalize_kernel(LayoutArgs a)
{
    extern __shared__ __attribute__((aligned(16))) int fin[];
    const int b = blockIdx.x, tid = threadIdx.x;
    const int ER = a.E + a.R;
    int *pre = fin, *tot = fin + ER, *off = fin + 2 * ER;
    const int tile_base = b * kLayoutTile;
    const int t = tile_base + tid;

    // this token's experts and its tile-local rows go out first: nothing
    // below the scan has to wait for memory except these loads
    int ek[KMAX];
    if (a.ntiles > 0)
        load_row_experts<KMAX>(a, t, ek);
    const bool vec_rows = (a.R & 3) == 0;
    const int tl = min(t, a.T - 1);  // clamped: loads stay inside the arrays
    int32_t *pir = a.pos_in_rank + (int64_t)tl * a.R;
    int32_t *sie = a.slot_in_expert + (int64_t)tl * a.K;
    u32x4 prow[EPX_MAX_RANKS / 4];
    int srow[KMAX];
    if (a.ntiles > 0) {
        if (vec_rows) {
#pragma unroll
            for (int j = 0; j < EPX_MAX_RANKS / 4; ++j)
                if (4 * j < a.R)
                    prow[j] = *reinterpret_cast<const u32x4 *>(pir + 4 * j);
        }
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            srow[k] = (k < a.K) ? sie[k] : -1;
    }

    // counts in earlier tiles and over all tiles, per expert then per rank;
    // 16 loads in flight per thread, from clamped rows masked afterwards
    for (int i = tid; i < ER; i += blockDim.x) {
        int p = 0, q = 0;
        for (int j0 = 0; j0 < a.ntiles; j0 += 16) {
            int v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u)
                v[u] = a.tile_cnt[(int64_t)min(j0 + u, a.ntiles - 1) * ER + i];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int c = (j0 + u < a.ntiles) ? v[u] : 0;
                p += (j0 + u < b) ? c : 0;
                q += c;
            }
        }
        pre[i] = p;
        tot[i] = q;
    }
    __syncthreads();
    if (tid < kWave)
        wave_exclusive_scan(tot, a.E, off);
    else if (tid < 2 * kWave)
        wave_exclusive_scan(tot + a.E, a.R, off + a.E + 1);
    __syncthreads();

    if (b == 0) {
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
        if (a.ntiles == 0 && a.channel_prefix)
            for (int i = tid; i < a.R * a.C; i += blockDim.x)
                a.channel_prefix[i] = 0;
    }
    if (a.ntiles == 0)
        return;

    // add the tile prefix to the tile-local ranks (already in registers)
    const int ntok = min(kLayoutTile, a.T - tile_base);
    if (t < a.T) {
        if (vec_rows) {
#pragma unroll
            for (int j = 0; j < EPX_MAX_RANKS / 4; ++j) {
                const int r = 4 * j;
                if (r < a.R) {
                    u32x4 o = prow[j];
                    o.x = (int)o.x >= 0 ? o.x + pre[a.E + r] : o.x;
                    o.y = (int)o.y >= 0 ? o.y + pre[a.E + r + 1] : o.y;
                    o.z = (int)o.z >= 0 ? o.z + pre[a.E + r + 2] : o.z;
                    o.w = (int)o.w >= 0 ? o.w + pre[a.E + r + 3] : o.w;
                    *reinterpret_cast<u32x4 *>(pir + r) = o;
                }
            }
        } else {
            for (int r = 0; r < a.R; ++r) {
                const int v = pir[r];
                if (v >= 0)
                    pir[r] = v + pre[a.E + r];
            }
        }
        if ((a.K & 3) == 0) {
#pragma unroll
            for (int k0 = 0; k0 < KMAX; k0 += 4) {
                if (k0 < a.K) {
                    int o[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        o[j] = ek[k0 + j] >= 0 ? srow[k0 + j] + pre[ek[k0 + j]] : srow[k0 + j];
                    *reinterpret_cast<u32x4 *>(sie + k0) =
                        u32x4{(uint32_t)o[0], (uint32_t)o[1], (uint32_t)o[2], (uint32_t)o[3]};
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < KMAX; ++k)
                if (k < a.K && ek[k] >= 0)
                    sie[k] = srow[k] + pre[ek[k]];
        }
    }
    if (a.channel_prefix) {
        Walk it(tid, blockDim.x, a.C);
        for (int i = tid; i < a.R * a.C; i += blockDim.x, it.next()) {
            const int64_t end = channel_end(a, it.col);
            if (end > tile_base && end <= tile_base + ntok)
                a.channel_prefix[i] += pre[a.E + it.row];
        }
    }
}

}  // namespace

size_t layout_workspace_bytes(int T, int E, int R)
{
    const size_t ntiles = ((size_t)T + kLayoutTile - 1) / kLayoutTile;
    return ntiles * (size_t)(E + R) * sizeof(int32_t);
}

template <int KMAX>
static void launch_layout_k(const LayoutArgs &a, hipStream_t stream)
{
    if (a.ntiles > 0)
        hipLaunchKernelGGL((layout_count_kernel<KMAX>), dim3(a.ntiles), dim3(kLayoutTile),
                           count_lds_bytes(a.E, a.R), stream, a);
    hipLaunchKernelGGL((layout_finalize_kernel<KMAX>), dim3(a.ntiles > 0 ? a.ntiles : 1),
                       dim3(kLayoutTile), finalize_lds_bytes(a.E, a.R), stream, a);
}

// The per-token top-k loops are unrolled to KMAX; the common K <= 8 gets a
// small kernel (instruction fetch matters for these short, few-block kernels).
hipError_t launch_layout(const LayoutArgs &a, hipStream_t stream)
{
    if (a.K <= 8)
        launch_layout_k<8>(a, stream);
    else
        launch_layout_k<EPX_MAX_TOPK>(a, stream);
    return hipGetLastError();
}

}  // namespace epx
