// dispatch.hip -- high-throughput dispatch (pack + permute, optional FP8) and
// the low-latency fixed-slot dispatch.
//
// One wave (64 lanes) per token. The wave first issues the loads of the
// token's row of x (16 bytes per lane per vector; quantising it to FP8 in
// registers when asked), then works out the token's destination rows while
// those loads are in flight, then writes the row to every destination with
// 16-byte stores: x is read from HBM once and each destination costs exactly
// one row write. Destination rows live in lanes and are broadcast with
// readlane, so the kernel needs no LDS and no barrier. The stores follow the
// paced sweep (dispatch_device.h): in ascending output order, each held until
// the wall clock reaches its place, so that the many waves' rows reach HBM
// as one sequential front rather than as random writes.
//
// [P2] "DeepEP 学习笔记" (DeepEP study notes), "dispatch 过程": a token goes,
// in token order, to every rank is_token_in_rank marks, together with its
// source index, top-k indices and weights. [P2] "DeepEP v2": one full
// activation per destination rank. [P1] "事件驱动 EP 内核的调度策略与零拷贝
// 通信", "高吞吐量模式：协调阶段与紧凑缓冲区": exact-size receive buffer, then
// a local permute into contiguous per-expert blocks. On one GPU the pack and
// the permute store the same register copy of the row, so the permute costs
// no second read. [P1] "低延迟模式：固定缓冲区与信号槽机制": fixed per-
// (source, expert) regions, FP8 payload. [P3] "DeepSeek DeepEP探索：低延迟分发",
// 3.2: the local path is an unrolled 16-byte vector copy with non-caching
// loads -- kept here as streaming 16-byte loads.
#include <atomic>

#include "dispatch_device.h"

namespace epx {
namespace {

template <bool FP8, int NV, bool CHUNKED>
__global__ __launch_bounds__(kWave) void dispatch_kernel(DispatchArgs a)
{
    const uint64_t t_entry = wall_clock64();
    const int t = CHUNKED ? a.t_begin + (int)blockIdx.x : (int)blockIdx.x;
    const int lane = threadIdx.x;
    if (blockIdx.x == 0 && lane == 0)
        stamp_launch(a, t_entry);
    const int64_t tk = (int64_t)t * a.K;
    const uint16_t *xrow = a.x + (size_t)t * a.h;

    // first pass of the row: issued before anything else, quantised (FP8)
    // once the destinations have been worked out
    typename std::conditional<FP8, RowFp8<NV>, RowBf16<NV>>::type row;
    row.load(reinterpret_cast<const u32x4 *>(xrow), 0, FP8 ? a.h >> 4 : a.h >> 3);

    // destinations from the layout's offsets and in-rank / in-expert ranks
    const int64_t e = lane < a.K ? a.topk_idx[tk + lane] : -1;
    const bool valid = e >= 0 && e < a.E;
    int64_t send_r = -1, recv_r = -1;
    if (a.send_x && lane < a.R) {
        const int p = a.pos_in_rank[(int64_t)t * a.R + lane];
        if (p >= 0)
            send_r = (int64_t)a.rank_off[lane] + p;
    }
    if (valid)
        recv_r = (int64_t)a.exp_off[(int)e] + a.slot_in_expert[tk + lane];
    const int64_t nsend = (a.sweep_bpt && a.send_x) ? a.rank_off[a.R] : 0;
    dispatch_token<FP8, CHUNKED>(a, t, row, xrow, e, send_r, recv_r, nsend, t_entry);
}

// Low-latency dispatch, one launch. Block b handles G consecutive tokens
// (G = 1 for decode batches up to 256 tokens, doubling with T up to 8, so
// the grid stays near one block per compute unit) with kLLWaves waves, 8/G
// per token. Every block histograms all T*K entries in LDS -- the full
// histogram gives the count slots, the part before the block's first token
// gives its slots, and the block's own earlier tokens (their entries kept
// in LDS) the rest; LDS atomics only add, so the result does not depend on
// their order, and the total counting work is (blocks) x T*K, linear in T
// up to T = 8 x 256. The row is cut into 1024-channel slices (eight
// 128-channel scale groups): a token's waves load, quantise and store its
// slices in turn to every destination of the token, so the row is read
// once, each element is quantised once, and a decode batch's few tokens
// still spread their work over many waves.
constexpr int kLLWaves = 8;
constexpr int kLLHistBatch = 2;

// Tokens per block of the low-latency kernel for a batch of T tokens.
inline int ll_tokens_per_block(int T)
{
    int g = 1;
    while (g < kLLWaves && (int64_t)g * 256 < T)
        g <<= 1;
    return g;
}

template <bool FP8>
__global__ __launch_bounds__(kLLWaves * kWave) void ll_dispatch_kernel(LLArgs a, int G)
{
    extern __shared__ int hist[];  // [E] all entries, [E] entries before the block's tokens,
                                   // [G][K] the experts of the block's tokens
    const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid >> 6;
    const int nthreads = kLLWaves * kWave;
    const int wpt = kLLWaves / G, j = w / wpt, wj = w - j * wpt;  // waves per token, token, wave of it
    const int t0 = blockIdx.x * G, t = t0 + j;
    int *hist_all = hist, *hist_before = hist + a.E, *blk_e = hist + 2 * a.E;
    const bool have_token = t < a.T;
    const int64_t tk = (int64_t)t * a.K;
    const uint16_t *xrow = a.x + (size_t)(have_token ? t : 0) * a.h;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(xrow);

    // the token's experts, lane k holding entry k, and the wave's first
    // slice go out first
    const int64_t ek = (have_token && lane < a.K) ? a.topk_idx[tk + lane] : -1;
    typename std::conditional<FP8, RowFp8<1>, RowBf16<2>>::type row;
    constexpr int per = decltype(row)::kPerPass;  // 1024 channels
    const int nitems = FP8 ? a.h >> 4 : a.h >> 3;
    const int nslices = (nitems + per - 1) / per;
    row.load(src, wj * per, have_token ? nitems : 0);  // zeros past the row

    // kLLHistBatch entries per thread in flight together (clamped, always
    // valid addresses, masked afterwards) instead of a load and a wait per
    // entry: T = 128 / 512 / 1024 take 5.42 / 9.33 / 15.8 us against 5.48 /
    // 9.6 / 16.2 (four at a time, with redundant clamped loads at T = 128,
    // was slower). The first batch goes out with the token's own entries,
    // before the LDS is cleared, so both loads' latencies overlap.
    const int64_t n_ent = (int64_t)a.T * a.K, before = (int64_t)t0 * a.K;
    int64_t ev[kLLHistBatch];
#pragma unroll
    for (int q = 0; q < kLLHistBatch; ++q)
        ev[q] = n_ent > 0 ? a.topk_idx[min((int64_t)tid + (int64_t)q * nthreads, n_ent - 1)] : -1;

    for (int i = tid; i < 2 * a.E; i += nthreads)
        hist[i] = 0;
    if (wj == 0 && lane < a.K)
        blk_e[j * a.K + lane] = (int)ek;  // -1 past the last token
    __syncthreads();
    for (int64_t i0 = tid; i0 < n_ent; i0 += (int64_t)kLLHistBatch * nthreads) {
        if (i0 != tid) {
#pragma unroll
            for (int q = 0; q < kLLHistBatch; ++q)
                ev[q] = a.topk_idx[min(i0 + (int64_t)q * nthreads, n_ent - 1)];
        }
#pragma unroll
        for (int q = 0; q < kLLHistBatch; ++q) {
            const int64_t i = i0 + (int64_t)q * nthreads, e = ev[q];
            if (i < n_ent && e != -1) {
                if (e >= 0 && e < a.E) {
                    atomicAdd(&hist_all[e], 1);
                    if (i < before)
                        atomicAdd(&hist_before[e], 1);
                } else if (blockIdx.x == 0) {
                    flag_error(a.err, EPX_DEV_BAD_ROUTE);
                }
            }
        }
    }
    __syncthreads();

    // count slots: every expert's count, written by a spread of blocks
    for (int e = blockIdx.x * nthreads + tid; e < a.E; e += gridDim.x * nthreads) {
        const int64_t region = a.R_buf == 1 ? e : (int64_t)e * a.R + a.src_rank;
        a.ll_count[region] = hist_all[e];
    }
    // the other buffer of a ping-pong pair: its count slots back to empty,
    // ready for the next step without a separate reset
    for (int64_t i = (int64_t)blockIdx.x * nthreads + tid; i < a.n_clear;
         i += (int64_t)gridDim.x * nthreads)
        a.clear_count[i] = -1;
    // fill of this source's regions: entries routed and the fullest region
    if (blockIdx.x == 0 && w == 0 && a.stats) {
        int sum = 0, mx = 0;
        for (int e = lane; e < a.E; e += kWave) {
            sum += hist_all[e];
            mx = max(mx, hist_all[e]);
        }
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            sum += __shfl_xor(sum, d, kWave);
            mx = max(mx, __shfl_xor(mx, d, kWave));
        }
        if (lane == 0) {
            a.stats[0] = sum;
            a.stats[1] = mx;
        }
    }
    if (!have_token)
        return;

    // the token's rows, lane k < K holding entry k's (the same in the
    // token's every wave); its first wave writes the handle and the source
    // index. Slot = entries before the block + entries of the block's
    // earlier tokens + earlier entries of this row, with the same expert.
    const bool valid = lane < a.K && ek >= 0 && ek < a.E;
    int rep = 0;
    for (int k2 = 0; k2 < a.K; ++k2)
        rep += (k2 < lane && readlane64(ek, k2) == ek);
    for (int i = 0; i < j * a.K; ++i)
        rep += (blk_e[i] == (int)ek);
    int dst = -1;
    if (valid) {
        const int slot = hist_before[ek] + rep;
        if (slot < a.cap) {
            const int64_t region = a.R_buf == 1 ? ek : ek * a.R + a.src_rank;
            dst = (int)(region * a.cap + slot);
        } else if (wj == 0) {
            flag_error(a.err, EPX_DEV_OVERFLOW);
        }
    }
    if (wj == 0 && lane < a.K) {
        a.pos_ll[tk + lane] = dst;
        if (dst >= 0)
            a.ll_src[dst] = t;
    }
    const uint64_t dbits = uniform64(__ballot(dst >= 0));
    const size_t row_bytes = FP8 ? (size_t)a.h : (size_t)a.h * 2;
    const int ld_s = scale_stride(a.h);
    for (int sl = wj; sl < nslices; sl += wpt) {
        if (sl != wj)
            row.load(src, sl * per, nitems);
        row.quantise(sl * per, nitems);
        for (uint64_t m = dbits; m; m &= m - 1) {
            const int r = readlane(dst, __builtin_ctzll(m));
            if constexpr (FP8)
                row.store(reinterpret_cast<uint8_t *>(a.ll_x) + (size_t)r * row_bytes,
                          a.ll_scales + (size_t)r * ld_s, sl * per, nitems);
            else
                row.store(reinterpret_cast<char *>(a.ll_x) + (size_t)r * row_bytes, sl * per,
                          nitems);
        }
    }
}

// The receiver's local permute in one launch: one wave per received row n,
// which loads the row (16 bytes per lane per vector) and its side row (at
// most 64 vectors, e.g. its FP8 scales), works out its destinations from
// lane k < K -- entry k's local expert e, row exp_off[e] + slot[n, k] --
// and stores both to every destination, with the handle and the source row.
// Rows are copied bit for bit (any payload); nontemporal stores: nothing
// here reads them back.
template <int NV>
__global__ __launch_bounds__(kWave) void permute_kernel(PermuteArgs a)
{
    const int n = blockIdx.x, lane = threadIdx.x;
    const int64_t nk = (int64_t)n * a.K;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(static_cast<const char *>(a.rows) +
                                                        (size_t)n * a.row_vecs * 16);
    RowBf16<NV> row;
    row.load(src, 0, a.row_vecs);
    const u32x4 side = lane < a.side_vecs
                           ? load16_stream(static_cast<const char *>(a.side) +
                                           ((size_t)n * a.side_vecs + lane) * 16)
                           : u32x4{0u, 0u, 0u, 0u};
    const int64_t e = lane < a.K ? a.idx[nk + lane] : -1;
    int dst = -1;
    if (lane < a.K) {
        if (e >= 0 && e < a.L) {
            const int64_t r = (int64_t)a.exp_off[(int)e] + a.slot[nk + lane];
            if (r >= 0 && r < a.cap)
                dst = (int)r;
            else
                flag_error(a.err, EPX_DEV_OVERFLOW);
        } else if (e != -1) {
            flag_error(a.err, EPX_DEV_BAD_ROUTE);
        }
        a.pos[nk + lane] = dst;
        if (dst >= 0)
            a.src_row[dst] = n;
    }
    const uint64_t dbits = uniform64(__ballot(dst >= 0));
    char *out = static_cast<char *>(a.out_rows);
    for (int v0 = 0; v0 < a.row_vecs; v0 += RowBf16<NV>::kPerPass) {
        if (v0 > 0)
            row.load(src, v0, a.row_vecs);
        for (uint64_t m = dbits; m; m &= m - 1) {
            const int r = readlane(dst, __builtin_ctzll(m));
            row.template store<StorePolicy::NT>(out + (size_t)r * a.row_vecs * 16, v0,
                                                a.row_vecs);
        }
    }
    if (a.side_vecs > 0)
        for (uint64_t m = dbits; m; m &= m - 1) {
            const int r = readlane(dst, __builtin_ctzll(m));
            if (lane < a.side_vecs)
                store16_stream(static_cast<char *>(a.out_side) +
                                   ((size_t)r * a.side_vecs + lane) * 16, side);
        }
}

__global__ __launch_bounds__(kWave) void fill_lines_kernel(u32x4 *p, uint32_t v)
{
    u32x4 *blk = p + (size_t)blockIdx.x * (kFillBlockBytes / 16);
    const u32x4 val = u32x4{v, v, v, v};
#pragma unroll
    for (int j = 0; j < (int)(kFillBlockBytes / 16 / kWave); ++j)
        blk[j * kWave + threadIdx.x] = val;
}

__global__ void fill_i32_kernel(int32_t *p, int64_t n, int32_t v)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

}  // namespace


// One-wave blocks of dispatch_kernel<FP8, NV, CHUNKED> a compute unit holds
// at once (the occupancy query, asked once per instantiation; 0 if it fails).
template <bool FP8, int NV, bool CHUNKED>
static int dispatch_blocks_per_cu()
{
    static std::atomic<int> cache{-1};
    int n = cache.load(std::memory_order_relaxed);
    if (n >= 0)
        return n;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, dispatch_kernel<FP8, NV, CHUNKED>, kWave,
                                                     0) != hipSuccess)
        n = 0;
    n = n < 0 ? 0 : n;
    cache.store(n, std::memory_order_relaxed);
    return n;
}

// A paced sweep needs every wave of a launch on the chip at once: a wave
// held back for a late row keeps its place, so a wave that found no place
// would wait behind it (such a wave stores unpaced: the late-wave check).
// Up to one round of waves, one launch paces the whole sweep; beyond, the
// tokens go in chunks of consecutive tokens, each its own launch sweeping
// its own rows, sized to the round the occupancy query reports for the
// chunked kernel, at 93% of the set rate (each chunk's sweep shares HBM
// with the loads of its own rows). Unpaced, or when the query fails, one
// launch takes all tokens. (One launch of all chunks' waves, each later
// round's rows due after the estimated rows of the rounds before it on one
// clock, was measured on the FP8 prefill at 429-450 us, no better than
// unpaced: a round's waves find places only as the previous round's last
// rows go out, and the rows due before their loads return go out as one
// burst that turns the front back into random writes.)
// Chunk size as a fraction of the round the occupancy query reports (the
// whole round: a wave that still finds no place is caught by the late-wave
// check and stores unpaced), and the chunks' sweep rate as a fraction of
// the set rate. Measured on the FP8 prefill (T = 16384, h = 7168, E = 256,
// R = 64): four chunks of a full round 402-405 us against 413-414 us for
// five of 7/8 of it; with four chunks, their schedules started when ready,
// the best effective chunk rate was ~5670 GB/s (398-401 us; 5490: 402-406,
// 5850: 418-423); started 3 us plus the chunk's x-row time after entry,
// 385-393 us at 93% of 6300-6500 (406 us at 93% of 6700).
constexpr int64_t kChunkRoundPermille = 1000;
constexpr int64_t kChunkRatePermille = 930;

template <bool FP8, int NV>
static void launch_dispatch_nv(const DispatchArgs &a, int cus, std::atomic<unsigned> *seq,
                               hipStream_t stream)
{
    DispatchArgs b = a;
    b.t_begin = 0;
    b.t_count = 0;
    b.stamp_slot = next_stamp_slot(seq);
    if (a.sweep_bpt == 0 || (int64_t)a.T <= (int64_t)dispatch_blocks_per_cu<FP8, NV, false>() * cus) {
        if (b.sweep_bpt)
            b.start_ticks = (uint32_t)(kDispatchStartUs[FP8] * b.wclk_per_us) +
                            load_ticks(a.T, a.h, b.sweep_bpt);
        hipLaunchKernelGGL((dispatch_kernel<FP8, NV, false>), dim3(a.T), dim3(kWave), 0, stream, b);
        return;
    }
    const int64_t round =
        (int64_t)dispatch_blocks_per_cu<FP8, NV, true>() * cus * kChunkRoundPermille / 1000;
    if (round <= 0) {
        b.sweep_bpt = 0;
        hipLaunchKernelGGL((dispatch_kernel<FP8, NV, false>), dim3(a.T), dim3(kWave), 0, stream, b);
        return;
    }
    const int64_t nchunk = (a.T + round - 1) / round;
    const int64_t size = (a.T + nchunk - 1) / nchunk;
    b.sweep_bpt = a.sweep_bpt * kChunkRatePermille / 1000 > 0
                      ? a.sweep_bpt * kChunkRatePermille / 1000 : 1;
    for (int64_t t0 = 0; t0 < a.T; t0 += size) {
        b.t_begin = (int)t0;
        b.t_count = (int)(a.T - t0 < size ? a.T - t0 : size);
        b.start_ticks = (uint32_t)(kDispatchStartUs[FP8] * b.wclk_per_us) +
                        load_ticks(b.t_count, a.h, b.sweep_bpt);
        if (t0 > 0)
            b.stamp_slot = next_stamp_slot(seq);
        hipLaunchKernelGGL((dispatch_kernel<FP8, NV, true>), dim3((unsigned)b.t_count), dim3(kWave),
                           0, stream, b);
    }
}

hipError_t launch_dispatch(const DispatchArgs &a, bool fp8, int cus, std::atomic<unsigned> *seq,
                           hipStream_t stream)
{
    if (a.T == 0)
        return hipSuccess;
    switch (pick_nv(a.h, fp8) + (fp8 ? 100 : 0)) {
    case 8: launch_dispatch_nv<false, 8>(a, cus, seq, stream); break;
    case 14: launch_dispatch_nv<false, 14>(a, cus, seq, stream); break;
    case 16: launch_dispatch_nv<false, 16>(a, cus, seq, stream); break;
    case 104: launch_dispatch_nv<true, 4>(a, cus, seq, stream); break;
    case 107: launch_dispatch_nv<true, 7>(a, cus, seq, stream); break;
    default: launch_dispatch_nv<true, 8>(a, cus, seq, stream); break;
    }
    return hipGetLastError();
}

template <bool FP8>
static void launch_ll(const LLArgs &a, hipStream_t stream)
{
    const int G = ll_tokens_per_block(a.T);
    const dim3 grid(a.T > 0 ? (a.T + G - 1) / G : 1);
    const size_t lds = sizeof(int) * (2 * (size_t)a.E + (size_t)G * a.K);
    hipLaunchKernelGGL((ll_dispatch_kernel<FP8>), grid, dim3(kLLWaves * kWave), lds, stream, a, G);
}

hipError_t launch_ll_dispatch(const LLArgs &a, bool fp8, hipStream_t stream)
{
    if (fp8)
        launch_ll<true>(a, stream);
    else
        launch_ll<false>(a, stream);
    return hipGetLastError();
}

// LDS reserved by each one-wave block of the permute (the kernel uses none),
// capping the blocks that share a compute unit's 160 KB and so the rows in
// flight. Measured on MI355X: bf16 rows of h = 7168 (29 811 rows into 8
// experts) 161 us at the 20 blocks per CU their registers allow, 154 us at
// five (three: 160 us); rows of h = 4096 (40 960 rows) 124 us at 32, 119 us
// at eight. FP8 rows, which carry scale rows, are fastest uncapped (81 us;
// 85 at five).
constexpr size_t kPermuteLdsLarge = 32768;  // rows over 512 vectors: 5 per CU
constexpr size_t kPermuteLdsSmall = 20480;  // rows up to 512 vectors: 8 per CU

hipError_t launch_permute(const PermuteArgs &a, hipStream_t stream)
{
    if (a.N == 0)
        return hipSuccess;
    const dim3 grid((unsigned)a.N), block(kWave);
    const bool small = a.row_vecs <= 8 * kWave;
    const size_t lds = a.side_vecs > 0 ? 0 : small ? kPermuteLdsSmall : kPermuteLdsLarge;
    if (small)
        hipLaunchKernelGGL(permute_kernel<8>, grid, block, lds, stream, a);
    else if (a.row_vecs <= 14 * kWave)
        hipLaunchKernelGGL(permute_kernel<14>, grid, block, lds, stream, a);
    else
        hipLaunchKernelGGL(permute_kernel<16>, grid, block, lds, stream, a);
    return hipGetLastError();
}

hipError_t launch_fill_lines(void *p, size_t n, uint32_t v, hipStream_t stream)
{
    const size_t blocks = n / kFillBlockBytes;
    if (blocks == 0)
        return hipSuccess;
    if (blocks > 0x7FFFFFFFu)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(fill_lines_kernel, dim3((unsigned)blocks), dim3(kWave), 0, stream,
                       static_cast<u32x4 *>(p), v);
    return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t *p, int64_t n, int32_t v, hipStream_t stream)
{
    if (n <= 0)
        return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256),
                       0, stream, p, n, v);
    return hipGetLastError();
}

}  // namespace epx
