// dispatch.hip -- high-throughput dispatch (pack + permute, optional FP8) and
// the low-latency fixed-slot dispatch.
//
// One wave (64 lanes) per token. The wave first issues the loads of the
// token's row of x (16 bytes per lane per vector; quantising it to FP8 in
// registers when asked), then works out the token's destination rows while
// those loads are in flight, then writes the row to every destination with
// 16-byte stores: x is read from HBM once and each destination costs exactly
// one row write. Destination rows live in lanes and are broadcast with
// readlane, so the kernel needs no LDS and no barrier.
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
#include <type_traits>

#include "epx_device.h"
#include "epx_internal.h"

namespace epx {
namespace {

// Per pass a lane holds NV items of the row: 16-byte bf16 vectors (8
// channels each) or 16-channel FP8 segments. NV is picked per h at launch so
// the row of the common hidden sizes fits one pass with no idle registers:
// bf16 NV = 8 (h <= 4096), 14 (h <= 7168), 16 (larger h, several passes);
// fp8 NV = 4, 7, 8 over the same ranges.

__device__ __forceinline__ int readlane(int v, int lane)
{
    return __builtin_amdgcn_readlane(v, lane);
}

// A 64-bit value of one lane, both halves moved as unsigned.
__device__ __forceinline__ int64_t readlane64(int64_t v, int lane)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), lane);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}


// One pass of a bf16 row held in registers: vector v of the pass is lane +
// 64*u for u < NV.
template <int NV>
struct RowBf16 {
    static constexpr int kPerPass = NV * kWave;
    u32x4 r[NV];
    __device__ __forceinline__ void load(const u32x4 *src, int v0, int nvec)
    {
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int v = v0 + u * kWave + lane_id();
            r[u] = (v < nvec) ? load16_stream(src + v) : u32x4{0u, 0u, 0u, 0u};
        }
    }
    __device__ __forceinline__ void quantise(int, int) {}
    __device__ __forceinline__ void store(char *dst_row, int v0, int nvec) const
    {
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int v = v0 + u * kWave + lane_id();
            if (v < nvec)
                store16_wt(dst_row + (size_t)v * 16, r[u]);
        }
    }
};

// x / s for a group scale s with rs = 1/s (both IEEE divisions, once per
// group): the product x*rs corrected by one fused residual step (Markstein's
// construction), with the sign of zero taken from x. Run over every pair of
// a finite bf16 x and a finite bf16 group maximum amax >= |x| on gfx950,
// this gives the same e4m3 code as the IEEE quotient x / s in all
// 1,065,402,240 cases (the quotients themselves differ only below the fp32
// normal range, which every e4m3 rounding sends to a signed zero).
__device__ __forceinline__ float quotient(float x, float s, float rs)
{
    const float q0 = x * rs;
    const float e = __builtin_fmaf(-q0, s, x);
    return __builtin_copysignf(__builtin_fmaf(e, rs, q0), x);
}

// e4m3 codes of two fp32 values placed in byte pair HI of w: gfx950's
// OCP E4M3FN convert, nearest even, which gives the format's code for every
// fp32 of magnitude <= 464 (checked on all of them).
template <bool HI>
__device__ __forceinline__ int cvt2_e4m3(float a, float b, int w)
{
    return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, w, HI);
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Largest magnitude pattern among the 16 bf16 values of a segment: an
// unsigned max over the patterns with the sign cleared, which orders like
// the magnitudes; an Inf or NaN pattern (>= 0x7F80) beats every finite one.
__device__ __forceinline__ uint32_t seg_abs_max_bits(const uint32_t (&p)[8])
{
    u16x2 m = __builtin_bit_cast(u16x2, p[0] & 0x7FFF7FFFu);
#pragma unroll
    for (int i = 1; i < 8; ++i)
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, p[i] & 0x7FFF7FFFu));
    return m.x > m.y ? m.x : m.y;
}

// One pass of an FP8 row: segment sg = s0 + lane + 64*u covers channels
// [16 sg, 16 sg + 16); a 128-channel group is 8 adjacent lanes, reduced with
// xor shuffles. Codes: e4m3 of x / s with s = max(amax, 1e-4) / 448 (IEEE),
// |x / s| <= 448 up to one rounding. A group holding an Inf or NaN takes a
// separate branch (uniform over the wave, almost never taken) that divides
// outright: amax over the non-NaN values, NaN quotients coded 0x7F.
// Scale rows are scale_stride(h) floats apart, a whole number of 128-byte
// lines, and written in full (zeros past the last group): a scattered row
// that ends inside a line leaves that line to be merged in memory with a
// neighbour written at another time, which costs far more than the pad.
template <int NV>
struct RowFp8 {
    static constexpr int kPerPass = NV * kWave;
    u32x4 q[NV];
    u32x4 lo[NV], hi[NV];  // the bf16 pass as loaded (lo: channels 0..7, hi: 8..15)
    u32x4 sv;   // scales of groups s0/8 + 4*lane .. +3 of the pass, +0 past the last group
    int n_sv;   // lanes holding a slice of the (padded) scale row in this pass
    // Issue the pass's loads; quantise() consumes them, so work placed in
    // between overlaps their latency.
    __device__ __forceinline__ void load(const u32x4 *src, int s0, int nseg)
    {
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int sg = s0 + u * kWave + lane_id();
            const bool active = sg < nseg;  // uniform over each 8-lane group
            lo[u] = active ? load16_stream(src + 2 * sg) : u32x4{0u, 0u, 0u, 0u};
            hi[u] = active ? load16_stream(src + 2 * sg + 1) : u32x4{0u, 0u, 0u, 0u};
        }
    }
    __device__ __forceinline__ void quantise(int s0, int nseg)
    {
        float sc[NV];
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const uint32_t p[8] = {lo[u].x, lo[u].y, lo[u].z, lo[u].w,
                                   hi[u].x, hi[u].y, hi[u].z, hi[u].w};
            float f[16];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                f[2 * i] = bf16_lo(p[i]);
                f[2 * i + 1] = bf16_hi(p[i]);
            }
            uint32_t abits = seg_abs_max_bits(p);
            abits = max(abits, (uint32_t)__shfl_xor((int)abits, 1, kWave));
            abits = max(abits, (uint32_t)__shfl_xor((int)abits, 2, kWave));
            abits = max(abits, (uint32_t)__shfl_xor((int)abits, 4, kWave));
            uint32_t wd[4];
            float s;
            if (__builtin_expect(__ballot(abits >= 0x7F80u) == 0, 1)) {
                s = fmaxf(__uint_as_float(abits << 16), 1e-4f) / 448.0f;
                const float rs = 1.0f / s;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int w = cvt2_e4m3<false>(quotient(f[4 * j], s, rs),
                                                   quotient(f[4 * j + 1], s, rs), 0);
                    wd[j] = (uint32_t)cvt2_e4m3<true>(quotient(f[4 * j + 2], s, rs),
                                                      quotient(f[4 * j + 3], s, rs), w);
                }
            } else {
                float amax = 0.0f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float a = fabsf(f[i]);
                    amax = (a > amax) ? a : amax;  // a NaN never wins
                }
#pragma unroll
                for (int d = 1; d < 8; d <<= 1) {
                    const float o = __shfl_xor(amax, d, kWave);
                    amax = (o > amax) ? o : amax;
                }
                s = fmaxf(amax, 1e-4f) / 448.0f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    uint32_t word = 0;
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const float v = f[4 * j + b] / s;
                        const uint32_t c = (v != v) ? 0x7Fu
                                                    : ((uint32_t)cvt2_e4m3<false>(v, 0.0f, 0) & 0xFFu);
                        word |= c << (8 * b);
                    }
                    wd[j] = word;
                }
            }
            q[u] = u32x4{wd[0], wd[1], wd[2], wd[3]};
            sc[u] = s;
        }
        // Group gl = 4L + j of the pass sits in pass item u = L/2, on the
        // lanes 8*(gl % 8) .. +7; collect four per lane for one store.
        const int L = lane_id(), g0 = s0 >> 3, ngrp = nseg >> 3;
        float g4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int u = 0; u < NV; ++u) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float v = __shfl(sc[u], 8 * (4 * (L & 1) + j), kWave);
                if ((L >> 1) == u && g0 + 4 * L + j < ngrp)
                    g4[j] = v;
            }
        }
        sv = u32x4{__float_as_uint(g4[0]), __float_as_uint(g4[1]), __float_as_uint(g4[2]),
                   __float_as_uint(g4[3])};
        n_sv = min(16, (scale_stride(nseg << 4) - g0) >> 2);
    }
    // Codes of the pass to one destination row, plus that row's slice of
    // the scale row (one 16-byte store by the first lanes).
    __device__ __forceinline__ void store(uint8_t *q_row, float *s_row, int s0, int nseg) const
    {
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int sg = s0 + u * kWave + lane_id();
            if (sg < nseg)
                store16_wt(q_row + (size_t)sg * 16, q[u]);
        }
        if (lane_id() < n_sv)
            store16_wt(s_row + (s0 >> 3) + 4 * lane_id(), sv);
    }
};

// Destination rows of one token, one per lane: lane r holds the rank-major
// row for rank r (bit r of rbits), lane k the expert-major row of entry k
// (bit k of vbits); -1 = skip (capacity overflow, already flagged).
struct Dests {
    uint64_t rbits, vbits;
    int send_row, recv_row;
};

// Write the token's row (the pass held in `row`, plus any further passes
// loaded here) to every destination: send rows in buffer a, recv rows in b.
template <bool FP8, typename Row>
__device__ __forceinline__ void scatter(Row &row, const Dests &d, const uint16_t *xrow, int h,
                                        void *a_x, float *a_s, void *b_x, float *b_s)
{
    const int nvec = h >> 3, nseg = h >> 4, ld_s = scale_stride(h);
    const int per_pass = Row::kPerPass;
    const int nitems = FP8 ? nseg : nvec;
    const size_t row_bytes = FP8 ? (size_t)h : (size_t)h * 2;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(xrow);
    for (int i0 = 0; i0 < nitems; i0 += per_pass) {
        if (i0 > 0) {
            row.load(src, i0, nitems);
            row.quantise(i0, nitems);
        }
        for (uint64_t m = d.rbits; m; m &= m - 1) {
            const int r = readlane(d.send_row, __builtin_ctzll(m));
            if (r < 0)
                continue;
            if constexpr (FP8)
                row.store(static_cast<uint8_t *>(a_x) + (size_t)r * row_bytes,
                          a_s + (size_t)r * ld_s, i0, nseg);
            else
                row.store(static_cast<char *>(a_x) + (size_t)r * row_bytes, i0, nvec);
        }
        for (uint64_t m = d.vbits; m; m &= m - 1) {
            const int r = readlane(d.recv_row, __builtin_ctzll(m));
            if (r < 0)
                continue;
            if constexpr (FP8)
                row.store(static_cast<uint8_t *>(b_x) + (size_t)r * row_bytes,
                          b_s + (size_t)r * ld_s, i0, nseg);
            else
                row.store(static_cast<char *>(b_x) + (size_t)r * row_bytes, i0, nvec);
        }
    }
}

template <bool FP8, int NV>
__global__ __launch_bounds__(kWave) void dispatch_kernel(DispatchArgs a)
{
    const int t = blockIdx.x, lane = threadIdx.x;
    const int64_t tk = (int64_t)t * a.K;
    const uint16_t *xrow = a.x + (size_t)t * a.h;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(xrow);

    // first pass of the row: issued before anything else, quantised (FP8)
    // once the destinations below have been worked out
    typename std::conditional<FP8, RowFp8<NV>, RowBf16<NV>>::type row;
    const int nitems = FP8 ? a.h >> 4 : a.h >> 3;
    row.load(src, 0, nitems);

    // destinations
    const int64_t e = lane < a.K ? a.topk_idx[tk + lane] : -1;
    const bool valid = e >= 0 && e < a.E;
    const int ei = valid ? (int)e : 0;
    Dests d;
    // no send buffer: the permute alone (a receiver arranging its rows)
    d.rbits = a.send_x ? uniform64(wave_or(valid ? (1ull << (ei / a.L)) : 0ull)) : 0ull;
    d.vbits = uniform64(__ballot(valid));
    d.send_row = -1;
    d.recv_row = -1;
    if (lane < a.R && ((d.rbits >> lane) & 1ull)) {
        const int64_t r = (int64_t)a.rank_off[lane] + a.pos_in_rank[(int64_t)t * a.R + lane];
        if (r >= 0 && r < a.send_cap)
            d.send_row = (int)r;
        else
            flag_error(a.err, EPX_DEV_OVERFLOW);
    }
    if (lane < a.K) {
        if (valid) {
            const int64_t r = (int64_t)a.exp_off[ei] + a.slot_in_expert[tk + lane];
            if (r >= 0 && r < a.recv_cap)
                d.recv_row = (int)r;
            else
                flag_error(a.err, EPX_DEV_OVERFLOW);
        }
        a.pos_exp[tk + lane] = d.recv_row;
        if (d.recv_row >= 0)
            a.recv_src[d.recv_row] = t;
    }
    // per send row: source token and the top-k list seen from that rank
    if (d.send_row >= 0) {
        const int64_t row = d.send_row;
        a.send_src[row] = t;
        for (int k = 0; k < a.K; ++k) {
            const int64_t ek = a.topk_idx[tk + k];
            const bool on_r = ek >= 0 && ek < a.E && (int)ek / a.L == lane;
            a.send_topk_idx[row * a.K + k] = on_r ? ek - (int64_t)lane * a.L : -1;
            a.send_topk_w[row * a.K + k] = on_r ? a.topk_w[tk + k] : 0.0f;
        }
    }

    row.quantise(0, nitems);
    scatter<FP8>(row, d, xrow, a.h, a.send_x, a.send_scales, a.recv_x, a.recv_scales);
}

// Low-latency dispatch, one launch. Block t handles token t with kLLWaves
// waves: together they histogram all T*K entries in LDS (decode batches are
// small) -- the full histogram gives the count slots, the part before token
// t gives t's slots; LDS atomics only add, so the result does not depend on
// their order -- then wave w loads and quantises the row itself (the other
// waves' copies come from L2) and writes the entries k with k % kLLWaves ==
// w. A decode batch has few tokens, so one wave per token would leave most
// of the chip idle and each wave writing K rows in turn.
constexpr int kLLWaves = 8;

template <bool FP8, int NV>
__global__ __launch_bounds__(kLLWaves * kWave) void ll_dispatch_kernel(LLArgs a)
{
    extern __shared__ int hist[];  // [E] all entries, [E] entries before token t
    const int t = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1), w = tid >> 6;
    const int nthreads = kLLWaves * kWave;
    int *hist_all = hist, *hist_before = hist + a.E;
    const bool have_token = t < a.T;
    const int64_t tk = (int64_t)t * a.K;
    const uint16_t *xrow = a.x + (size_t)t * a.h;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(xrow);

    // the token's experts, lane k holding entry k, and its row go out first
    const int64_t ek = (have_token && lane < a.K) ? a.topk_idx[tk + lane] : -1;
    typename std::conditional<FP8, RowFp8<NV>, RowBf16<NV>>::type row;
    const int nitems = FP8 ? a.h >> 4 : a.h >> 3;
    if (have_token)
        row.load(src, 0, nitems);

    for (int i = tid; i < 2 * a.E; i += nthreads)
        hist[i] = 0;
    __syncthreads();
    const int64_t n_ent = (int64_t)a.T * a.K;
    for (int64_t i = tid; i < n_ent; i += nthreads) {
        const int64_t e = a.topk_idx[i];
        if (e == -1)
            continue;
        if (e < 0 || e >= a.E) {
            if (t == 0)
                flag_error(a.err, EPX_DEV_BAD_ROUTE);
            continue;
        }
        atomicAdd(&hist_all[e], 1);
        if (i < tk)
            atomicAdd(&hist_before[e], 1);
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

    // this wave's entries: lane k < K with k % kLLWaves == w
    const bool mine = lane < a.K && (lane % kLLWaves) == w;
    const int64_t e = mine ? ek : -1;
    const bool valid = e >= 0 && e < a.E;
    int rep = 0;  // earlier entries of this row with the same expert
    for (int k2 = 0; k2 < a.K; ++k2)
        rep += (k2 < lane && readlane64(ek, k2) == ek);
    Dests d;
    d.rbits = 0;
    d.vbits = uniform64(__ballot(valid));
    d.send_row = -1;
    d.recv_row = -1;
    if (mine) {
        if (valid) {
            const int slot = hist_before[e] + rep;
            if (slot < a.cap) {
                const int64_t region = a.R_buf == 1 ? e : e * a.R + a.src_rank;
                d.recv_row = (int)(region * a.cap + slot);
                a.ll_src[d.recv_row] = t;
            } else {
                flag_error(a.err, EPX_DEV_OVERFLOW);
            }
        }
        a.pos_ll[tk + lane] = d.recv_row;
    }
    if (d.vbits) {
        row.quantise(0, nitems);
        scatter<FP8>(row, d, xrow, a.h, nullptr, nullptr, a.ll_x, a.ll_scales);
    }
}

__global__ void fill_i32_kernel(int32_t *p, int64_t n, int32_t v)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

}  // namespace

// Items per lane per pass for hidden size h (see the comment on NV above).
static int pick_nv(int h, bool fp8)
{
    if (h <= 4096)
        return fp8 ? 4 : 8;
    if (h <= 7168)
        return fp8 ? 7 : 14;
    return fp8 ? 8 : 16;
}

template <bool FP8, int NV>
static void launch_dispatch_nv(const DispatchArgs &a, hipStream_t stream)
{
    hipLaunchKernelGGL((dispatch_kernel<FP8, NV>), dim3(a.T), dim3(kWave), 0, stream, a);
}

hipError_t launch_dispatch(const DispatchArgs &a, bool fp8, hipStream_t stream)
{
    if (a.T == 0)
        return hipSuccess;
    switch (pick_nv(a.h, fp8) + (fp8 ? 100 : 0)) {
    case 8: launch_dispatch_nv<false, 8>(a, stream); break;
    case 14: launch_dispatch_nv<false, 14>(a, stream); break;
    case 16: launch_dispatch_nv<false, 16>(a, stream); break;
    case 104: launch_dispatch_nv<true, 4>(a, stream); break;
    case 107: launch_dispatch_nv<true, 7>(a, stream); break;
    default: launch_dispatch_nv<true, 8>(a, stream); break;
    }
    return hipGetLastError();
}

template <bool FP8, int NV>
static void launch_ll_nv(const LLArgs &a, hipStream_t stream)
{
    const dim3 grid(a.T > 0 ? a.T : 1);
    const size_t lds = sizeof(int) * 2 * (size_t)a.E;
    hipLaunchKernelGGL((ll_dispatch_kernel<FP8, NV>), grid, dim3(kLLWaves * kWave), lds, stream,
                       a);
}

hipError_t launch_ll_dispatch(const LLArgs &a, bool fp8, hipStream_t stream)
{
    switch (pick_nv(a.h, fp8) + (fp8 ? 100 : 0)) {
    case 8: launch_ll_nv<false, 8>(a, stream); break;
    case 14: launch_ll_nv<false, 14>(a, stream); break;
    case 16: launch_ll_nv<false, 16>(a, stream); break;
    case 104: launch_ll_nv<true, 4>(a, stream); break;
    case 107: launch_ll_nv<true, 7>(a, stream); break;
    default: launch_ll_nv<true, 8>(a, stream); break;
    }
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
