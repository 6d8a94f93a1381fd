// dispatch_device.h -- device code of the dispatch kernels, shared by the
// dispatch, low-latency and fused layout + dispatch kernels: a row held in
// registers (bf16, or FP8 quantised once per token) and its scatter to every
// destination row with 16-byte stores.
#pragma once

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
    // vectors v0 + u * 64 + lane of a row of nvec vectors; zeros past its end
    __device__ __forceinline__ void load(const u32x4 *src, int v0, int nvec)
    {
        const __amdgpu_buffer_rsrc_t rs = row_rsrc(src, (uint32_t)nvec * 16u);
#pragma unroll
        for (int u = 0; u < NV; ++u)
            r[u] = load16_row(rs, (uint32_t)(v0 + u * kWave + lane_id()) * 16u);
    }
    __device__ __forceinline__ void quantise(int, int) {}
    template <StorePolicy POL = StorePolicy::WT>
    __device__ __forceinline__ void store(char *dst_row, int v0, int nvec) const
    {
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int v = v0 + u * kWave + lane_id();
            if (v < nvec)
                store16_row<POL>(dst_row, (uint32_t)v * 16, r[u]);
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

// The e4m3 codes of one 16-channel segment (lo: channels 0..7, hi: 8..15)
// and the scale of its 128-channel group, whose 8 segments sit on 8 adjacent
// lanes and are reduced with xor shuffles. Codes: e4m3 of x / s with
// s = max(amax, 1e-4) / 448 (IEEE), |x / s| <= 448 up to one rounding. A
// group holding an Inf or NaN takes a separate branch (uniform over the
// wave, almost never taken) that divides outright: amax over the non-NaN
// values, NaN quotients coded 0x7F.
__device__ __forceinline__ void quantise_segment(const u32x4 &lo, const u32x4 &hi, u32x4 &q,
                                                 float &s)
{
    const uint32_t p[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
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
    q = u32x4{wd[0], wd[1], wd[2], wd[3]};
}

// One pass of an FP8 row: segment sg = s0 + lane + 64*u covers channels
// [16 sg, 16 sg + 16), quantised by quantise_segment. Scale rows are
// scale_stride(h) floats apart, a whole number of 128-byte lines, and
// written in full (zeros past the last group): a scattered row that ends
// inside a line leaves that line to be merged in memory with a neighbour
// written at another time, which costs far more than the pad.
template <int NV>
struct RowFp8 {
    static constexpr int kPerPass = NV * kWave;
    u32x4 q[NV];
    u32x4 lo[NV], hi[NV];  // the bf16 pass as loaded (lo: channels 0..7, hi: 8..15)
    u32x4 sv;   // scales of groups s0/8 + 4*lane .. +3 of the pass, +0 past the last group
    int n_sv;   // lanes holding a slice of the (padded) scale row in this pass
    // Issue the pass's loads; quantise() consumes them, so work placed in
    // between overlaps their latency.
    // segments s0 + u * 64 + lane of a row of nseg segments; zeros past its
    // end (whole 8-lane groups, as nseg is a multiple of 8)
    __device__ __forceinline__ void load(const u32x4 *src, int s0, int nseg)
    {
        const __amdgpu_buffer_rsrc_t rs = row_rsrc(src, (uint32_t)nseg * 32u);
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const uint32_t off = (uint32_t)(s0 + u * kWave + lane_id()) * 32u;
            lo[u] = load16_row(rs, off);
            hi[u] = load16_row(rs, off + 16u);
        }
    }
    __device__ __forceinline__ void quantise(int s0, int nseg)
    {
        float sc[NV];
#pragma unroll
        for (int u = 0; u < NV; ++u)
            quantise_segment(lo[u], hi[u], q[u], sc[u]);
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
        // the pass's own groups (2 lanes per item); the last pass also
        // writes the zero padding up to the scale stride
        const bool last = s0 + kPerPass >= nseg;
        n_sv = min(16, last ? (scale_stride(nseg << 4) - g0) >> 2 : 2 * NV);
    }
    // Codes of the pass to one destination row, plus that row's slice of
    // the scale row (one 16-byte store by the first lanes).
    template <StorePolicy POL = StorePolicy::WT>
    __device__ __forceinline__ void store(uint8_t *q_row, float *s_row, int s0, int nseg) const
    {
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int sg = s0 + u * kWave + lane_id();
            if (sg < nseg)
                store16_row<POL>(q_row, (uint32_t)sg * 16, q[u]);
        }
        if (lane_id() < n_sv)
            store16_row<POL>(s_row, (uint32_t)((s0 >> 3) + 4 * lane_id()) * 4, sv);
    }
};

// Destination rows of one token, one per lane: lane r holds the rank-major
// row for rank r (bit r of rbits), lane k the expert-major row of entry k
// (bit k of vbits); -1 = skip (capacity overflow, already flagged).
struct Dests {
    uint64_t rbits, vbits;
    int send_row, recv_row;
    // a chunked sweep only: the destination's segment (lane r: rank r's
    // rows; lane k: entry k's expert's rows) as first row and row count
    int send_seg, send_n, recv_seg, recv_n;
};

// Smallest value over the wave.
__device__ __forceinline__ int wave_min(int v)
{
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1)
        v = min(v, __shfl_xor(v, d, kWave));
    return v;
}

// The paced sweep. Scattered row stores from many waves reach HBM as
// random writes (a fill in random order tops out at 5.0-5.3 TB/s on MI355X
// whatever the chunk size), while writes that the running waves make to
// adjacent addresses go at sequential-fill speed (6.5 TB/s). When every
// token's wave is on the chip at once, the scatter can be made sequential
// in time: each wave stores its rows in ascending order of their place in
// the output -- all send rows, then all receive rows -- and holds each row
// back until the wall clock has run (row's byte offset in that order) /
// sweep_bpt ticks since its schedule started (when the wave became ready,
// but no earlier than the launch's start offset). All waves then write near
// one front that moves through the output at the set rate. Only the time of
// each store changes, never what is stored; every wait is bounded by the
// clock.
struct Sweep {
    static constexpr bool kChunked = false;
    uint64_t t0;        // wall clock at the start of the wave's schedule
    uint32_t bpt;       // bytes per tick (0: no pacing)
    int64_t nsend;      // send rows ahead of the receive rows in the sweep
    int64_t row_bytes;  // bytes of one destination row (FP8: codes and scale row)
    // wait for the row whose place in the sweep is o
    __device__ __forceinline__ void wait(int64_t o) const
    {
        if (bpt == 0)
            return;
        const uint64_t due = t0 + (uint64_t)(o * row_bytes) / bpt;
        while (wall_clock64() < due)
            __builtin_amdgcn_s_sleep(1);
    }
};

// Launch stamps (see DispatchArgs::stamps): device-coherent vector store and
// load of one 64-bit word.
__device__ __forceinline__ void stamp_store(unsigned long long *p, uint64_t v)
{
    __hip_atomic_store(p, (unsigned long long)v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t stamp_load(const unsigned long long *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Block 0 of a paced launch stamps the wall clock at its start (workgroups
// are dispatched in index order, so no wave of the launch starts much
// before it); call from one lane.
__device__ __forceinline__ void stamp_launch(const DispatchArgs &a, uint64_t t_entry)
{
    if (a.sweep_bpt && a.stamps)
        stamp_store(a.stamps + a.stamp_slot, t_entry | 1ull);
}

// True when a wave that entered the kernel at t_entry is late: more than
// a.late_ticks after block 0 did, i.e. it only found a place after waves of
// the first round had ended. Read well after the wave's start (once its row
// has arrived), when block 0's stamp has long been stored; a word left by an
// earlier launch is older still, so it can only make a wave look late (its
// stores then go out unpaced: the same bytes, only not on the sweep).
__device__ __forceinline__ bool wave_is_late(const DispatchArgs &a, uint64_t t_entry)
{
    if (!a.stamps)
        return false;
    const uint64_t s = uniform64(stamp_load(a.stamps + a.stamp_slot));
    return (int64_t)(t_entry - s) > (int64_t)a.late_ticks;
}

// The sweep of one chunk of a dispatch launched in chunks of consecutive
// tokens (too many tokens for one round of waves). Rows sit in token order
// inside every segment (a rank's rows, an expert's rows), so a chunk's rows
// are one run per segment; a row's place among the chunk's rows is
// estimated from its place g in the whole sweep and its segment's first row
// a and size n as (g - a) + (a * cnt - n * tb) / T, for the chunk's tokens
// [tb, tb + cnt) -- exact when routing is spread evenly over the tokens,
// and only a timing estimate otherwise.
struct SweepChunk : Sweep {
    static constexpr bool kChunked = true;
    int64_t tb, cnt, T;
    __device__ __forceinline__ void wait(int64_t g, int64_t a, int64_t n) const
    {
        const int64_t o = g - a + (a * cnt - n * tb) / T;
        Sweep::wait(o < 0 ? 0 : o);
    }
};

// Write the token's row (the pass held in `row`, plus any further passes
// loaded here) to every destination, send rows (buffer a, rank order) then
// receive rows (buffer b, ascending row), each when the sweep reaches it.
// FP8 rows go out with the nontemporal policy, bf16 rows write-through.
template <bool FP8, typename Row, typename SW>
__device__ __forceinline__ void scatter(Row &row, const Dests &d, const uint16_t *xrow, int h,
                                        void *a_x, float *a_s, void *b_x, float *b_s,
                                        const SW &sw)
{
    const int nvec = h >> 3, nseg = h >> 4, ld_s = scale_stride(h);
    const int per_pass = Row::kPerPass;
    const int nitems = FP8 ? nseg : nvec;
    const size_t row_bytes = FP8 ? (size_t)h : (size_t)h * 2;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(xrow);
    const int lane = lane_id();
    for (int i0 = 0; i0 < nitems; i0 += per_pass) {
        if (i0 > 0) {
            row.load(src, i0, nitems);
            row.quantise(i0, nitems);
        }
        for (uint64_t m = d.rbits; m; m &= m - 1) {  // rank order is row order
            const int lr = __builtin_ctzll(m);
            const int r = readlane(d.send_row, lr);
            if (r < 0)
                continue;
            if constexpr (SW::kChunked)
                sw.wait(r, readlane(d.send_seg, lr), readlane(d.send_n, lr));
            else
                sw.wait(r);
            if constexpr (FP8)
                row.template store<StorePolicy::NT>(static_cast<uint8_t *>(a_x) + (size_t)r * row_bytes,
                                                    a_s + (size_t)r * ld_s, i0, nseg);
            else
                row.store(static_cast<char *>(a_x) + (size_t)r * row_bytes, i0, nvec);
        }
        // receive rows, smallest first when paced (skipped rows, -1, sort
        // last), else in top-k order
        const int key = ((d.vbits >> lane) & 1ull) ? (d.recv_row < 0 ? INT32_MAX - 1 : d.recv_row)
                                                   : INT32_MAX;
        for (uint64_t m = d.vbits; m;) {
            int k;
            if (sw.bpt) {
                const int kmin = wave_min(((m >> lane) & 1ull) ? key : INT32_MAX);
                k = __builtin_ctzll(m & uniform64(__ballot(key == kmin)));
            } else {
                k = __builtin_ctzll(m);
            }
            m &= ~(1ull << k);
            const int r = readlane(d.recv_row, k);
            if (r < 0)
                continue;
            if constexpr (SW::kChunked)
                sw.wait(sw.nsend + r, sw.nsend + readlane(d.recv_seg, k), readlane(d.recv_n, k));
            else
                sw.wait(sw.nsend + r);
            if constexpr (FP8)
                row.template store<StorePolicy::NT>(static_cast<uint8_t *>(b_x) + (size_t)r * row_bytes,
                                                    b_s + (size_t)r * ld_s, i0, nseg);
            else
                row.store(static_cast<char *>(b_x) + (size_t)r * row_bytes, i0, nvec);
        }
    }
}

// The destinations of token t in the high-throughput dispatch, from one
// wave: lane k < K holds the token's expert e (or -1) and recv_r, its
// expert-major row (exp_off[e] + slot), or -1; lane r < R holds send_r, its
// rank-major row (rank_off[r] + pos_in_rank[t, r]) if the token goes to rank
// r, else -1 (always -1 when there is no send buffer). Rows are checked
// against the capacities (a row past one is dropped). With meta, the wave
// also flags overflows and writes the handle and the per-row metadata; when
// several waves share a token, exactly one of them passes meta.
__device__ __forceinline__ Dests token_dests(const DispatchArgs &a, int t, int64_t e,
                                             int64_t send_r, int64_t recv_r, bool meta)
{
    const int lane = lane_id();
    const int64_t tk = (int64_t)t * a.K;
    const bool valid = lane < a.K && e >= 0 && e < a.E;
    Dests d;
    d.rbits = uniform64(__ballot(lane < a.R && send_r >= 0));
    d.vbits = uniform64(__ballot(valid));
    d.send_row = -1;
    d.recv_row = -1;
    if (lane < a.R && send_r >= 0) {
        if (send_r < a.send_cap)
            d.send_row = (int)send_r;
        else if (meta)
            flag_error(a.err, EPX_DEV_OVERFLOW);
    }
    if (lane < a.K) {
        if (valid) {
            if (recv_r >= 0 && recv_r < a.recv_cap)
                d.recv_row = (int)recv_r;
            else if (meta)
                flag_error(a.err, EPX_DEV_OVERFLOW);
        }
        if (meta) {
            a.pos_exp[tk + lane] = d.recv_row;
            if (d.recv_row >= 0)
                a.recv_src[d.recv_row] = t;
        }
    }
    // per send row: source token and the top-k list seen from that rank
    if (meta && d.send_row >= 0) {
        const int64_t row_i = d.send_row;
        a.send_src[row_i] = t;
        for (int k = 0; k < a.K; ++k) {
            const int64_t ek = a.topk_idx[tk + k];
            const bool on_r = ek >= 0 && ek < a.E && div_by_magic((int)ek, a.L_mul) == lane;
            a.send_topk_idx[row_i * a.K + k] = on_r ? ek - (int64_t)lane * a.L : -1;
            a.send_topk_w[row_i * a.K + k] = on_r ? a.topk_w[tk + k] : 0.0f;
        }
    }
    return d;
}

// The per-token part of the high-throughput dispatch, for a wave holding
// token t's row (first pass loaded, not yet quantised) and its lanes as in
// token_dests: checks, handle and metadata, then the row to every
// destination. nsend: the number of send rows (the receive rows' place in
// the sweep; 0 without a send buffer). The wave's schedule starts when it
// gets here, but no earlier than a.start_ticks after its entry (t_entry); a
// late wave (entered more than a.late_ticks after block 0) stores unpaced.
// CHUNKED: the launch is one chunk [a.t_begin, a.t_begin + a.t_count) of the
// tokens, and the lanes' segments are read from the layout offsets.
template <bool FP8, bool CHUNKED = false, typename Row>
__device__ __forceinline__ void dispatch_token(const DispatchArgs &a, int t, Row &row,
                                               const uint16_t *xrow, int64_t e, int64_t send_r,
                                               int64_t recv_r, int64_t nsend, uint64_t t_entry)
{
    typename std::conditional<CHUNKED, SweepChunk, Sweep>::type sw;
    const uint64_t ready = wall_clock64(), start = t_entry + a.start_ticks;
    sw.t0 = ready > start ? ready : start;
    sw.bpt = a.sweep_bpt;
    sw.nsend = nsend;
    sw.row_bytes = FP8 ? (int64_t)a.h + 4 * (int64_t)scale_stride(a.h) : 2 * (int64_t)a.h;
    Dests d = token_dests(a, t, e, send_r, recv_r, true);
    if (sw.bpt && wave_is_late(a, t_entry))
        sw.bpt = 0;
    if constexpr (CHUNKED) {
        sw.tb = a.t_begin;
        sw.cnt = a.t_count;
        sw.T = a.T;
        const int lane = lane_id();
        d.send_seg = d.send_n = d.recv_seg = d.recv_n = 0;
        if (send_r >= 0 && lane < a.R) {
            d.send_seg = a.rank_off[lane];
            d.send_n = a.rank_off[lane + 1] - d.send_seg;
        }
        if (recv_r >= 0 && e >= 0 && e < a.E) {
            d.recv_seg = a.exp_off[(int)e];
            d.recv_n = a.exp_off[(int)e + 1] - d.recv_seg;
        }
    }
    row.quantise(0, FP8 ? a.h >> 4 : a.h >> 3);
    scatter<FP8>(row, d, xrow, a.h, a.send_x, a.send_scales, a.recv_x, a.recv_scales, sw);
}

// One slice of a token's row (items s0 .. s0 + Row::kPerPass - 1, loaded in
// `row`, whole 128-channel groups for FP8) to every destination in d.
template <bool FP8, typename Row>
__device__ __forceinline__ void scatter_slice(Row &row, const Dests &d, int s0,
                                              const DispatchArgs &a)
{
    const int nitems = FP8 ? a.h >> 4 : a.h >> 3, ld_s = scale_stride(a.h);
    const size_t row_bytes = FP8 ? (size_t)a.h : (size_t)a.h * 2;
    row.quantise(s0, nitems);
    for (uint64_t m = d.rbits; m; m &= m - 1) {
        const int r = readlane(d.send_row, __builtin_ctzll(m));
        if (r < 0)
            continue;
        if constexpr (FP8)
            row.template store<StorePolicy::NT>(static_cast<uint8_t *>(a.send_x) + (size_t)r * row_bytes,
                                                a.send_scales + (size_t)r * ld_s, s0, nitems);
        else
            row.store(static_cast<char *>(a.send_x) + (size_t)r * row_bytes, s0, nitems);
    }
    for (uint64_t m = d.vbits; m; m &= m - 1) {
        const int r = readlane(d.recv_row, __builtin_ctzll(m));
        if (r < 0)
            continue;
        if constexpr (FP8)
            row.template store<StorePolicy::NT>(static_cast<uint8_t *>(a.recv_x) + (size_t)r * row_bytes,
                                                a.recv_scales + (size_t)r * ld_s, s0, nitems);
        else
            row.store(static_cast<char *>(a.recv_x) + (size_t)r * row_bytes, s0, nitems);
    }
}

}  // namespace

// Items per lane per pass for hidden size h (see the comment on NV above).
inline int pick_nv(int h, bool fp8)
{
    if (h <= 4096)
        return fp8 ? 4 : 8;
    if (h <= 7168)
        return fp8 ? 7 : 14;
    return fp8 ? 8 : 16;
}

}  // namespace epx
