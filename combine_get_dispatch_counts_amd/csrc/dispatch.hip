// dispatch.hip -- high-throughput dispatch (pack + permute, optional FP8) and
// the low-latency fixed-slot dispatch.
//
// Both kernels give one token to one block: the block reads the token's row
// of x from HBM once (16-byte loads), optionally quantises it to FP8 in
// registers, and writes it to every destination row with 16-byte streaming
// stores, so each destination costs exactly one row write.
//
// [P2] "DeepEP 学习笔记" (DeepEP study notes), "dispatch 过程": a token goes,
// in token order, to every rank is_token_in_rank marks, together with its
// source index, top-k indices and weights. [P2] "DeepEP v2": one full
// activation per destination rank. [P1] "事件驱动 EP 内核的调度策略与零拷贝
// 通信", "高吞吐量模式：协调阶段与紧凑缓冲区": exact-size receive buffer, then
// a local permute into contiguous per-expert blocks. On one GPU the pack and
// the permute read the same register copy of the row, so the permute costs
// no second read. [P1] "低延迟模式：固定缓冲区与信号槽机制": fixed per-
// (source, expert) regions, FP8 payload. [P3] "DeepSeek DeepEP探索：低延迟分发",
// 3.2: the local path is an unrolled 16-byte vector copy with non-caching
// loads and stores -- kept here as streaming 16-byte moves.
#include "epx_device.h"
#include "epx_internal.h"

namespace epx {
namespace {

constexpr int kBlock = 128;                 // 2 waves per token
constexpr int kMaxDst = 2 * EPX_MAX_TOPK;  // <= K rank rows + K expert rows
constexpr int kVecBf16 = 8;                // 16-byte vectors per thread per pass
constexpr int kSegFp8 = 4;                 // 16-channel segments per thread per pass

// Copy one bf16 row (h channels) to n destination rows. Destination d < n_a
// lives in buffer a, the rest in buffer b; rows[d] < 0 means "skip".
__device__ __forceinline__ void scatter_bf16(const uint16_t *__restrict__ xrow, int h,
                             const int64_t *rows, int n_a, int n, char *base_a, char *base_b)
{
    const int nvec = h >> 3;
    const size_t row_bytes = (size_t)h * 2;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(xrow);
    for (int v0 = 0; v0 < nvec; v0 += kBlock * kVecBf16) {
        u32x4 r[kVecBf16];
#pragma unroll
        for (int u = 0; u < kVecBf16; ++u) {
            const int v = v0 + u * kBlock + (int)threadIdx.x;
            r[u] = (v < nvec) ? load16_stream(src + v) : u32x4{0u, 0u, 0u, 0u};
        }
        for (int d = 0; d < n; ++d) {
            const int64_t row = rows[d];
            if (row < 0)
                continue;
            char *dst = (d < n_a ? base_a : base_b) + (size_t)row * row_bytes;
#pragma unroll
            for (int u = 0; u < kVecBf16; ++u) {
                const int v = v0 + u * kBlock + (int)threadIdx.x;
                if (v < nvec)
                    store16_stream(dst + (size_t)v * 16, r[u]);
            }
        }
    }
}

// Quantise one bf16 row to e4m3 with one fp32 scale per 128 channels and copy
// codes + scales to n destination rows (same destination rules as above).
// A lane owns 16 consecutive channels, so a 128-channel group is 8 adjacent
// lanes; amax is reduced over them with xor shuffles. h % 128 == 0.
__device__ __forceinline__ void scatter_fp8(const uint16_t *__restrict__ xrow, int h, const int64_t *rows,
                            int n_a, int n, uint8_t *q_a, float *s_a, uint8_t *q_b, float *s_b)
{
    const int nseg = h >> 4;
    const int ngrp = h >> 7;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(xrow);
    for (int s0 = 0; s0 < nseg; s0 += kBlock * kSegFp8) {
        u32x4 q[kSegFp8];
        float sc[kSegFp8];
#pragma unroll
        for (int u = 0; u < kSegFp8; ++u) {
            const int sg = s0 + u * kBlock + (int)threadIdx.x;
            const bool active = sg < nseg;  // uniform over each 8-lane group
            u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
            if (active) {
                lo = load16_stream(src + 2 * sg);
                hi = load16_stream(src + 2 * sg + 1);
            }
            float f[16];
            const uint32_t p[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                f[2 * i] = bf16_lo(p[i]);
                f[2 * i + 1] = bf16_hi(p[i]);
            }
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                amax = fmaxf(amax, fabsf(f[i]));
            amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
            amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
            amax = fmaxf(amax, __shfl_xor(amax, 4, kWave));
            const float s = fmaxf(amax, 1e-4f) / 448.0f;
            uint32_t wd[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                wd[j] = f32_to_e4m3(f[4 * j] / s) | (f32_to_e4m3(f[4 * j + 1] / s) << 8) |
                        (f32_to_e4m3(f[4 * j + 2] / s) << 16) |
                        (f32_to_e4m3(f[4 * j + 3] / s) << 24);
            q[u] = u32x4{wd[0], wd[1], wd[2], wd[3]};
            sc[u] = s;
        }
        for (int d = 0; d < n; ++d) {
            const int64_t row = rows[d];
            if (row < 0)
                continue;
            uint8_t *qd = (d < n_a ? q_a : q_b) + (size_t)row * h;
            float *sd = (d < n_a ? s_a : s_b) + (size_t)row * ngrp;
#pragma unroll
            for (int u = 0; u < kSegFp8; ++u) {
                const int sg = s0 + u * kBlock + (int)threadIdx.x;
                if (sg < nseg) {
                    store16_stream(qd + (size_t)sg * 16, q[u]);
                    if ((sg & 7) == 0)
                        sd[sg >> 3] = sc[u];
                }
            }
        }
    }
}

template <bool FP8>
__global__ __launch_bounds__(kBlock) void dispatch_kernel(DispatchArgs a)
{
    __shared__ int64_t s_row[kMaxDst];
    __shared__ int s_rank[EPX_MAX_TOPK];
    __shared__ int s_nsend, s_n;
    const int t = blockIdx.x, tid = threadIdx.x;
    const int64_t tk = (int64_t)t * a.K;

    if (tid < kWave) {
        const int lane = tid;
        const int64_t e = lane < a.K ? a.topk_idx[tk + lane] : -1;
        const bool valid = e >= 0 && e < a.E;
        const int ei = valid ? (int)e : 0;
        const uint64_t rbits = wave_or(valid ? (1ull << (ei / a.L)) : 0ull);
        const int nsend = __popcll(rbits);
        // rank-major rows: lane r owns rank r; ascending ranks
        if (lane < a.R && ((rbits >> lane) & 1ull)) {
            const int j = __popcll(rbits & lanes_below(lane));
            int64_t row = (int64_t)a.rank_off[lane] + a.pos_in_rank[(int64_t)t * a.R + lane];
            if (row < 0 || row >= a.send_cap) {
                flag_error(a.err, EPX_DEV_OVERFLOW);
                row = -1;
            }
            s_row[j] = row;
            s_rank[j] = lane;
        }
        // expert-major rows: valid entries in k order
        const uint64_t vbits = __ballot(valid);
        if (lane < a.K) {
            int32_t pe = -1;
            if (valid) {
                const int j = nsend + __popcll(vbits & lanes_below(lane));
                int64_t row = (int64_t)a.exp_off[ei] + a.slot_in_expert[tk + lane];
                if (row < 0 || row >= a.recv_cap) {
                    flag_error(a.err, EPX_DEV_OVERFLOW);
                    row = -1;
                } else {
                    pe = (int32_t)row;
                }
                s_row[j] = row;
            }
            a.pos_exp[tk + lane] = pe;
        }
        if (lane == 0) {
            s_nsend = nsend;
            s_n = nsend + __popcll(vbits);
        }
    }
    __syncthreads();
    const int nsend = s_nsend, n = s_n;

    // per-row metadata: source token, and the top-k list seen from the row's rank
    for (int i = tid; i < nsend * a.K; i += kBlock) {
        const int j = i / a.K, k = i - j * a.K;
        const int64_t row = s_row[j];
        if (row < 0)
            continue;
        const int r = s_rank[j];
        const int64_t e = a.topk_idx[tk + k];
        const bool on_r = e >= 0 && e < a.E && (int)e / a.L == r;
        a.send_topk_idx[row * a.K + k] = on_r ? e - (int64_t)r * a.L : -1;
        a.send_topk_w[row * a.K + k] = on_r ? a.topk_w[tk + k] : 0.0f;
    }
    if (tid < n) {
        const int64_t row = s_row[tid];
        if (row >= 0) {
            if (tid < nsend)
                a.send_src[row] = t;
            else
                a.recv_src[row] = t;
        }
    }

    const uint16_t *xrow = a.x + (size_t)t * a.h;
    if (FP8)
        scatter_fp8(xrow, a.h, s_row, nsend, n, static_cast<uint8_t *>(a.send_x), a.send_scales,
                    static_cast<uint8_t *>(a.recv_x), a.recv_scales);
    else
        scatter_bf16(xrow, a.h, s_row, nsend, n, static_cast<char *>(a.send_x),
                     static_cast<char *>(a.recv_x));
}

// Low-latency dispatch, one launch. Block t handles token t; every block
// first histograms all T*K entries in LDS (decode batches are small): the
// full histogram gives the count slots, the part before token t gives t's
// slots. LDS atomics only add, so the result does not depend on their order.
template <bool FP8>
__global__ __launch_bounds__(kBlock) void ll_dispatch_kernel(LLArgs a)
{
    extern __shared__ int hist[];  // [E] all entries, [E] entries before token t
    __shared__ int64_t s_row[EPX_MAX_TOPK];
    __shared__ int s_n;
    const int t = blockIdx.x, tid = threadIdx.x;
    int *hist_all = hist, *hist_before = hist + a.E;
    for (int i = tid; i < 2 * a.E; i += kBlock)
        hist[i] = 0;
    __syncthreads();
    const int64_t n_ent = (int64_t)a.T * a.K;
    const int64_t tk = (int64_t)t * a.K;
    for (int64_t i = tid; i < n_ent; i += kBlock) {
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
    for (int e = blockIdx.x * kBlock + tid; e < a.E; e += gridDim.x * kBlock) {
        const int64_t region = a.R_buf == 1 ? e : (int64_t)e * a.R + a.src_rank;
        a.ll_count[region] = hist_all[e];
    }
    if (t >= a.T)
        return;

    if (tid < kWave) {
        const int lane = tid;
        const int64_t e = lane < a.K ? a.topk_idx[tk + lane] : -1;
        const bool valid = e >= 0 && e < a.E;
        int rep = 0;  // earlier entries of this row with the same expert
        if (valid)
            for (int k2 = 0; k2 < lane; ++k2)
                rep += (a.topk_idx[tk + k2] == e);
        const uint64_t vbits = __ballot(valid);
        if (lane < a.K) {
            int32_t p = -1;
            if (valid) {
                const int j = __popcll(vbits & lanes_below(lane));
                const int slot = hist_before[e] + rep;
                int64_t row = -1;
                if (slot < a.cap) {
                    const int64_t region = a.R_buf == 1 ? e : e * a.R + a.src_rank;
                    row = region * a.cap + slot;
                    a.ll_src[row] = t;
                    p = (int32_t)row;
                } else {
                    flag_error(a.err, EPX_DEV_OVERFLOW);
                }
                s_row[j] = row;
            }
            a.pos_ll[tk + lane] = p;
        }
        if (lane == 0)
            s_n = __popcll(vbits);
    }
    __syncthreads();

    const uint16_t *xrow = a.x + (size_t)t * a.h;
    if (FP8)
        scatter_fp8(xrow, a.h, s_row, 0, s_n, nullptr, nullptr, static_cast<uint8_t *>(a.ll_x),
                    a.ll_scales);
    else
        scatter_bf16(xrow, a.h, s_row, 0, s_n, nullptr, static_cast<char *>(a.ll_x));
}

__global__ void fill_i32_kernel(int32_t *p, int64_t n, int32_t v)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

}  // namespace

hipError_t launch_dispatch(const DispatchArgs &a, bool fp8, hipStream_t stream)
{
    if (a.T == 0)
        return hipSuccess;
    if (fp8)
        hipLaunchKernelGGL(dispatch_kernel<true>, dim3(a.T), dim3(kBlock), 0, stream, a);
    else
        hipLaunchKernelGGL(dispatch_kernel<false>, dim3(a.T), dim3(kBlock), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_ll_dispatch(const LLArgs &a, bool fp8, hipStream_t stream)
{
    const dim3 grid(a.T > 0 ? a.T : 1);
    const size_t lds = sizeof(int) * 2 * (size_t)a.E;
    if (fp8)
        hipLaunchKernelGGL(ll_dispatch_kernel<true>, grid, dim3(kBlock), lds, stream, a);
    else
        hipLaunchKernelGGL(ll_dispatch_kernel<false>, grid, dim3(kBlock), lds, stream, a);
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
