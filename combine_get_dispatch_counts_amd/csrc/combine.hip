// combine.hip -- reduce expert outputs back into source-token order.
//
// [P2] "DeepEP 学习笔记" (DeepEP study notes), "combine 过程": the handle
// saved by dispatch routes each expert output back to its source token,
// where the outputs are reduced. [P1] "事件驱动 EP 内核的调度策略与零拷贝通信",
// "低延迟模式：固定缓冲区与信号槽机制": combine stays in BF16.
//
// The two-stage form ([P2] "DeepEP v2": the destination rank reduces its own
// experts' outputs for a token into one rank-level partial result, the
// source reduces over ranks) uses the same reduction twice: stage 1 per
// rank-major row over that rank's entries, stage 2 per token over its
// partial rows in rank order.
//
// Many small blocks: block (t, part) is one wave that owns 64 consecutive
// 16-byte column vectors of token t's output row (h = 7168 gives 14 blocks
// per token). Lane k < K loads the handle row and weight of entry k; the
// valid entries are then walked in k order with wave-uniform readlanes,
// 8 row loads in flight per lane at a time, each folded into 8 fp32
// accumulators with fmaf: acc = fmaf(w_k, y_k, acc) from +0.0f, rounded to
// bf16 nearest-even at the end. No LDS, no barrier; HBM-bound (K row reads
// and one row write per token).
#include "epx_device.h"
#include "epx_internal.h"

namespace epx {
namespace {

// Fold the rows named by the lanes into fp32 columns: lane j holds row p
// (-1 = skip) and weight w of entry j; entries are taken in lane order,
// acc = fmaf(w, y[p], acc) from +0.0f. The wave covers P slices of 64
// 16-byte column vectors, slice q being vectors (part*P + q)*64 + lane, and
// keeps B entries x P vectors of loads in flight per lane; the bf16 result
// goes to out_row.
template <int P, int B>
__device__ __forceinline__ void reduce_rows(const uint16_t *y, int h, int p, float w, int part,
                                            uint16_t *out_row)
{
    const int lane = threadIdx.x;
    const int nvec = h >> 3;
    uint64_t todo = uniform64(__ballot(p >= 0));  // valid entries, lane order
    const size_t row_bytes = (size_t)h * 2;
    int v[P];
    bool live[P];
#pragma unroll
    for (int q = 0; q < P; ++q) {
        v[q] = (part * P + q) * kWave + lane;
        live[q] = v[q] < nvec;
    }
    const char *ybase = reinterpret_cast<const char *>(y);

    float acc[P][8];
#pragma unroll
    for (int q = 0; q < P; ++q)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc[q][i] = 0.0f;
    while (todo) {
        u32x4 yv[B][P];
        float wk[B];
        bool use[B];
#pragma unroll
        for (int j = 0; j < B; ++j) {
            use[j] = todo != 0;
            wk[j] = 0.0f;
            int row = -1;
            if (use[j]) {
                const int k = __builtin_ctzll(todo);
                todo &= todo - 1;
                row = __builtin_amdgcn_readlane(p, k);
                wk[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k));
            }
#pragma unroll
            for (int q = 0; q < P; ++q)
                yv[j][q] = (use[j] && live[q] && row >= 0)
                               ? load16_stream(ybase + (size_t)row * row_bytes + (size_t)v[q] * 16)
                               : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < B; ++j) {
            if (use[j]) {
#pragma unroll
                for (int q = 0; q < P; ++q) {
                    const uint32_t e[4] = {yv[j][q].x, yv[j][q].y, yv[j][q].z, yv[j][q].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[q][2 * i] = __builtin_fmaf(wk[j], bf16_lo(e[i]), acc[q][2 * i]);
                        acc[q][2 * i + 1] =
                            __builtin_fmaf(wk[j], bf16_hi(e[i]), acc[q][2 * i + 1]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int q = 0; q < P; ++q) {
        if (live[q]) {
            u32x4 o;
            o.x = f32_to_bf16(acc[q][0]) | (f32_to_bf16(acc[q][1]) << 16);
            o.y = f32_to_bf16(acc[q][2]) | (f32_to_bf16(acc[q][3]) << 16);
            o.z = f32_to_bf16(acc[q][4]) | (f32_to_bf16(acc[q][5]) << 16);
            o.w = f32_to_bf16(acc[q][6]) | (f32_to_bf16(acc[q][7]) << 16);
            store16_stream(out_row + (size_t)v[q] * 8, o);
        }
    }
}

// Slices per wave and entries per load batch of each kernel.
constexpr int kCombP = 1, kCombB = 8;        // one-stage: K entries per token
// Stage 1 (about K/R entries per row): two slices per wave, one entry at a
// time, 35 registers and the full 32 waves per CU. Measured at the prefill
// shape: 144.9 us against 151.5 us for four slices of two entries (83
// registers, 20 waves per CU); one slice per wave 181 us (each wave's chain
// of metadata loads dominates); fewer waves per CU always slower.
constexpr int kPartP = 2, kPartB = 1;
constexpr int kFinalP = 1, kFinalB = 8;      // stage 2: up to R partial rows per token

__global__ __launch_bounds__(kWave) void combine_kernel(CombineArgs a, int split)
{
    const int t = blockIdx.x / split, part = blockIdx.x - t * split;
    const int lane = threadIdx.x;
    const int64_t tk = (int64_t)t * a.K;
    int p = -1;
    float w = 0.0f;
    if (lane < a.K) {
        p = a.pos[tk + lane];
        w = a.topk_w[tk + lane];
        if (p >= a.n_rows) {
            if (part == 0)
                flag_error(a.err, EPX_DEV_BAD_HANDLE);
            p = -1;
        }
    }
    reduce_rows<kCombP, kCombB>(a.y, a.h, p, w, part, a.out + (size_t)t * a.h);
}

// Stage 1 of the two-stage combine: rank-major row i (token send_src[i])
// reduces the entries of its own rank (send_topk_idx >= 0), whose expert
// rows the token's handle pos_exp names.
__global__ __launch_bounds__(kWave) void combine_partial_kernel(PartialArgs a, int split)
{
    const int64_t i = blockIdx.x / split;
    const int part = (int)(blockIdx.x - i * split);
    if (a.num_rows && i >= *a.num_rows)
        return;
    const int lane = threadIdx.x;
    const int t = a.send_src[i];
    const bool t_ok = t >= 0 && t < a.T;
    if (!t_ok && lane == 0 && part == 0)
        flag_error(a.err, EPX_DEV_BAD_HANDLE);
    int p = -1;
    float w = 0.0f;
    if (t_ok && lane < a.K) {
        const int64_t idx = a.send_topk_idx[i * a.K + lane];
        w = a.send_topk_w[i * a.K + lane];
        if (idx >= 0) {
            p = a.pos_exp[(int64_t)t * a.K + lane];
            if (p >= a.n_rows) {
                if (part == 0)
                    flag_error(a.err, EPX_DEV_BAD_HANDLE);
                p = -1;
            }
        }
    }
    reduce_rows<kPartP, kPartB>(a.y, a.h, p, w, part, a.partial + (size_t)i * a.h);
}

// Stage 2: token t adds its partial rows, one per rank it went to, in rank
// order (weight 1: fmaf(1, y, acc) rounds exactly like acc + y).
__global__ __launch_bounds__(kWave) void combine_final_kernel(FinalArgs a, int split)
{
    const int t = blockIdx.x / split, part = blockIdx.x - t * split;
    const int lane = threadIdx.x;
    int p = -1;
    if (lane < a.R) {
        const int32_t pr = a.pos_in_rank[(int64_t)t * a.R + lane];
        if (pr >= 0) {
            const int64_t row = (int64_t)a.rank_off[lane] + pr;
            if (row < a.n_rows) {
                p = (int)row;
            } else if (part == 0) {
                flag_error(a.err, EPX_DEV_BAD_HANDLE);
            }
        }
    }
    reduce_rows<kFinalP, kFinalB>(a.partial, a.h, p, 1.0f, part, a.out + (size_t)t * a.h);
}

}  // namespace

// LDS reserved by each one-wave block of the one-stage and final combine
// (the kernels use none): 9 KB lets at most 17 blocks share a compute unit's
// 160 KB, against the 32 their registers allow. Fewer row reads in flight
// gather faster; measured on MI355X at h = 7168: the combine 87.8 against
// 86.7 us (T = 4096) and 356-363 against 349-358 us (T = 16384), the final
// stage 80.0 against 78.6 us; level at h = 4096; 12 blocks or fewer slower.
// The first stage, one entry per load batch, wants every wave it can hold
// (20 blocks per CU: 146 -> 169 us).
constexpr size_t kCombLdsBytes = 9216;

// Waves per output row when each covers P slices of 64 column vectors.
static int combine_split(int h, int P) { return ((h >> 3) + P * kWave - 1) / (P * kWave); }

hipError_t launch_combine(const CombineArgs &a, hipStream_t stream)
{
    if (a.T == 0)
        return hipSuccess;
    const int split = combine_split(a.h, kCombP);
    const int64_t blocks = (int64_t)a.T * split;
    if (blocks > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(kWave), kCombLdsBytes, stream, a, split);
    return hipGetLastError();
}

hipError_t launch_combine_partial(const PartialArgs &a, hipStream_t stream)
{
    if (a.cap_rows == 0)
        return hipSuccess;
    const int split = combine_split(a.h, kPartP);
    const int64_t blocks = a.cap_rows * split;
    if (blocks > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(combine_partial_kernel, dim3((unsigned)blocks), dim3(kWave), 0, stream, a,
                       split);
    return hipGetLastError();
}

hipError_t launch_combine_final(const FinalArgs &a, hipStream_t stream)
{
    if (a.T == 0)
        return hipSuccess;
    const int split = combine_split(a.h, kFinalP);
    const int64_t blocks = (int64_t)a.T * split;
    if (blocks > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(combine_final_kernel, dim3((unsigned)blocks), dim3(kWave), kCombLdsBytes, stream, a,
                       split);
    return hipGetLastError();
}

}  // namespace epx
