// combine.hip -- reduce expert outputs back into source-token order.
//
// [P2] "DeepEP 学习笔记" (DeepEP study notes), "combine 过程": the handle
// saved by dispatch routes each expert output back to its source token,
// where the outputs are reduced. [P1] "事件驱动 EP 内核的调度策略与零拷贝通信",
// "低延迟模式：固定缓冲区与信号槽机制": combine stays in BF16.
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

constexpr int kBatch = 8;  // row loads in flight per lane

__global__ __launch_bounds__(kWave) void combine_kernel(CombineArgs a, int split)
{
    const int t = blockIdx.x / split, part = blockIdx.x - t * split;
    const int lane = threadIdx.x;
    const int nvec = a.h >> 3;
    const int v = part * kWave + lane;
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
    uint64_t todo = uniform64(__ballot(p >= 0));  // valid entries, k order
    const size_t row_bytes = (size_t)a.h * 2;
    const char *ycol = reinterpret_cast<const char *>(a.y) + (size_t)v * 16;
    const bool live = v < nvec;

    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        acc[i] = 0.0f;
    while (todo) {
        u32x4 y[kBatch];
        float wk[kBatch];
        bool use[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            use[j] = todo != 0;
            y[j] = u32x4{0u, 0u, 0u, 0u};
            wk[j] = 0.0f;
            if (use[j]) {
                const int k = __builtin_ctzll(todo);
                todo &= todo - 1;
                const int row = __builtin_amdgcn_readlane(p, k);
                wk[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k));
                if (live && row >= 0)
                    y[j] = load16_stream(ycol + (size_t)row * row_bytes);
            }
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if (use[j]) {
                const uint32_t q[4] = {y[j].x, y[j].y, y[j].z, y[j].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] = __builtin_fmaf(wk[j], bf16_lo(q[i]), acc[2 * i]);
                    acc[2 * i + 1] = __builtin_fmaf(wk[j], bf16_hi(q[i]), acc[2 * i + 1]);
                }
            }
        }
    }
    if (live) {
        u32x4 o;
        o.x = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
        o.y = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
        o.z = f32_to_bf16(acc[4]) | (f32_to_bf16(acc[5]) << 16);
        o.w = f32_to_bf16(acc[6]) | (f32_to_bf16(acc[7]) << 16);
        store16_stream(a.out + (size_t)t * a.h + (size_t)v * 8, o);
    }
}

}  // namespace

hipError_t launch_combine(const CombineArgs &a, hipStream_t stream)
{
    if (a.T == 0)
        return hipSuccess;
    const int split = ((a.h >> 3) + kWave - 1) / kWave;
    const int64_t blocks = (int64_t)a.T * split;
    if (blocks > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(kWave), 0, stream, a, split);
    return hipGetLastError();
}

}  // namespace epx
