// combine.hip -- reduce expert outputs back into source-token order.
//
// [P2] "DeepEP 学习笔记" (DeepEP study notes), "combine 过程": the handle
// saved by dispatch routes each expert output back to its source token,
// where the outputs are reduced. [P1] "事件驱动 EP 内核的调度策略与零拷贝通信",
// "低延迟模式：固定缓冲区与信号槽机制": combine stays in BF16.
//
// One block per token. Wave 0 compacts the token's valid handle rows (k
// order kept) into LDS; then each thread owns 16-byte column vectors and,
// for each, issues up to 8 row loads at once before folding them into 8
// fp32 accumulators with fmaf in k order: acc = fmaf(w_k, y_k, acc) from
// +0.0f, rounded to bf16 nearest-even at the end. HBM-bound: K row reads and
// one row write per token.
#include "epx_device.h"
#include "epx_internal.h"

namespace epx {
namespace {

constexpr int kBlock = 128;
constexpr int kBatch = 8;  // row loads in flight per vector

__global__ __launch_bounds__(kBlock) void combine_kernel(CombineArgs a)
{
    __shared__ int64_t s_row[EPX_MAX_TOPK];
    __shared__ float s_w[EPX_MAX_TOPK];
    __shared__ int s_n;
    const int t = blockIdx.x, tid = threadIdx.x;
    const int64_t tk = (int64_t)t * a.K;
    if (tid < kWave) {
        const int lane = tid;
        int64_t p = lane < a.K ? a.pos[tk + lane] : -1;
        if (p >= a.n_rows) {
            flag_error(a.err, EPX_DEV_BAD_HANDLE);
            p = -1;
        }
        const bool valid = p >= 0;
        const uint64_t vbits = __ballot(valid);
        if (valid) {
            const int j = __popcll(vbits & lanes_below(lane));
            s_row[j] = p;
            s_w[j] = a.topk_w[tk + lane];
        }
        if (lane == 0)
            s_n = __popcll(vbits);
    }
    __syncthreads();
    const int n = s_n;
    const int nvec = a.h >> 3;
    const size_t row_bytes = (size_t)a.h * 2;
    const char *ybase = reinterpret_cast<const char *>(a.y);
    uint16_t *orow = a.out + (size_t)t * a.h;

    for (int v = tid; v < nvec; v += kBlock) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc[i] = 0.0f;
        for (int k0 = 0; k0 < n; k0 += kBatch) {
            u32x4 y[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                y[j] = (k0 + j < n)
                           ? load16_stream(ybase + (size_t)s_row[k0 + j] * row_bytes + (size_t)v * 16)
                           : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                if (k0 + j < n) {
                    const float w = s_w[k0 + j];
                    const uint32_t p[4] = {y[j].x, y[j].y, y[j].z, y[j].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[2 * i] = __builtin_fmaf(w, bf16_lo(p[i]), acc[2 * i]);
                        acc[2 * i + 1] = __builtin_fmaf(w, bf16_hi(p[i]), acc[2 * i + 1]);
                    }
                }
            }
        }
        u32x4 o;
        o.x = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
        o.y = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
        o.z = f32_to_bf16(acc[4]) | (f32_to_bf16(acc[5]) << 16);
        o.w = f32_to_bf16(acc[6]) | (f32_to_bf16(acc[7]) << 16);
        store16_stream(orow + (size_t)v * 8, o);
    }
}

}  // namespace

hipError_t launch_combine(const CombineArgs &a, hipStream_t stream)
{
    if (a.T == 0)
        return hipSuccess;
    hipLaunchKernelGGL(combine_kernel, dim3(a.T), dim3(kBlock), 0, stream, a);
    return hipGetLastError();
}

}  // namespace epx
