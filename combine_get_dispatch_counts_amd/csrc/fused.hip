// fused.hip -- get_dispatch_layout and the high-throughput dispatch in one
// launch.
//
// [P2] "DeepEP v2": the v2 dispatch kernel computes the layout itself (its
// notify warps take the place of get_dispatch_layout) while its dispatch
// warps move the data, in one launch. Here the first blocks of the grid are
// the layout's blocks (layout_device.h: one per 256-token tile, then the
// totals block) and the rest are dispatch blocks of kLayoutThreads threads,
// one wave per token. A dispatch wave issues its row's loads at once, then
// waits for two things the layout blocks publish as self-contained tagged
// 64-bit words (tag << 32 | value, the same scheme as the tiles' look-back,
// so no ordering between different addresses is relied on): the totals
// (from which each dispatch block scans the offsets into LDS) and its
// token's final in-rank positions and in-expert slots. It then goes on
// exactly as the two-launch dispatch does (dispatch_device.h). The layout's
// own outputs are written as by epx_get_dispatch_layout, for the caller.
//
// The waits are bounded (flagging EPX_DEV_WORKSPACE), and the layout blocks
// come first in the grid, so the blocks they wait for are dispatched first.
// The row loads overlap the layout's critical path; the second launch and
// the re-read of pos_in_rank / slot_in_expert from memory disappear.
#include "dispatch_device.h"
#include "layout_device.h"

namespace epx {
namespace {

constexpr int kFusedTokens = kLayoutThreads / kWave;  // tokens per dispatch block

// Wait until the word each needing lane reads carries the call's tag
// (bounded; false on time-out). Wave-uniform loop.
__device__ bool wait_tagged(const uint64_t *p, bool need, uint32_t tag, uint64_t &w)
{
    int polls = 0;
    w = need ? pub_load(p) : 0;
    while (__any(need && (uint32_t)(w >> 32) != tag)) {
        if (++polls > kSpinLimit)
            return false;
        __builtin_amdgcn_s_sleep(2);
        if (need && (uint32_t)(w >> 32) != tag)
            w = pub_load(p);
    }
    return true;
}

template <int KMAX, bool FP8, int NV>
__global__ __launch_bounds__(kLayoutThreads) void fused_kernel(FusedArgs f)
{
    extern __shared__ __attribute__((aligned(16))) char lds[];
    if ((int)blockIdx.x <= f.lay.ntiles) {  // the layout's blocks (or T = 0)
        layout_block<KMAX>(f.lay, lds, f.tok, f.tot);
        return;
    }
    const DispatchArgs &a = f.disp;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid >> 6;
    const int t = (blockIdx.x - f.lay.ntiles - 1) * kFusedTokens + w;
    const bool have = t < a.T;
    const int ER = a.E + a.R;
    int *tot = reinterpret_cast<int *>(lds + count_lds_bytes(a.E, a.R));
    int *off = tot + 2 * ER;  // [E+1] expert offsets, then [R+1] rank offsets
    __shared__ int s_ok;
    __shared__ uint32_t s_tag;

    // the row and the token's experts go out first
    const int64_t tk = (int64_t)t * a.K;
    const uint16_t *xrow = a.x + (size_t)(have ? t : 0) * a.h;
    typename std::conditional<FP8, RowFp8<NV>, RowBf16<NV>>::type row;
    if (have)
        row.load(reinterpret_cast<const u32x4 *>(xrow), 0, FP8 ? a.h >> 4 : a.h >> 3);
    const int64_t e = (have && lane < a.K) ? a.topk_idx[tk + lane] : -1;

    // this block's arrival on the call counter (every block of the grid takes one)
    if (tid == 0) {
        const unsigned long long v = atomicAdd(&f.lay.hdr->calls, 1ull);
        const uint32_t arrived = (uint32_t)v;
        s_ok = arrived < gridDim.x;
        s_tag = (uint32_t)(v >> 32) + 1u;
        if (arrived == gridDim.x - 1)
            atomicAdd(&f.lay.hdr->calls, (1ull << 32) - (unsigned long long)gridDim.x);
    }
    __syncthreads();
    const uint32_t tag = s_tag;
    if (!s_ok) {
        if (tid == 0)
            flag_error(a.err, EPX_DEV_WORKSPACE);
        return;
    }

    // the totals, then the offsets scanned once per block into LDS
    if (w == 0) {
        bool ok = true;
        for (int c0 = 0; c0 < ER; c0 += kWave) {
            const int c = c0 + lane;
            uint64_t word;
            ok &= wait_tagged(f.tot + min(c, ER - 1), c < ER, tag, word);
            if (c < ER)
                tot[c] = (int)((uint32_t)word & 0x7FFFFFFFu);
        }
        if (!ok && lane == 0)
            flag_error(a.err, EPX_DEV_WORKSPACE);
    }
    __syncthreads();
    if (tid < kWave)
        wave_exclusive_scan(tot, a.E, off);
    else if (tid < 2 * kWave)
        wave_exclusive_scan(tot + a.E, a.R, off + a.E + 1);
    __syncthreads();
    if (!have)
        return;

    // the token's final positions (lane r < R) and slots (lane k < K)
    const uint64_t *tw = f.tok + (int64_t)t * (a.R + a.K);
    uint64_t pw, sw;
    const bool ok_p = wait_tagged(tw + min(lane, a.R - 1), lane < a.R, tag, pw);
    const bool ok_s = wait_tagged(tw + a.R + min(lane, a.K - 1), lane < a.K, tag, sw);
    if (!(ok_p && ok_s) && lane == 0)
        flag_error(a.err, EPX_DEV_WORKSPACE);
    int64_t send_r = -1, recv_r = -1;
    if (ok_p && lane < a.R) {
        const int p = (int)(uint32_t)pw;
        if (p >= 0)
            send_r = (int64_t)off[a.E + 1 + lane] + p;
    }
    const bool valid = e >= 0 && e < a.E;
    if (ok_s && valid) {
        const int sl = (int)(uint32_t)sw;
        recv_r = sl >= 0 ? (int64_t)off[(int)e] + sl : -1;
    }
    dispatch_token<FP8>(a, t, row, xrow, e, send_r, recv_r);
}

template <int KMAX, bool FP8, int NV>
void launch_fused_k(const FusedArgs &f, hipStream_t stream)
{
    const int64_t disp_blocks = (f.disp.T + kFusedTokens - 1) / kFusedTokens;
    const int64_t blocks = f.lay.ntiles > 0 ? f.lay.ntiles + 1 + disp_blocks : 1;
    hipLaunchKernelGGL((fused_kernel<KMAX, FP8, NV>), dim3((unsigned)blocks),
                       dim3(kLayoutThreads), layout_lds_bytes(f.lay.E, f.lay.R), stream, f);
}

template <int KMAX>
void launch_fused_kmax(const FusedArgs &f, bool fp8, hipStream_t stream)
{
    switch (pick_nv(f.disp.h, fp8) + (fp8 ? 100 : 0)) {
    case 8: launch_fused_k<KMAX, false, 8>(f, stream); break;
    case 14: launch_fused_k<KMAX, false, 14>(f, stream); break;
    case 16: launch_fused_k<KMAX, false, 16>(f, stream); break;
    case 104: launch_fused_k<KMAX, true, 4>(f, stream); break;
    case 107: launch_fused_k<KMAX, true, 7>(f, stream); break;
    default: launch_fused_k<KMAX, true, 8>(f, stream); break;
    }
}

}  // namespace

size_t fused_workspace_bytes(int T, int K, int E, int R)
{
    const size_t base = layout_workspace_bytes(T, E, R);
    if (base == 0)
        return 0;
    // the layout's, then the totals row, then the tokens' words
    return base + (size_t)(E + R) * sizeof(uint64_t) + (size_t)T * (R + K) * sizeof(uint64_t);
}

hipError_t launch_fused(const FusedArgs &f, bool fp8, hipStream_t stream)
{
    if (f.lay.K <= 8)
        launch_fused_kmax<8>(f, fp8, stream);
    else
        launch_fused_kmax<EPX_MAX_TOPK>(f, fp8, stream);
    return hipGetLastError();
}

}  // namespace epx
