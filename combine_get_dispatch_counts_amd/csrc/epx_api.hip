// epx_api.hip -- the C ABI declared in include/epx.h: argument checks, then
// kernel launches on the caller's stream. No call here allocates device
// memory except epx_create (the context's error word and stamp ring), and no
// call waits for the GPU except epx_get_error and epx_calibrate_sweep_rate.
#include <stdint.h>
#include <stdlib.h>

#include <mutex>
#include <new>

#include <hip/hip_runtime.h>

#include "epx.h"
#include "epx_internal.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_routing(int T, int K, int E, int R)
{
    if (T < 0 || K < 1 || K > EPX_MAX_TOPK || E < 1 || E > EPX_MAX_EXPERTS || R < 1 ||
        R > EPX_MAX_RANKS || E % R != 0)
        return EPX_EINVAL;
    if ((int64_t)T * K > INT32_MAX)
        return EPX_EINVAL;
    return EPX_OK;
}

int check_hidden(int h, int fp8)
{
    if (h < 8 || h % 8 != 0)
        return EPX_EINVAL;
    if (fp8 && h % 128 != 0)
        return EPX_EUNSUPPORTED;
    return EPX_OK;
}

// The context's device must be the current one: kernels launch there.
int check_ctx(const epx_ctx *ctx)
{
    if (!ctx)
        return EPX_EINVAL;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess)
        return EPX_EHIP;
    return cur == ctx->device ? EPX_OK : EPX_EINVAL;
}

int launched(hipError_t e) { return e == hipSuccess ? EPX_OK : EPX_EHIP; }

}  // namespace

// The workspace of epx_get_dispatch_layout_noalloc, for callers that cannot
// allocate: a device array that each GPU the library runs on holds (its own
// copy) until the process ends. In host code its name stands for no device
// address: kernels and fills only ever get the address from
// hipGetSymbolAddress, looked up once per device.
static __device__ __align__(256) unsigned char scratch[EPX_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on `device` (the current device), found
// on the first call for that device and kept.
int noalloc_scratch_setup(int device, void **ptr)
{
    if (device < 0 || device >= kMaxDevices)
        return EPX_EINVAL;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return EPX_EHIP;
        g_scratch_ptr[device] = p;
    }
    *ptr = g_scratch_ptr[device];
    return EPX_OK;
}

}  // namespace

extern "C" {

int epx_create(epx_ctx **out, int device)
{
    if (!out)
        return EPX_EINVAL;
    *out = nullptr;
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess)
        return EPX_EHIP;
    if (device < 0 || device >= n)
        return EPX_EINVAL;
    int prev = 0;
    if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(device) != hipSuccess)
        return EPX_EHIP;
    epx_ctx *c = new (std::nothrow) epx_ctx();
    int rc = EPX_OK;
    if (!c) {
        rc = EPX_EHIP;
    } else {
        c->device = device;
        c->sweep_gbps[0] = epx::kSweepGBpsBf16;
        c->sweep_gbps[1] = epx::kSweepGBpsFp8;
        c->stamp_seq.store(0u);
        if (hipDeviceGetAttribute(&c->cus, hipDeviceAttributeMultiprocessorCount, device) !=
                hipSuccess ||
            hipDeviceGetAttribute(&c->wclk_khz, hipDeviceAttributeWallClockRate, device) !=
                hipSuccess ||
            hipMalloc(reinterpret_cast<void **>(&c->dev), sizeof(epx::CtxDev)) != hipSuccess ||
            hipMemset(c->dev, 0, sizeof(epx::CtxDev)) != hipSuccess ||
            noalloc_scratch_setup(device, &c->scratch) != EPX_OK) {
            if (c->dev)
                (void)hipFree(c->dev);
            delete c;
            c = nullptr;
            rc = EPX_EHIP;
        } else {
            c->d_err = &c->dev->err;
        }
    }
    (void)hipSetDevice(prev);
    *out = c;
    return rc;
}

int epx_destroy(epx_ctx *ctx)
{
    if (!ctx)
        return EPX_EINVAL;
    int prev = 0;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(ctx->device);
    const hipError_t e = hipFree(ctx->dev);
    (void)hipSetDevice(prev);
    delete ctx;
    return e == hipSuccess ? EPX_OK : EPX_EHIP;
}

const char *epx_strerror(int code)
{
    switch (code) {
    case EPX_OK: return "ok";
    case EPX_EINVAL: return "invalid argument (shape, parameter, pointer or device)";
    case EPX_ECAPACITY: return "capacity exceeded (T > cap, or workspace too small)";
    case EPX_EUNSUPPORTED: return "unsupported (FP8 needs h % 128 == 0)";
    case EPX_EHIP: return "HIP runtime or launch error";
    case EPX_EDEVICE: return "a kernel reported an error (see the device flags)";
    default: return "unknown error code";
    }
}

int epx_workspace_size(int T, int K, int E, int R, size_t *bytes)
{
    if (!bytes)
        return EPX_EINVAL;
    const int rc = check_routing(T, K, E, R);
    if (rc != EPX_OK)
        return rc;
    *bytes = epx::layout_workspace_bytes(T, E, R);
    return EPX_OK;
}

int epx_scale_stride(int h)
{
    if (check_hidden(h, 1) != EPX_OK)
        return 0;
    return epx::scale_stride(h);
}

size_t epx_ll_size_hint(int max_tokens_per_rank, int h, int R, int E, int fp8)
{
    if (max_tokens_per_rank < 1 || check_hidden(h, fp8) != EPX_OK || R < 1 || E < 1 ||
        E % R != 0)
        return 0;
    // every array of the layout starts on a 128-byte boundary
    const auto up = [](size_t n) { return (n + 127) / 128 * 128; };
    const size_t rows = (size_t)E * R * max_tokens_per_rank;
    size_t total = up(rows * (fp8 ? (size_t)h : (size_t)h * 2));
    if (fp8)
        total += up(rows * (size_t)epx::scale_stride(h) * sizeof(float));
    total += up(rows * sizeof(int32_t));                 // source index per row
    total += up((size_t)E * R * sizeof(int32_t));        // count per region
    return up(total);
}

// Checks and packs the layout call's arguments (the workspace is checked by
// the caller, against its own size).
static int layout_args(epx_ctx *ctx, const int64_t *topk_idx, int T, int K, int E, int R, int C,
                       int32_t *num_tokens_per_expert, int32_t *num_tokens_per_rank,
                       uint8_t *is_token_in_rank, int32_t *rank_off, int32_t *exp_off,
                       int32_t *pos_in_rank, int32_t *slot_in_expert, int32_t *channel_prefix,
                       int32_t *totals, int32_t *totals_host_mapped, void *ws,
                       epx::LayoutArgs &a)
{
    int rc = check_ctx(ctx);
    if (rc != EPX_OK)
        return rc;
    if ((rc = check_routing(T, K, E, R)) != EPX_OK)
        return rc;
    if (channel_prefix && (C < 1 || C > (1 << 20)))
        return EPX_EINVAL;
    if (!num_tokens_per_expert || !num_tokens_per_rank || !rank_off || !exp_off || !totals)
        return EPX_EINVAL;
    if (T > 0 && (!topk_idx || !is_token_in_rank || !pos_in_rank || !slot_in_expert))
        return EPX_EINVAL;
    if (T > 0 && (!aligned16(is_token_in_rank) || !aligned16(pos_in_rank) ||
                  !aligned16(slot_in_expert)))
        return EPX_EINVAL;
    const size_t need = epx::layout_workspace_bytes(T, E, R);
    if (need > 0 && !ws)
        return EPX_EINVAL;
    a = epx::LayoutArgs{};
    a.topk_idx = topk_idx;
    a.T = T; a.K = K; a.E = E; a.R = R; a.L = E / R;
    a.L_mul = epx::div_magic(E / R);
    a.C = channel_prefix ? C : 0;
    a.ntiles = (T + epx::kLayoutTile - 1) / epx::kLayoutTile;
    a.hdr = static_cast<epx::LayoutHdr *>(ws);
    a.pub = need ? reinterpret_cast<uint64_t *>(static_cast<char *>(ws) + sizeof(epx::LayoutHdr))
                 : nullptr;
    a.num_tokens_per_expert = num_tokens_per_expert;
    a.num_tokens_per_rank = num_tokens_per_rank;
    a.is_token_in_rank = is_token_in_rank;
    a.rank_off = rank_off;
    a.exp_off = exp_off;
    a.pos_in_rank = pos_in_rank;
    a.slot_in_expert = slot_in_expert;
    a.channel_prefix = channel_prefix;
    a.totals = totals;
    a.totals_host_mapped = totals_host_mapped;
    a.err = ctx->d_err;
    return EPX_OK;
}

int epx_get_dispatch_layout(epx_ctx *ctx, const int64_t *topk_idx, int T, int K, int E, int R,
                            int C, int32_t *num_tokens_per_expert, int32_t *num_tokens_per_rank,
                            uint8_t *is_token_in_rank, int32_t *rank_off, int32_t *exp_off,
                            int32_t *pos_in_rank, int32_t *slot_in_expert,
                            int32_t *channel_prefix, int32_t *totals,
                            int32_t *totals_host_mapped, void *ws, size_t ws_bytes,
                            hipStream_t stream)
{
    epx::LayoutArgs a;
    const int rc = layout_args(ctx, topk_idx, T, K, E, R, C, num_tokens_per_expert,
                               num_tokens_per_rank, is_token_in_rank, rank_off, exp_off,
                               pos_in_rank, slot_in_expert, channel_prefix, totals,
                               totals_host_mapped, ws, a);
    if (rc != EPX_OK)
        return rc;
    if (ws_bytes < epx::layout_workspace_bytes(T, E, R))
        return EPX_ECAPACITY;
    return launched(epx::launch_layout(a, stream));
}

int epx_get_dispatch_layout_noalloc(epx_ctx *ctx, const int64_t *topk_idx, int T, int K, int E,
                                    int R, int C, int32_t *num_tokens_per_expert,
                                    int32_t *num_tokens_per_rank, uint8_t *is_token_in_rank,
                                    int32_t *rank_off, int32_t *exp_off, int32_t *pos_in_rank,
                                    int32_t *slot_in_expert, int32_t *channel_prefix,
                                    int32_t *totals, int32_t *totals_host_mapped,
                                    hipStream_t stream)
{
    if (!ctx)
        return EPX_EINVAL;
    epx::LayoutArgs a;
    const int rc = layout_args(ctx, topk_idx, T, K, E, R, C, num_tokens_per_expert,
                               num_tokens_per_rank, is_token_in_rank, rank_off, exp_off,
                               pos_in_rank, slot_in_expert, channel_prefix, totals,
                               totals_host_mapped, ctx->scratch, a);
    if (rc != EPX_OK)
        return rc;
    const size_t need = epx::layout_workspace_bytes(T, E, R);
    if (need > EPX_NOALLOC_SCRATCH_BYTES)
        return EPX_ECAPACITY;
    // the array keeps what the last call left: the part this call uses
    // starts from zero (a fill kernel, so a captured graph may hold it)
    if (a.ntiles > 1) {
        const hipError_t e = epx::launch_fill_i32(static_cast<int32_t *>(ctx->scratch),
                                                  (int64_t)(need / sizeof(int32_t)), 0, stream);
        if (e != hipSuccess)
            return EPX_EHIP;
    }
    return launched(epx::launch_layout(a, stream));
}

// Checks and packs the dispatch call's arguments.
static int dispatch_args(epx_ctx *ctx, const uint16_t *x, int h, const int64_t *topk_idx,
                         const float *topk_w, int T, int K, int E, int R,
                         const int32_t *rank_off, const int32_t *exp_off,
                         const int32_t *pos_in_rank, const int32_t *slot_in_expert, int fp8,
                         void *send_x, float *send_scales, int32_t *send_src,
                         int64_t *send_topk_idx, float *send_topk_w, int64_t send_cap_rows,
                         void *recv_x, float *recv_scales, int32_t *recv_src,
                         int64_t recv_cap_rows, int32_t *pos_exp, epx::DispatchArgs &a)
{
    int rc = check_ctx(ctx);
    if (rc != EPX_OK)
        return rc;
    if ((rc = check_routing(T, K, E, R)) != EPX_OK)
        return rc;
    if ((rc = check_hidden(h, fp8)) != EPX_OK)
        return rc;
    if (send_cap_rows < 0 || recv_cap_rows < 0)
        return EPX_EINVAL;
    const bool pack = send_x != nullptr;  // else the permute alone
    if (T > 0) {
        if (!x || !topk_idx || !exp_off || !slot_in_expert || !pos_exp || !recv_x || !recv_src)
            return EPX_EINVAL;
        if (pack && (!topk_w || !rank_off || !pos_in_rank || !send_src || !send_topk_idx ||
                     !send_topk_w))
            return EPX_EINVAL;
        if (fp8 && (!recv_scales || !aligned16(recv_scales) ||
                    (pack && (!send_scales || !aligned16(send_scales)))))
            return EPX_EINVAL;
        if (!aligned16(x) || !aligned16(recv_x) || (pack && !aligned16(send_x)))
            return EPX_EINVAL;
    }
    a = epx::DispatchArgs{};
    a.x = x; a.topk_idx = topk_idx; a.topk_w = topk_w;
    a.h = h; a.T = T; a.K = K; a.E = E; a.R = R; a.L = E / R;
    a.L_mul = epx::div_magic(E / R);
    a.rank_off = rank_off; a.exp_off = exp_off;
    a.pos_in_rank = pos_in_rank; a.slot_in_expert = slot_in_expert;
    a.send_x = send_x; a.send_scales = send_scales; a.send_src = send_src;
    a.send_topk_idx = send_topk_idx; a.send_topk_w = send_topk_w; a.send_cap = send_cap_rows;
    a.recv_x = recv_x; a.recv_scales = recv_scales; a.recv_src = recv_src;
    a.recv_cap = recv_cap_rows; a.pos_exp = pos_exp;
    a.err = ctx->d_err;
    // the paced sweep's rate in bytes per wall-clock tick (GB/s = 1e6 B per ms);
    // the permute alone reads a row for every row it writes, so the write
    // rate alone does not describe its traffic: it is left unpaced
    const int64_t gbps = pack ? ctx->sweep_gbps[fp8 ? 1 : 0] : 0;
    a.sweep_bpt = ctx->wclk_khz > 0 ? (uint32_t)(gbps * 1000000 / ctx->wclk_khz) : 0u;
    if (gbps > 0 && a.sweep_bpt == 0)
        a.sweep_bpt = 1;
    // at most T*min(K,R) send rows and T*K receive rows
    const int64_t row_bytes = fp8 ? (int64_t)h + 4 * (int64_t)epx::scale_stride(h) : 2 * (int64_t)h;
    const int64_t bound = (int64_t)T * (K + (K < R ? K : R)) * row_bytes;
    if (bound <= (fp8 ? epx::kSweepMinBytesFp8 : epx::kSweepMinBytesBf16))
        a.sweep_bpt = 0;
    // a row longer than one register pass is stored a slice per pass, and
    // only the first pass could keep to the schedule: such rows go unpaced
    if (h > epx::kSweepMaxChannels)
        a.sweep_bpt = 0;
    // late waves: an eighth of the longest sweep the call can have, kept
    // within [4, 16] microseconds of the wall clock
    a.stamps = ctx->dev->stamp;
    a.start_ticks = 0;
    a.wclk_per_us = (uint32_t)(ctx->wclk_khz / 1000);
    if (a.sweep_bpt) {
        const int64_t lo = (int64_t)ctx->wclk_khz * 4 / 1000, hi = (int64_t)ctx->wclk_khz * 16 / 1000;
        int64_t lt = bound / a.sweep_bpt / 8;
        lt = lt < lo ? lo : (lt > hi ? hi : lt);
        a.late_ticks = (uint32_t)lt;
    }
    return EPX_OK;
}

int epx_dispatch(epx_ctx *ctx, const uint16_t *x, int h, const int64_t *topk_idx,
                 const float *topk_w, int T, int K, int E, int R, const int32_t *rank_off,
                 const int32_t *exp_off, const int32_t *pos_in_rank,
                 const int32_t *slot_in_expert, int fp8, void *send_x, float *send_scales,
                 int32_t *send_src, int64_t *send_topk_idx, float *send_topk_w,
                 int64_t send_cap_rows, void *recv_x, float *recv_scales, int32_t *recv_src,
                 int64_t recv_cap_rows, int32_t *pos_exp, hipStream_t stream)
{
    epx::DispatchArgs a;
    const int rc = dispatch_args(ctx, x, h, topk_idx, topk_w, T, K, E, R, rank_off, exp_off,
                                 pos_in_rank, slot_in_expert, fp8, send_x, send_scales, send_src,
                                 send_topk_idx, send_topk_w, send_cap_rows, recv_x, recv_scales,
                                 recv_src, recv_cap_rows, pos_exp, a);
    if (rc != EPX_OK)
        return rc;
    return launched(epx::launch_dispatch(a, fp8 != 0, ctx->cus, &ctx->stamp_seq, stream));
}

int epx_permute(epx_ctx *ctx, const void *rows, int row_bytes, const void *side, int side_bytes,
                const int64_t *local_topk_idx, int N, int K, int L, const int32_t *exp_off,
                const int32_t *slot_in_expert, void *out_rows, void *out_side,
                int32_t *src_row, int64_t cap_rows, int32_t *pos, hipStream_t stream)
{
    const int rc = check_ctx(ctx);
    if (rc != EPX_OK)
        return rc;
    if (N < 0 || K < 1 || K > EPX_MAX_TOPK || L < 1 || L > EPX_MAX_EXPERTS || cap_rows < 0 ||
        cap_rows > INT32_MAX || (int64_t)N * K > INT32_MAX)
        return EPX_EINVAL;
    if (row_bytes < 16 || row_bytes % 16 != 0 || row_bytes > (1 << 20) || side_bytes < 0 ||
        side_bytes % 16 != 0 || side_bytes > 16 * 64)
        return EPX_EINVAL;
    if (N > 0) {
        if (!rows || !local_topk_idx || !exp_off || !slot_in_expert || !out_rows || !src_row ||
            !pos || (side_bytes > 0 && (!side || !out_side)))
            return EPX_EINVAL;
        if (!aligned16(rows) || !aligned16(out_rows) ||
            (side_bytes > 0 && (!aligned16(side) || !aligned16(out_side))))
            return EPX_EINVAL;
    }
    epx::PermuteArgs a{};
    a.rows = rows; a.side = side; a.row_vecs = row_bytes / 16; a.side_vecs = side_bytes / 16;
    a.idx = local_topk_idx; a.N = N; a.K = K; a.L = L;
    a.exp_off = exp_off; a.slot = slot_in_expert;
    a.out_rows = out_rows; a.out_side = out_side; a.src_row = src_row; a.pos = pos;
    a.cap = cap_rows; a.err = ctx->d_err;
    return launched(epx::launch_permute(a, stream));
}

int epx_set_sweep_rate(epx_ctx *ctx, int bf16_gbps, int fp8_gbps)
{
    if (!ctx || bf16_gbps < 0 || fp8_gbps < 0 || bf16_gbps > EPX_MAX_SWEEP_GBPS ||
        fp8_gbps > EPX_MAX_SWEEP_GBPS)
        return EPX_EINVAL;
    ctx->sweep_gbps[0] = bf16_gbps;
    ctx->sweep_gbps[1] = fp8_gbps;
    return EPX_OK;
}

int epx_get_sweep_rate(epx_ctx *ctx, int *bf16_gbps, int *fp8_gbps)
{
    if (!ctx || !bf16_gbps || !fp8_gbps)
        return EPX_EINVAL;
    *bf16_gbps = ctx->sweep_gbps[0];
    *fp8_gbps = ctx->sweep_gbps[1];
    return EPX_OK;
}

int epx_calibrate_sweep_rate(epx_ctx *ctx, void *scratch, size_t bytes, int *fill_gbps,
                             hipStream_t stream)
{
    int rc = check_ctx(ctx);
    if (rc != EPX_OK)
        return rc;
    if (!scratch || !aligned16(scratch) || bytes < epx::kCalibMinBytes)
        return EPX_EINVAL;
    const size_t n = bytes / epx::kFillBlockBytes * epx::kFillBlockBytes;
    hipEvent_t ev[2] = {nullptr, nullptr};
    if (hipEventCreate(&ev[0]) != hipSuccess || hipEventCreate(&ev[1]) != hipSuccess) {
        for (hipEvent_t e : ev)
            if (e)
                (void)hipEventDestroy(e);
        return EPX_EHIP;
    }
    // three warm-up fills, then the median of nine timed ones
    constexpr int kWarm = 3, kTimed = 9;
    float ms[kTimed];
    rc = EPX_OK;
    for (int i = 0; i < kWarm + kTimed && rc == EPX_OK; ++i) {
        const bool timed = i >= kWarm;
        if (timed && hipEventRecord(ev[0], stream) != hipSuccess)
            rc = EPX_EHIP;
        if (rc == EPX_OK && epx::launch_fill_lines(scratch, n, (uint32_t)i, stream) != hipSuccess)
            rc = EPX_EHIP;
        if (rc == EPX_OK && timed &&
            (hipEventRecord(ev[1], stream) != hipSuccess || hipEventSynchronize(ev[1]) != hipSuccess ||
             hipEventElapsedTime(&ms[i - kWarm], ev[0], ev[1]) != hipSuccess))
            rc = EPX_EHIP;
    }
    (void)hipEventDestroy(ev[0]);
    (void)hipEventDestroy(ev[1]);
    if (rc != EPX_OK)
        return rc;
    for (int i = 1; i < kTimed; ++i)  // insertion sort
        for (int j = i; j > 0 && ms[j] < ms[j - 1]; --j) {
            const float t = ms[j];
            ms[j] = ms[j - 1];
            ms[j - 1] = t;
        }
    const float med = ms[kTimed / 2];
    if (!(med > 0.0f))
        return EPX_EHIP;
    const double gbps = (double)n / (med * 1e-3) / 1e9;
    const double b = gbps * epx::kCalibBf16Permille / 1000.0, f = gbps * epx::kCalibFp8Permille / 1000.0;
    ctx->sweep_gbps[0] = b > EPX_MAX_SWEEP_GBPS ? EPX_MAX_SWEEP_GBPS : (int)b;
    ctx->sweep_gbps[1] = f > EPX_MAX_SWEEP_GBPS ? EPX_MAX_SWEEP_GBPS : (int)f;
    if (fill_gbps)
        *fill_gbps = gbps > INT32_MAX ? INT32_MAX : (int)gbps;
    return EPX_OK;
}

int epx_fused_workspace_size(int T, int K, int E, int R, size_t *bytes)
{
    if (!bytes)
        return EPX_EINVAL;
    const int rc = check_routing(T, K, E, R);
    if (rc != EPX_OK)
        return rc;
    *bytes = epx::fused_workspace_bytes(T, K, E, R);
    return EPX_OK;
}

int epx_fused_launches(epx_ctx *ctx, int T, int h, int K, int E, int R, int fp8, int *launches)
{
    if (!launches)
        return EPX_EINVAL;
    int rc = check_ctx(ctx);
    if (rc != EPX_OK)
        return rc;
    if ((rc = check_routing(T, K, E, R)) != EPX_OK || (rc = check_hidden(h, fp8)) != EPX_OK)
        return rc;
    epx::FusedArgs f{};
    f.lay.T = T;
    f.lay.K = K;
    f.lay.E = E;
    f.lay.R = R;
    f.lay.ntiles = (T + epx::kLayoutTile - 1) / epx::kLayoutTile;
    f.disp.T = T;
    f.disp.h = h;
    f.cus = ctx->cus;
    return epx::fused_launches(f, fp8 != 0, launches) == hipSuccess ? EPX_OK : EPX_EHIP;
}

int epx_dispatch_fused(epx_ctx *ctx, const uint16_t *x, int h, const int64_t *topk_idx,
                       const float *topk_w, int T, int K, int E, int R, int C,
                       int32_t *num_tokens_per_expert, int32_t *num_tokens_per_rank,
                       uint8_t *is_token_in_rank, int32_t *rank_off, int32_t *exp_off,
                       int32_t *pos_in_rank, int32_t *slot_in_expert, int32_t *channel_prefix,
                       int32_t *totals, int32_t *totals_host_mapped, void *ws, size_t ws_bytes,
                       int fp8, void *send_x, float *send_scales, int32_t *send_src,
                       int64_t *send_topk_idx, float *send_topk_w, int64_t send_cap_rows,
                       void *recv_x, float *recv_scales, int32_t *recv_src,
                       int64_t recv_cap_rows, int32_t *pos_exp, hipStream_t stream)
{
    epx::FusedArgs f{};
    int rc = layout_args(ctx, topk_idx, T, K, E, R, C, num_tokens_per_expert,
                         num_tokens_per_rank, is_token_in_rank, rank_off, exp_off, pos_in_rank,
                         slot_in_expert, channel_prefix, totals, totals_host_mapped, ws, f.lay);
    if (rc != EPX_OK)
        return rc;
    if (T > 0 && !send_x)  // the fused call always packs
        return EPX_EINVAL;
    rc = dispatch_args(ctx, x, h, topk_idx, topk_w, T, K, E, R, rank_off, exp_off, pos_in_rank,
                       slot_in_expert, fp8, send_x, send_scales, send_src, send_topk_idx,
                       send_topk_w, send_cap_rows, recv_x, recv_scales, recv_src, recv_cap_rows,
                       pos_exp, f.disp);
    if (rc != EPX_OK)
        return rc;
    if (ws_bytes < epx::fused_workspace_bytes(T, K, E, R))
        return EPX_ECAPACITY;
    f.cus = ctx->cus;
    return launched(epx::launch_fused(f, fp8 != 0, &ctx->stamp_seq, stream));
}

int epx_combine(epx_ctx *ctx, const uint16_t *expert_out, int64_t n_rows, int h,
                const float *topk_w, const int32_t *pos, int T, int K, uint16_t *out,
                hipStream_t stream)
{
    int rc = check_ctx(ctx);
    if (rc != EPX_OK)
        return rc;
    if (T < 0 || K < 1 || K > EPX_MAX_TOPK || n_rows < 0 || (int64_t)T * K > INT32_MAX)
        return EPX_EINVAL;
    if ((rc = check_hidden(h, 0)) != EPX_OK)
        return rc;
    if (T > 0) {
        if (!topk_w || !pos || !out || (n_rows > 0 && !expert_out))
            return EPX_EINVAL;
        if (!aligned16(out) || !aligned16(expert_out))
            return EPX_EINVAL;
    }
    epx::CombineArgs a{};
    a.y = expert_out; a.n_rows = n_rows; a.h = h; a.T = T; a.K = K;
    a.topk_w = topk_w; a.pos = pos; a.out = out; a.err = ctx->d_err;
    return launched(epx::launch_combine(a, stream));
}

int epx_combine_partial(epx_ctx *ctx, const uint16_t *expert_out, int64_t n_rows, int h,
                        const int32_t *send_src, const int64_t *send_topk_idx,
                        const float *send_topk_w, const int32_t *pos_exp, int T, int K,
                        int64_t send_cap_rows, const int32_t *num_send_rows, uint16_t *partial,
                        hipStream_t stream)
{
    int rc = check_ctx(ctx);
    if (rc != EPX_OK)
        return rc;
    if (T < 0 || K < 1 || K > EPX_MAX_TOPK || n_rows < 0 || send_cap_rows < 0 ||
        (int64_t)T * K > INT32_MAX || send_cap_rows > INT32_MAX)
        return EPX_EINVAL;
    if ((rc = check_hidden(h, 0)) != EPX_OK)
        return rc;
    if (send_cap_rows > 0) {
        if (!send_src || !send_topk_idx || !send_topk_w || !partial || (T > 0 && !pos_exp) ||
            (n_rows > 0 && !expert_out))
            return EPX_EINVAL;
        if (!aligned16(partial) || !aligned16(expert_out))
            return EPX_EINVAL;
    }
    epx::PartialArgs a{};
    a.y = expert_out; a.n_rows = n_rows; a.h = h; a.T = T; a.K = K;
    a.send_src = send_src; a.send_topk_idx = send_topk_idx; a.send_topk_w = send_topk_w;
    a.pos_exp = pos_exp; a.cap_rows = send_cap_rows; a.num_rows = num_send_rows;
    a.partial = partial; a.err = ctx->d_err;
    return launched(epx::launch_combine_partial(a, stream));
}

int epx_combine_final(epx_ctx *ctx, const uint16_t *partial, int64_t n_partial_rows, int h,
                      const int32_t *rank_off, const int32_t *pos_in_rank, int T, int R,
                      uint16_t *out, hipStream_t stream)
{
    int rc = check_ctx(ctx);
    if (rc != EPX_OK)
        return rc;
    if (T < 0 || R < 1 || R > EPX_MAX_RANKS || n_partial_rows < 0 ||
        n_partial_rows > INT32_MAX)
        return EPX_EINVAL;
    if ((rc = check_hidden(h, 0)) != EPX_OK)
        return rc;
    if (T > 0) {
        if (!rank_off || !pos_in_rank || !out || (n_partial_rows > 0 && !partial))
            return EPX_EINVAL;
        if (!aligned16(out) || !aligned16(partial))
            return EPX_EINVAL;
    }
    epx::FinalArgs a{};
    a.partial = partial; a.n_rows = n_partial_rows; a.h = h; a.T = T; a.R = R;
    a.rank_off = rank_off; a.pos_in_rank = pos_in_rank; a.out = out; a.err = ctx->d_err;
    return launched(epx::launch_combine_final(a, stream));
}

int epx_ll_reset(epx_ctx *ctx, int32_t *ll_count, int64_t n, hipStream_t stream)
{
    const int rc = check_ctx(ctx);
    if (rc != EPX_OK)
        return rc;
    if (n < 0 || (n > 0 && !ll_count))
        return EPX_EINVAL;
    return launched(epx::launch_fill_i32(ll_count, n, -1, stream));
}

int epx_ll_dispatch(epx_ctx *ctx, const uint16_t *x, int h, const int64_t *topk_idx, int T,
                    int K, int E, int R, int src_rank, int cap, int R_buf, int fp8, void *ll_x,
                    float *ll_scales, int32_t *ll_src, int32_t *ll_count, int32_t *pos_ll,
                    int32_t *next_ll_count, int64_t n_next, int32_t *ll_stats,
                    hipStream_t stream)
{
    int rc = check_ctx(ctx);
    if (rc != EPX_OK)
        return rc;
    if ((rc = check_routing(T, K, E, R)) != EPX_OK)
        return rc;
    if ((rc = check_hidden(h, fp8)) != EPX_OK)
        return rc;
    if (cap < 1 || src_rank < 0 || src_rank >= R || (R_buf != R && R_buf != 1))
        return EPX_EINVAL;
    if ((int64_t)E * R_buf * cap > INT32_MAX)
        return EPX_EINVAL;
    if (T > cap)
        return EPX_ECAPACITY;
    if (!ll_count || (T > 0 && (!x || !topk_idx || !ll_x || !ll_src || !pos_ll)))
        return EPX_EINVAL;
    if (T > 0 && fp8 && (!ll_scales || !aligned16(ll_scales)))
        return EPX_EINVAL;
    if (T > 0 && (!aligned16(x) || !aligned16(ll_x)))
        return EPX_EINVAL;
    if (n_next < 0 || (n_next > 0 && !next_ll_count))
        return EPX_EINVAL;
    if (n_next > 0) {  // the two count arrays of a pair must not overlap
        const int32_t *c0 = ll_count, *c1 = ll_count + (int64_t)E * R_buf;
        const int32_t *n0 = next_ll_count, *n1 = next_ll_count + n_next;
        if (n0 < c1 && c0 < n1)
            return EPX_EINVAL;
    }
    epx::LLArgs a{};
    a.x = x; a.topk_idx = topk_idx; a.h = h; a.T = T; a.K = K; a.E = E; a.R = R;
    a.src_rank = src_rank; a.cap = cap; a.R_buf = R_buf;
    a.ll_x = ll_x; a.ll_scales = ll_scales; a.ll_src = ll_src; a.ll_count = ll_count;
    a.pos_ll = pos_ll; a.err = ctx->d_err;
    a.clear_count = next_ll_count; a.n_clear = n_next; a.stats = ll_stats;
    return launched(epx::launch_ll_dispatch(a, fp8 != 0, stream));
}

int epx_get_error(epx_ctx *ctx, int *device_flags, hipStream_t stream)
{
    const int rc = check_ctx(ctx);
    if (rc != EPX_OK)
        return rc;
    if (!device_flags)
        return EPX_EINVAL;
    int v = 0;
    if (hipMemcpyAsync(&v, ctx->d_err, sizeof(int), hipMemcpyDeviceToHost, stream) != hipSuccess)
        return EPX_EHIP;
    if (epx::launch_fill_i32(ctx->d_err, 1, 0, stream) != hipSuccess)
        return EPX_EHIP;
    if (hipStreamSynchronize(stream) != hipSuccess)
        return EPX_EHIP;
    *device_flags = v;
    return v ? EPX_EDEVICE : EPX_OK;
}

}  // extern "C"
