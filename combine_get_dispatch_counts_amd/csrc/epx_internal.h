// epx_internal.h -- launcher interface between the C ABI (epx_api.hip) and
// the kernel translation units. Argument checking happens in epx_api.hip;
// launchers assume valid shapes and return the HIP launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace epx {

// Launch stamps of the paced sweep: a paced launch takes the next slot of a
// ring of this many 64-bit words in the context's device memory (a chunked
// dispatch one slot per chunk), where its first block stores the wall clock
// at its start.
constexpr int kStampSlots = 64;

// Device memory of a context: the error word (EPX_DEV_* bits) on a line of
// its own, then the stamp ring.
struct CtxDev {
    int err;
    int pad[31];
    unsigned long long stamp[kStampSlots];
};

}  // namespace epx

struct epx_ctx {
    int device;
    int cus;                 // compute units of the device
    epx::CtxDev *dev;        // device memory of the context
    int *d_err;              // &dev->err
    int wclk_khz;            // rate of the device's constant wall clock (wall_clock64)
    int sweep_gbps[2];       // paced row-store sweep rate for bf16 and FP8 rows (0: off)
    std::atomic<unsigned> stamp_seq;  // next slot of the stamp ring
    void *scratch;           // device address of this device's no-alloc scratch array
};

namespace epx {

// Default rates of the paced sweep of the high-throughput dispatch's row
// stores (GB/s of destination rows), with each launch's schedule started as
// below, measured on MI355X: some 6% below the rate at which the paced
// front outruns the memory system on some GPUs, where a launch turns into
// random writes and takes 10-25% longer (bf16 prefill, T = 4096: 151-153 us
// at 6600-6700 back to back, but 171 us at 6900 on one of two GPUs and
// 163 us under a kernel-trace profiler at 6600, against 153 us at 6450;
// FP8 at T = 16384 in chunks 385-389 us at 6400-6500, 394 at 6300, 406 at
// 6700; FP8 at T = 4096 in one launch 88-90 us at 6400-6700, 96-97 at 6900).
constexpr int kSweepGBpsBf16 = 6450;
constexpr int kSweepGBpsFp8 = 6400;
// Pacing holds every wave to its schedule, which costs a few microseconds;
// it repays that only once the rows no longer fit in the
// memory-side cache (256 MiB on MI355X) and must reach HBM within the launch.
// Calls whose row bound (T*(K + min(K,R)) rows) is at most this many bytes are
// left unpaced. Measured at h = 7168, E = 256, R = 32, top-8: bf16 loses with
// pacing up to T = 1280 (235 MB bound: 39.3 us against 36.7 at T = 1024; 294
// MB: 52.0 against 45.7 at T = 1280) and gains from T = 1536 (352 MB: 60.8
// against 65.4); FP8, whose quantisation keeps its unpaced store rate lower,
// gains from T = 1152 (137 MB: 31.2 against 35.1; 182 MB: 38.1 against 43.7
// at T = 1536).
constexpr int64_t kSweepMinBytesBf16 = 320ll << 20;
constexpr int64_t kSweepMinBytesFp8 = 128ll << 20;
// Channels of one register pass of the dispatch kernels' largest row
// (bf16: 16 vectors of 8 channels per lane; FP8: 8 segments of 16): a
// longer row is stored one pass at a time and is left unpaced.
constexpr int kSweepMaxChannels = 8192;

// Where a launch's schedule starts. A paced wave holds each row until its
// place in the sweep falls due, counted from the start of its schedule.
// Started when the wave is ready, the schedules of a launch's waves begin
// over the spread of their row loads (and, in the fused kernel, of the
// layout hand-over, 12-20 us in at the prefill shape): the front is blurred,
// and a wave whose first rows are due before it is ready sends them out
// together as random writes. So a wave starts its schedule when it is ready
// but no earlier than a fixed time after its entry: kDispatchStartUs (the
// dispatch kernel, one launch or a chunk; FP8 rows are quantised once
// loaded, so they take longer) or kFusedStartUs (the fused kernel) plus the
// time the launch's x rows take at its sweep rate. Most waves are ready by
// then; the front starts sharp and keeps up at higher rates. Measured on
// MI355X (HIP events, back to back unless flushed): prefill dispatch
// (T = 4096, h = 7168, E = 256, R = 32, top-8) 154-156 us started when
// ready at 6300 GB/s, 151-152 us from 1 us + x at 6600 (153 us from 3 us;
// the front fell behind at 6900 on one of two GPUs: 171 us); fused step
// flushed / back to back 257 / 254 us against 252-253 / 250 us from 9 us + x
// at 6600; skewed dispatch (T = 8192, h = 4096, E = 64, R = 8, top-6) 130
// against 124-125 us at 6600; FP8 at T = 4096 91-92 against 90 us (on the
// 64-rank routing 97-99 against 92 us; 94 us from 1 us + x), FP8 in chunks
// at T = 16384 400-403 us started when ready at 6100 against 386-392 us
// from 3 us + x at 6400.
constexpr int64_t kDispatchStartUs[2] = {1, 3};  // bf16, FP8
constexpr int64_t kFusedStartUs = 9;

// Ticks for n_tokens rows of h bf16 channels at bpt bytes per tick (0 when
// unpaced).
inline uint32_t load_ticks(int64_t n_tokens, int h, uint32_t bpt)
{
    return bpt ? (uint32_t)(n_tokens * 2 * (int64_t)h / bpt) : 0u;
}

// Calibration (epx_calibrate_sweep_rate): the sweep rates as a fraction of
// the same device's sequential fill rate, measured with launch_fill_lines
// over a buffer larger than the memory-side cache: the defaults above over
// the 6.75 TB/s that fill reached on the GPU they were first measured on.
constexpr int kCalibBf16Permille = 956;
constexpr int kCalibFp8Permille = 948;
constexpr size_t kCalibMinBytes = 512ull << 20;

// The multiplier of floor(e / L) = e * m >> 20 for 0 <= e < 512 and
// 1 <= L <= 512 (an expert and the experts per rank, within
// EPX_MAX_EXPERTS): with m = ceil(2^20 / L) = (2^20 + d) / L, 0 <= d < L,
// e * m / 2^20 exceeds e / L by e * d / (L * 2^20) < 1 / L, because
// e * L < 2^18, so the floor is unchanged; e * m < 2^29 fits in 32 bits.
__host__ __device__ constexpr uint32_t div_magic(int L)
{
    return (uint32_t)(((1u << 20) + (uint32_t)L - 1u) / (uint32_t)L);
}

// fp32 entries per row of an FP8 scale array for hidden size h: the h/128
// group scales rounded up to a multiple of 32, so every row is a whole
// number of 128-byte lines (entries past h/128 hold +0).
__host__ __device__ constexpr int scale_stride(int h)
{
    return ((h >> 7) + 31) & ~31;
}

// Tokens per layout tile: 4 waves of 64 tokens, one token per thread.
constexpr int kLayoutWaves = 4;
constexpr int kLayoutTile = 64 * kLayoutWaves;
constexpr int kLayoutThreads = 2 * kLayoutTile;  // two threads per token of a tile

// Head of the layout workspace (the rest: published words [ntiles, E + R]).
// Zero before the first call; every call leaves it ready for the next.
struct LayoutHdr {
    unsigned long long calls;  // calls completed << 32 (the low half stays 0); the
                               // call's tag (in published words) is calls >> 32, + 1
    int pad[14];
    unsigned int done;  // blocks of the current call that have finished
    int pad2[15];
};

struct LayoutArgs {
    const int64_t *topk_idx;
    int T, K, E, R, L, C;
    uint32_t L_mul;   // div_magic(L): rank of an expert as a multiply and shift
    int ntiles;       // 256-token tiles (the layout kernel's launcher sets its own)
    int subs;         // blocks per tile of the layout kernel (set by its launcher)
    int tile_tokens;  // tokens per tile of the layout kernel (set by its launcher)
    LayoutHdr *hdr;
    uint64_t *pub;  // [ntiles, E + R]
    int32_t *num_tokens_per_expert, *num_tokens_per_rank;
    uint8_t *is_token_in_rank;
    int32_t *rank_off, *exp_off, *pos_in_rank, *slot_in_expert, *channel_prefix;
    int32_t *totals, *totals_host_mapped;
    int *err;
};

size_t layout_workspace_bytes(int T, int E, int R);
hipError_t launch_layout(const LayoutArgs &a, hipStream_t stream);

struct DispatchArgs {
    const uint16_t *x;
    const int64_t *topk_idx;
    const float *topk_w;
    int h, T, K, E, R, L;
    uint32_t L_mul;   // div_magic(L)
    const int32_t *rank_off, *exp_off, *pos_in_rank, *slot_in_expert;
    void *send_x;
    float *send_scales;
    int32_t *send_src;
    int64_t *send_topk_idx;
    float *send_topk_w;
    int64_t send_cap;
    void *recv_x;
    float *recv_scales;
    int32_t *recv_src;
    int64_t recv_cap;
    int32_t *pos_exp;
    int *err;
    // The paced sweep (0: off): each wave stores its token's rows in
    // ascending order of their place in the sweep -- the send rows, then the
    // receive rows -- and none before its own start plus that row's byte
    // offset in the sweep divided by sweep_bpt (bytes per wall-clock tick).
    uint32_t sweep_bpt;
    // This launch's tokens [t_begin, t_begin + t_count) when a dispatch too
    // large for one round of waves is launched in chunks (t_count 0: one
    // launch takes all T); each chunk sweeps its own rows.
    int t_begin, t_count;
    // Late waves of a paced launch: block 0 stores the wall clock at its
    // start in stamps[stamp_slot]; a wave that starts more than late_ticks
    // after it did not find a place in the launch's first round of waves
    // and stores its rows unpaced, so it holds no place waiting for rows
    // that were due long ago (null: no check).
    unsigned long long *stamps;
    int stamp_slot;
    uint32_t late_ticks;
    // Where a paced wave's schedule starts: when the wave has its
    // destinations, but no earlier than start_ticks after it entered the
    // kernel (0 but for the fused launch). wclk_per_us: wall-clock ticks per
    // microsecond.
    uint32_t start_ticks;
    uint32_t wclk_per_us;
};

// Launch the dispatch (cus: compute units of the device). The sweep is paced
// when every token's wave is on the chip at once; with more tokens than that,
// the dispatch is launched in chunks of consecutive tokens that each fit one
// round, each chunk pacing its own rows.
// The next slot of a context's stamp ring (0 without a ring counter).
inline int next_stamp_slot(std::atomic<unsigned> *seq)
{
    return seq ? (int)(seq->fetch_add(1u, std::memory_order_relaxed) % kStampSlots) : 0;
}

// The paced launches take consecutive slots of the stamp ring from *seq.
hipError_t launch_dispatch(const DispatchArgs &a, bool fp8, int cus, std::atomic<unsigned> *seq,
                           hipStream_t stream);

// The receiver's permute (epx_permute): N rows of row_vecs 16-byte vectors
// and side rows of side_vecs vectors into per-local-expert blocks.
struct PermuteArgs {
    const void *rows, *side;
    int row_vecs, side_vecs;
    const int64_t *idx;  // [N, K] local expert indices
    int N, K, L;
    const int32_t *exp_off, *slot;
    void *out_rows, *out_side;
    int32_t *src_row, *pos;
    int64_t cap;
    int *err;
};

hipError_t launch_permute(const PermuteArgs &a, hipStream_t stream);

struct LLArgs {
    const uint16_t *x;
    const int64_t *topk_idx;
    int h, T, K, E, R, src_rank, cap, R_buf;
    void *ll_x;
    float *ll_scales;
    int32_t *ll_src, *ll_count, *pos_ll;
    int32_t *clear_count;  // the other buffer's counts, set to -1 (or null)
    int64_t n_clear;
    int32_t *stats;        // [2]: entries routed, fullest region (or null)
    int *err;
};

hipError_t launch_ll_dispatch(const LLArgs &a, bool fp8, hipStream_t stream);

// Layout and dispatch in one launch: the layout's arguments (workspace head
// and tile words included) and the dispatch's (its layout pointers unused).
struct FusedArgs {
    LayoutArgs lay;
    DispatchArgs disp;
    int cus;  // compute units of the device
};

size_t fused_workspace_bytes(int T, int K, int E, int R);
hipError_t launch_fused(const FusedArgs &f, bool fp8, std::atomic<unsigned> *seq,
                        hipStream_t stream);
hipError_t fused_launches(const FusedArgs &f, bool fp8, int *launches);
hipError_t launch_fill_i32(int32_t *p, int64_t n, int32_t v, hipStream_t stream);

// A sequential fill of n bytes (a multiple of kFillBlockBytes) with the
// word v: each one-wave block writes one contiguous kFillBlockBytes chunk
// with 16-byte stores, chunks in block order (of the fill patterns measured
// on MI355X, 4 KB per wave is the fastest: 6.75-6.79 TB/s, against 6.0-6.1
// for 16 KB per 256-thread block and 6.5-6.6 for hipMemsetD32).
constexpr size_t kFillBlockBytes = 4096;
hipError_t launch_fill_lines(void *p, size_t n, uint32_t v, hipStream_t stream);

struct CombineArgs {
    const uint16_t *y;
    int64_t n_rows;
    int h, T, K;
    const float *topk_w;
    const int32_t *pos;
    uint16_t *out;
    int *err;
};

hipError_t launch_combine(const CombineArgs &a, hipStream_t stream);

struct PartialArgs {
    const uint16_t *y;  // expert outputs [n_rows, h]
    int64_t n_rows;
    int h, T, K;
    const int32_t *send_src;
    const int64_t *send_topk_idx;
    const float *send_topk_w;
    const int32_t *pos_exp;
    int64_t cap_rows;         // rank-major rows launched
    const int32_t *num_rows;  // device row count, or null (all cap_rows)
    uint16_t *partial;        // [cap_rows, h]
    int *err;
};

struct FinalArgs {
    const uint16_t *partial;  // [n_rows, h]
    int64_t n_rows;
    int h, T, R;
    const int32_t *rank_off, *pos_in_rank;
    uint16_t *out;
    int *err;
};

hipError_t launch_combine_partial(const PartialArgs &a, hipStream_t stream);
hipError_t launch_combine_final(const FinalArgs &a, hipStream_t stream);

}  // namespace epx
