// epx_device.h -- device-side helpers shared by the libepx kernels (gfx950).
//
// bf16 is the top half of an fp32 pattern; f32_to_bf16 rounds to nearest
// even, written from that definition. (FP8 codes come from gfx950's OCP
// E4M3FN convert instruction, see dispatch.hip.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "epx.h"
#include "epx_internal.h"

namespace epx {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// fp32 -> bf16 bits, nearest even. Adding 0x7FFF plus the lowest kept bit
// carries into the kept half exactly when the dropped half is above the
// midpoint, or at it with an odd kept half. NaN -> canonical 0x7FC0.
__device__ __forceinline__ uint32_t f32_to_bf16(float v)
{
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// floor(e / L) for 0 <= e < 512, with m = div_magic(L) (epx_internal.h): a
// multiply and shift in place of a 25-instruction division sequence.
__device__ __forceinline__ int div_by_magic(int e, uint32_t m)
{
    return (int)(((uint32_t)e * m) >> 20);
}

__device__ __forceinline__ void flag_error(int *err, int bits)
{
    atomicOr(err, bits);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ uint64_t lanes_below(int lane)
{
    return lane == 0 ? 0ull : (~0ull >> (kWave - lane));
}

__device__ __forceinline__ u32x4 load16(const void *p)
{
    return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ u32x4 load16_stream(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// Loads of a row of `bytes` bytes (a multiple of 16) through a raw buffer
// descriptor built from the row base: a 16-byte load at an offset at or past
// the end returns zeros without touching memory, so the loads of a row need
// no branches, and with none the compiler counts them exactly when it places
// its waits (a guarded load per vector made it wait for the whole row before
// the first use of anything loaded earlier). Nontemporal hint.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 load16_row(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2 /* nt */);
}

__device__ __forceinline__ void store16_stream(void *p, u32x4 v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

// Row stores of the dispatch kernels: 16 bytes at byte offset off (per
// lane) of a row whose base is the same for the whole wave. Policy WT: the
// sc1 cache-policy bit (device-coherent write-through), through a buffer
// store on a descriptor built from the row base, so the compiler knows it
// for a store (an inline-assembly store made it wait for every earlier
// memory operation before each one: one store in flight per wave, 5x slower
// when few tokens are dispatched). Policy NT: the nontemporal hint, 4-5%
// faster for the FP8 scatter's 7 KB rows and 256-byte scale rows. Both are
// vector-memory stores; nothing in the kernel reads the data back, and the
// kernel's end makes it visible to later work.
enum class StorePolicy { WT, NT };

template <StorePolicy POL>
__device__ __forceinline__ void store16_row(void *row, uint32_t off, u32x4 v)
{
    if constexpr (POL == StorePolicy::NT) {
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(static_cast<char *>(row) + off));
    } else {
        // raw buffer: stride 0, the largest record count, 32-bit data format
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc(row, 0, 0x7FFFFFF0, 0x00020000);
        __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 16 /* sc1 */);
    }
}

// Inclusive sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_sum(int v)
{
    const int lane = lane_id();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int o = __shfl_up(v, d, kWave);
        if (lane >= d)
            v += o;
    }
    return v;
}

// A 64-bit value every lane holds alike, moved to scalar registers. The
// builtin returns a signed int: each half goes through uint32_t so the low
// half is zero-extended, never sign-extended into the high half.
__device__ __forceinline__ uint64_t uniform64(uint64_t v)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | (uint64_t)lo;
}

__device__ __forceinline__ uint64_t wave_or(uint64_t v)
{
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1)
        v |= __shfl_xor(v, d, kWave);
    return v;
}

}  // namespace epx
