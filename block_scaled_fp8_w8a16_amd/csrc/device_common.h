// Device helpers shared by the W8A16 kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace w8a16 {
namespace dev {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Swizzle of the 16-byte chunk index inside a 128-byte weight row: rows
// r and r^8 differ in the low bit, so the 16 lanes of one ds_read_b128
// phase (rows 0..15, same logical chunk) hit distinct banks whether the LDS
// serves 8 or 16 lanes per cycle.
__device__ __forceinline__ uint32_t wswz(uint32_t r) { return (r & 7u) ^ (r >> 3); }

// Bytes 0,1 (HI = false) or 2,3 (HI = true) of `raw` -> two BF16 in one dword,
// the lower byte in the lower half.
template <bool HI>
__device__ __forceinline__ uint32_t bf16_pair_from_fp8(uint32_t raw)
{
    auto v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, v);
}

// 16 FP8 bytes -> two MFMA operands of 8 BF16 (bytes 0..7, bytes 8..15).
__device__ __forceinline__ void dequant16(u32x4_t raw, bf16x8_t &lo, bf16x8_t &hi)
{
    u32x4_t l, h;
    l.x = bf16_pair_from_fp8<false>(raw.x);
    l.y = bf16_pair_from_fp8<true>(raw.x);
    l.z = bf16_pair_from_fp8<false>(raw.y);
    l.w = bf16_pair_from_fp8<true>(raw.y);
    h.x = bf16_pair_from_fp8<false>(raw.z);
    h.y = bf16_pair_from_fp8<true>(raw.z);
    h.z = bf16_pair_from_fp8<false>(raw.w);
    h.w = bf16_pair_from_fp8<true>(raw.w);
    lo = __builtin_bit_cast(bf16x8_t, l);
    hi = __builtin_bit_cast(bf16x8_t, h);
}

// Buffer resources.  A raw buffer load through a resource that spans
// exactly the bytes it may read returns zeros, without a memory access, for
// an offset at or past the resource's byte count.  Kernels use that for
// rows past m or n, K steps past the end and ring prefetches past a wave's
// last step: the loads need no branches, and the compiler's wait counts
// stay exact (a load under a branch makes it wait for every load in flight
// at the next use of any of them).
constexpr int kRsrcWord3 = 0x00020000;     // raw 32-bit data format, no swizzle
constexpr uint32_t kOob = 0x80000000u;     // past every resource (each < 2^31 bytes)
constexpr int kCacheNt = 2;                // nontemporal hint of a load

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const uint8_t *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}

template <bool NT>
__device__ __forceinline__ u32x4_t load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(u32x4_t,
                              __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, NT ? kCacheNt : 0));
}

__device__ __forceinline__ uint32_t load4(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

// Step offset between the K walks of consecutive tiles (odd, so tile t
// starts at step 37t mod span and neighbouring tiles are far apart).
constexpr uint32_t kRotStride = 37;

// Round-to-nearest-even FP32 -> BF16 bits (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    __bf16 b = static_cast<__bf16>(f);
    return (uint32_t)__builtin_bit_cast(uint16_t, b);
}

// Map the hardware workgroup id to a logical id so that logical ids that
// are close (the K splits of one tile, then neighbouring tiles) run on the
// same XCD: workgroups are dispatched round-robin over the 8 XCDs.
__device__ __forceinline__ uint32_t logical_wg(uint32_t bid, uint32_t grid)
{
    const uint32_t X = 8;
    const uint32_t q = grid / X, r = grid % X;
    const uint32_t xcd = bid % X, slot = bid / X;
    return xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// 16-byte store at agent scope: two 8-byte agent-scope atomic stores, which
// gfx950 issues with the sc1 bit, writing through this XCD's L2 so that a
// CU on any XCD can read the data once the store has completed (s_waitcnt
// vmcnt(0)).  Unlike a release fence, nothing else in the L2 is written back.
__device__ __forceinline__ void store_agent(f32x4_t *p, f32x4_t v)
{
    uint64_t *q = reinterpret_cast<uint64_t *>(p);
    // bit-cast the whole vector: clang reads element 0 for a bit_cast of a
    // single vector element (v.y)
    const u32x4_t u = __builtin_bit_cast(u32x4_t, v);
    const uint64_t lo = (uint64_t)u.x | ((uint64_t)u.y << 32);
    const uint64_t hi = (uint64_t)u.z | ((uint64_t)u.w << 32);
    __hip_atomic_store(q, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16-byte load at agent scope (two 8-byte agent-scope atomic loads, sc1):
// misses this CU's L1, so it sees what store_agent() wrote on any XCD.
__device__ __forceinline__ f32x4_t load_agent(const f32x4_t *p)
{
    const uint64_t *q = reinterpret_cast<const uint64_t *>(p);
    const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    f32x4_t v;
    v.x = __builtin_bit_cast(float, (uint32_t)lo);
    v.y = __builtin_bit_cast(float, (uint32_t)(lo >> 32));
    v.z = __builtin_bit_cast(float, (uint32_t)hi);
    v.w = __builtin_bit_cast(float, (uint32_t)(hi >> 32));
    return v;
}

// Cache-policy operand of the global_load_lds builtin for the non-temporal
// hint (the `nt` bit on gfx950).
constexpr int kNonTemporal = 2;

// LDS pointer type of the global_load_lds builtin (LDS DMA).
typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt vmcnt(N) with lgkmcnt and expcnt left alone.  The memory clobber
// keeps LDS reads of the DMA'd data from moving above the wait.
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that does not drain outstanding global loads (the
// ordinary __syncthreads() waits for every in-flight DMA step): it waits only
// for this wave's LDS reads, so no wave can refill a buffer another wave is
// still reading.  The DMA data of a step is covered by wait_vm() before it.
__device__ __forceinline__ void barrier_lds()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Store four adjacent outputs C[row][col..col+3] (FP32 -> BF16).
__device__ __forceinline__ void store_c4(const GemmArgs &g, f32x4_t v, uint32_t row,
                                         uint32_t col)
{
    if (row >= g.m || col >= g.n)
        return;
    uint16_t *dst = reinterpret_cast<uint16_t *>(g.c) + (size_t)row * g.c_stride + col;
    uint32_t b0 = f32_to_bf16_bits(v.x), b1 = f32_to_bf16_bits(v.y);
    uint32_t b2 = f32_to_bf16_bits(v.z), b3 = f32_to_bf16_bits(v.w);
    if (col + 3 < g.n && (reinterpret_cast<uintptr_t>(dst) & 7u) == 0) {
        u32x2_t packed;
        packed.x = b0 | (b1 << 16);
        packed.y = b2 | (b3 << 16);
        *reinterpret_cast<u32x2_t *>(dst) = packed;
    } else {
        dst[0] = (uint16_t)b0;
        if (col + 1 < g.n) dst[1] = (uint16_t)b1;
        if (col + 2 < g.n) dst[2] = (uint16_t)b2;
        if (col + 3 < g.n) dst[3] = (uint16_t)b3;
    }
}

}  // namespace dev
}  // namespace w8a16
