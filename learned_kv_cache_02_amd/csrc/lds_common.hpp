// Helpers of the kernels that stage tiles through LDS with direct HBM -> LDS
// copies (global_load_lds): an explicit vector-memory wait and a workgroup
// barrier that adds no waits of its own.
#pragma once

#include "device_common.hpp"

namespace nectar {

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt low bits [3:0], high bits [15:14]; expcnt and lgkmcnt at their maxima).
template <int N> __device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef __attribute__((address_space(3))) void lds_void;

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Transposing LDS read (ds_read_b64_tr_b16): every lane names one 8-byte slot
// of four 16-bit elements; in each group of 16 lanes, lane 4a + b receives
// element b of the slots named by lanes a, a + 4, a + 8 and a + 12 of its
// group, in that order.  `byte_off` is a byte offset from `base`.
__device__ __forceinline__ u32x2 lds_read_tr16(const void *base, uint32_t byte_off) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4 *)((__attribute__((address_space(3))) char *)base + byte_off));
    return __builtin_bit_cast(u32x2, v);
}

// Swizzle of stages read by transposing reads (lds_read_tr16).  Piece j of row r is
// stored at position j ^ tr_swizzle(r).  A transposing read of four rows
// 4k .. 4k + 3 and four consecutive pieces 4i .. 4i + 3 (two per 16-lane group)
// then touches sixteen distinct positions, and any 16 lanes eight distinct
// positions mod 8: every bank once per 256 bytes.  (With the plain r & 15 the
// sixteen fall on four positions, a four-way bank conflict.)
__device__ __forceinline__ int tr_swizzle(int r) { return ((r & 1) * 10) ^ ((r & 2) << 1) ^ ((r >> 2) & 1); }

// Workgroup barrier that the compiler may not move memory operations across
// (the bare builtin is not a memory barrier to the optimiser) and that adds
// no waits of its own: the LDS copies are waited for explicitly above it.
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Workgroup barrier after this wave's LDS accesses have completed (its
// vector-memory loads may still be in flight).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace nectar
