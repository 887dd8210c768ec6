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

// Workgroup barrier that the compiler may not move memory operations across
// (the bare builtin is not a memory barrier to the optimiser) and that adds
// no waits of its own: the LDS copies are waited for explicitly above it.
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

}  // namespace nectar
