// fc_sync.h -- device helpers of the self-synchronizing transfers: wavefront-uniform verdicts on the
// scalar unit, agent-scope relaxed accesses, and sender pacing.  Internal to libfc.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fc.h"
#include "fc_launch.h"

namespace fc {

// Slot pointers of the receivers, the only table read from the argument segment (the scalars lead the
// kernels' argument lists and arrive preloaded in registers).  Entries past R repeat rank R-1.
struct LLSlots {
    const uint64_t* p[kMaxRanks];
};

// 1 if x != 0, else 0, for a wavefront-uniform x, on the scalar unit (written out because the compiler
// turns the comparison into a vector select and a read-back).  s_min_u32 also sets SCC.
__device__ __forceinline__ uint32_t s_nonzero(uint32_t x) {
    uint32_t y;
    asm("s_min_u32 %0, %1, 1" : "=s"(y) : "s"(x) : "scc");
    return y;
}

// Agent-scope relaxed atomic accesses: coherent across the per-XCD L2 caches of the chip, ordering
// nothing else.  A 64-bit one moves an epoch-tagged slot (payload and epoch word) as one unit.
__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_relaxed(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The counter group of this workgroup: the receivers' workgroups add their counts to FC_COUNTER_GROUPS
// groups 512 bytes apart (by workgroup index), so that their device-scope atomics, all issued at about
// the same time, do not queue on one address.
__device__ __forceinline__ uint32_t* counter_group(uint32_t* counters) {
    return counters + (blockIdx.x % FC_COUNTER_GROUPS) * FC_COUNTER_STRIDE;
}

// A slow sender, for runs where the receiver starts first: `pace` sleeps of 8 x 64 clocks.
__device__ __forceinline__ void pace_sleep(int pace) {
    for (int i = 0; i < pace; ++i) __builtin_amdgcn_s_sleep(8);
}

}  // namespace fc
