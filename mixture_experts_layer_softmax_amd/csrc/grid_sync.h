// grid_sync.h -- the grid barrier of the single-launch decode kernel (decode_fused.hip), also
// timed on its own by a probe (probe.hip).
//
// Grid barrier: block b publishes arrival by a release store of the barrier's value into its
// own word; block 0 polls every block's word, then releases a shared `go` word; the others poll
// `go`, then acquire.  Values are 4 S + i for barrier i of call S, where S is a sequence number
// in the workspace that block 0 advances at the end of each call: values only grow, so the
// words need no reset and an uninitialised workspace works from the first call.  Every spin is
// bounded: after `spin_limit` polls it counts a time-out in the workspace and goes on, so a
// grid that could not be co-resident finishes (with unspecified outputs) instead of hanging.
#pragma once

#include "device.h"
#include "launch.h"

namespace moe {
namespace {

__device__ __forceinline__ uint64_t load_agent(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void grid_barrier(GridSync* gs, uint64_t v, unsigned spin_limit) {
    __syncthreads();  // every wave's stores of this phase are in L2
    if (threadIdx.x == 0)
        __hip_atomic_store(&gs->arrive[blockIdx.x], v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    if (blockIdx.x == 0) {
        for (int b = threadIdx.x; b < int(gridDim.x); b += blockDim.x) {
            unsigned n = 0;
            while (load_agent(&gs->arrive[b]) != v) {
                if (++n > spin_limit) {
                    __hip_atomic_fetch_add(&gs->timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            __hip_atomic_store(&gs->go, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    } else if (threadIdx.x == 0) {
        unsigned n = 0;
        while (load_agent(&gs->go) != v) {
            if (++n > spin_limit) {
                __hip_atomic_fetch_add(&gs->timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
}

}  // namespace
}  // namespace moe
