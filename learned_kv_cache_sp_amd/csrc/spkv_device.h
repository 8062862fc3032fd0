// Device-side helpers shared by the HIP kernels of libspkv (not by the host API).
#pragma once

#include <hip/hip_runtime.h>

namespace spkv {

// Device-scope (all XCDs) relaxed loads and stores.  Used to hand partial
// results from one workgroup to another within a launch: the producer stores
// with store_dev, waits for its stores (s_waitcnt), then bumps an arrival
// counter with a device-scope atomic; the workgroup that arrives last reads
// the partials with load_dev.  These bypass the per-XCD L2 copies, so no L2
// write-back or invalidate of the whole cache is needed.
__device__ inline void store_dev(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float load_dev(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline int arrive_dev(int *counter) {
    return __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void reset_dev(int *counter) {
    __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// arrival whose count nobody waits for here (the atomic returns nothing)
__device__ inline void arrive_nr_dev(int *counter, int n = 1) {
    (void)__hip_atomic_fetch_add(counter, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline int load_dev(const int *p) {
    return __hip_atomic_load(const_cast<int *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Poll *counter until it has reached target (compared modulo 2^32, so
// counters that only ever grow may wrap), at most `limit` times; false if it
// never did.  Only for counts that are bumped by workgroups which never wait
// for the poller, so the wait ends once they have run.
__device__ inline bool wait_reach_dev(const int *counter, int target, int limit) {
    for (int i = 0; i < limit; ++i) {
        if ((int)((unsigned)load_dev(counter) - (unsigned)target) >= 0) return true;
        __builtin_amdgcn_s_sleep(2);
    }
    return false;
}

}  // namespace spkv
