// Hand-offs between the workgroups of one persistent launch (the fused MoE
// layer and the fused dense FFN).
//
// Hand-off data is written with device-scope atomic stores and read with
// device-scope atomic loads, which are coherent across the XCDs' L2 caches by
// themselves; a count follows the completion of its contributor's stores
// (vmcnt 0). Measured alternatives: device-scope release/acquire fences write
// back or invalidate whole L2 caches per wavefront (13x slower); one counter or
// flag shared by every workgroup serializes at ~10 ns per access (4x slower).
// So a count with many contributors is split over kSyncRep sub-counters on
// lines of their own, and a flag many workgroups poll is replicated on kSyncRep
// lines (words and offsets in launch.hpp).
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace w4 {

__device__ __forceinline__ void put32(void* p, uint32_t v) {
    __hip_atomic_store(reinterpret_cast<uint32_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put64(void* p, uint64_t v) {
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t get32(const void* p) {
    return __hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t get64(const void* p) {
    return __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned count(unsigned* p) {
    return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Contributors to a split count of n: contributor i counts on sub-counter
// i % kSyncRep (whose share is n / kSyncRep, one more for the first n %
// kSyncRep); the one completing a sub-counter counts on the top word, and the
// one completing that (min(n, kSyncRep) sub-counters) is told so.
__device__ inline bool split_count(unsigned* sync, int sub_base, int top, int i, int n) {
    const int r = i % kSyncRep;
    const unsigned share = n / kSyncRep + (r < n % kSyncRep ? 1 : 0);
    if (count(sync + sub_base + r * kSyncLine) != share - 1) return false;
    const unsigned subs = n < kSyncRep ? n : kSyncRep;
    return count(sync + top) == subs - 1;
}

// Workgroup-wide: thread 0 polls the workgroup's replica of a flag until it is
// >= 1, at most `limit` times (a give-up sets err_bit in the error word); the
// barrier orders the workgroup's later loads after the poll that saw it.
__device__ inline bool wg_wait_flag(unsigned* sync, long long limit, int rep_base, unsigned err_bit,
                                    int* sflag) {
    if (threadIdx.x == 0) {
        const unsigned* p = sync + rep_base + (blockIdx.x % kSyncRep) * kSyncLine;
        bool ok = false;
        for (long long n = 0;; ++n) {
            if (get32(p) >= 1u) { ok = true; break; }
            if (n >= limit) break;
            __builtin_amdgcn_s_sleep(2);
        }
        if (!ok) atomicOr(sync + kSyncErr, err_bit);
        *sflag = ok;
    }
    __syncthreads();
    const bool ok = *sflag != 0;
    __syncthreads();
    return ok;
}

// The thread index as a value the compiler cannot trace to threadIdx: every
// lane-dependent address of an item is then computed inside the item, not
// hoisted out of the persistent loop (hoisted, the invariants of every item
// kind would stay live at once and the kernel would need far more registers).
__device__ __forceinline__ int item_tid() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// Blocks of `threads` threads of one kernel that fit on a CU at once
// (occupancy API), cached per (kernel, LDS bytes, device); 0 when the kernel
// needs scratch: scratch-backed waves are rationed by the runtime in a way the
// occupancy query does not see, so residency would not be guaranteed.
int resident_per_cu(const void* kern, int threads, size_t lds, int dev);

// A persistent grid for `items` work items: min(items, resident blocks on the
// whole device), or 0 (launch nothing) when residency cannot be guaranteed.
int persistent_grid(const void* kern, int threads, size_t lds, int items, hipError_t* err);

}  // namespace w4
