// Epoch counters for waits between the workgroups of one launch
// ("CuTeDSL at Perplexity", grid synchronisation: workgroups of one launch
// signal each other through counters in global memory instead of ending the
// launch).
//
// A counter lives in a workspace header that is zero before the first call.
// Every call adds exactly kEpoch (2^16) to each counter it uses: one member
// adds kEpoch minus the weight of all the others, every other member its own
// positive weight.  Between calls a counter is a multiple of kEpoch, so the
// arrival that brings it to the next multiple is the last of the call, and a
// waiter is done once the counter has moved a whole epoch past the multiple
// below the value it saw on arrival -- no reset and no generation word (the
// counters wrap modulo 2^32, itself a multiple of kEpoch).
#pragma once

#include "device_utils.hpp"

namespace moe {
namespace gsync {

constexpr uint32_t kEpoch = 1u << 16;
// Polls of one wait before it gives up (each poll sleeps ~64 clocks and makes
// a device-scope load): on the order of a second.
constexpr uint32_t kSpinLimit = 1u << 22;

// Header words (uint32 index) shared by the kernels that wait.
constexpr int kWordBarrierTop = 0;      // single-launch dispatch: top barrier counter
constexpr int kWordError = 2;           // nonzero once any wait timed out (sticky)
constexpr int kWordBarrierGroup0 = 32;  // dispatch: group g's counter at 32 * (g + 1), g < 8

// Waits until every vector memory operation of the calling wave has
// completed: its stores have reached the L2.  A workgroup barrier does not
// wait for them (it waits for LDS only), so every wave whose global writes a
// later device-scope release by one thread of the workgroup must cover calls
// this before that barrier; the release then writes the whole L2 back.
// (s_waitcnt encoding on gfx9: vmcnt 0, expcnt and lgkmcnt not waited on.)
__device__ __forceinline__ void wave_stores_done() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Adds w (acquire-release, device scope); returns the value before.
__device__ __forceinline__ uint32_t arrive(uint32_t* ctr, uint32_t w) {
    return __hip_atomic_fetch_add(ctr, w, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}

// True if an arrival of weight w that saw `old` completed the epoch.
__device__ __forceinline__ bool completes(uint32_t old, uint32_t w) { return ((old + w) & (kEpoch - 1u)) == 0u; }

// The multiple of kEpoch a call started from, given a value seen before the
// call's epoch completed.
__device__ __forceinline__ uint32_t epoch_base(uint32_t seen) { return seen & ~(kEpoch - 1u); }

// Polls (relaxed: no cache invalidation per poll; the caller's fence
// acquires) until *ctr is a whole epoch past base.  After kSpinLimit polls it
// sets the error word and returns false.
__device__ inline bool wait_epoch(const uint32_t* ctr, uint32_t base, uint32_t* err_word) {
    uint32_t polls = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - base < kEpoch) {
        __builtin_amdgcn_s_sleep(1);
        if (++polls == kSpinLimit) {
            __hip_atomic_fetch_or(err_word, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
    }
    return true;
}

}  // namespace gsync
}  // namespace moe
