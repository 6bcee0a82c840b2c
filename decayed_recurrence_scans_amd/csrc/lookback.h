// lookback.h -- the cross-workgroup exchange used by the time-segmented kernels.
//
// A workgroup that owns a later time segment waits for the aggregates that the
// workgroups of the earlier segments publish.  Virtual ids run earlier segments
// first.  The WKV and EMA chained kernels take them from an atomic ticket in
// start order, so every wait is on a workgroup that is already running; the
// linear-attention kernel uses the workgroup id (no atomic before its first
// load) and, where a wait runs out, computes the missing aggregate itself.
// Data go through device-coherent (sc1) stores and loads; the producer waits
// for its stores to complete before it stores the flag, so no cache write-back
// or invalidation is needed.  Waits are bounded and what runs out is counted in
// the workspace.
//
// Workspace counters (the first 256 bytes, zero before the first use): [0] next
// ticket, [1] finished workgroups, [2] epoch, [3] waits that ran out.  The last
// workgroup of a launch re-arms [0] and [1] and advances the epoch, so flags
// written by earlier launches never match.
#pragma once

#include "common.h"

namespace drs {

// A segment flag: low word (epoch << 4) | (tag << 2) | state, high word its
// complement, so that bytes left in the workspace by an earlier call never read as
// a valid flag.  The tag names the counter set whose epoch the writer took (one
// launch may run several problems, each with its own counters in the workspace's
// first 256 bytes): a flag left by a call on another counter set, whose epoch may
// have the same value, does not match either.
__device__ __forceinline__ unsigned long long flag_word(unsigned epoch, unsigned state, unsigned tag = 0u) {
    const unsigned lo = ((epoch & 0x0fffffffu) << 4) | ((tag & 3u) << 2) | state;
    return (unsigned long long)lo | ((unsigned long long)(~lo) << 32);
}
__device__ __forceinline__ unsigned flag_state(unsigned long long f, unsigned epoch, unsigned tag = 0u) {
    const unsigned lo = (unsigned)f, hi = (unsigned)(f >> 32);
    if (hi != ~lo || (lo >> 2) != (((epoch & 0x0fffffffu) << 2) | (tag & 3u))) return 0u;
    return lo & 3u;
}
// Flag states: the segment's aggregate is published; then (only when the final
// state overwrites the initial state in place) the segment has also finished
// reading the initial state.
constexpr unsigned kAgg = 1u, kFolded = 2u;

// device-coherent (sc1) 8-byte store / load of two floats
__device__ __forceinline__ void coherent_store2(float *p, float a, float b) {
    const unsigned long long v = (unsigned long long)__float_as_uint(a) |
                                 ((unsigned long long)__float_as_uint(b) << 32);
    __hip_atomic_store(reinterpret_cast<unsigned long long *>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coherent_load2(const float *p, float &a, float &b) {
    const unsigned long long v = __hip_atomic_load(reinterpret_cast<const unsigned long long *>(p),
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    a = __uint_as_float((unsigned)v);
    b = __uint_as_float((unsigned)(v >> 32));
}
// Every earlier store of this wave has completed (for sc1 stores: is visible
// device-wide) before any later memory operation is issued.
__device__ __forceinline__ void wait_stores_complete() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}


}  // namespace drs
