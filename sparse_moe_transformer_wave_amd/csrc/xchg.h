// xchg.h -- launch tags and exchange words of the persistent launches (kPersistentGrid
// workgroups, one per CU): the single-token and dense single-token layers (decode1.hip) and
// the small-batch layer (decode_few.hip).
//
// Workgroups of one launch trade data through 64-bit words {launch tag, payload} written
// with agent-scope stores and read with agent-scope loads: one aligned 64-bit access carries
// the payload and its readiness together, so there are no grid barriers, fences or
// cache-wide write-backs.  The tag comes from the workspace head's launch counters (one per
// workgroup index, see common.h): a word left by an earlier launch carries an older tag and
// never matches.  Every wait is bounded.
#pragma once

#include "common.h"

namespace flint {

constexpr int kSpin = 1 << 16;  // bounded waits (each try is a ~1 us round trip)

// This workgroup's launch counter (one thread reads it; the caller broadcasts the tag and
// writes the counter back plus one with bump_launches).
__device__ __forceinline__ uint32_t read_launches(uint8_t *head)
{
    return __hip_atomic_load(reinterpret_cast<uint32_t *>(head + kHeadCounters) + blockIdx.x, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void bump_launches(uint8_t *head, uint32_t launches)
{
    __hip_atomic_store(reinterpret_cast<uint32_t *>(head + kHeadCounters) + blockIdx.x, launches + 1u,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t diag_word(const uint8_t *head)
{
    return __hip_atomic_load(reinterpret_cast<uint32_t *>(const_cast<uint8_t *>(head) + kHeadDiag),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void put_word(uint64_t *p, uint32_t tag, float v)
{
    __hip_atomic_store(p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// h of two slots at one row of I: bf16(lo) in bits 0-15, bf16(hi) in bits 16-31.
__device__ __forceinline__ void put_h2(uint64_t *p, uint32_t tag, float lo, float hi)
{
    __hip_atomic_store(p, ((uint64_t)tag << 32) | f2bf(lo) | (f2bf(hi) << 16), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t get_word(const uint64_t *p)
{
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until the words w[q] (q < nq, read from p + stride * q) all carry `tag`.  The
// missing ones are re-read together, so each try costs one round trip however many are
// late.  Bounded: on timeout (at once when `giveup`, the head's diagnostic switch) the error
// flag is set and the stale values are kept.
template <int N>
__device__ __forceinline__ void await_words(const uint64_t *p, int stride, int nq, uint64_t *w, uint32_t tag,
                                            uint8_t *head, bool giveup)
{
    for (int n = 0;; n++) {
        bool miss = false;
#pragma unroll
        for (int q = 0; q < N; q++) miss |= q < nq && (uint32_t)(w[q] >> 32) != tag;
        if (!miss) break;
        if (giveup || n >= kSpin) {
            __hip_atomic_fetch_or(reinterpret_cast<uint32_t *>(head + kHeadError), kWsWaitTimeout, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int q = 0; q < N; q++)
            if (q < nq && (uint32_t)(w[q] >> 32) != tag) w[q] = get_word(p + (size_t)stride * q);
    }
}

// True when every one of a persistent launch's kPersistentGrid workgroups can be resident at
// once: a device with at least that many CUs and room on a CU for one workgroup of `kernel`
// with `threads` threads and `dyn` bytes of dynamic LDS (decode1.hip; cached per device).
bool persistent_fits(const void *kernel, int threads, size_t dyn);

}  // namespace flint
