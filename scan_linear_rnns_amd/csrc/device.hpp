// device.hpp -- device-side building blocks shared by the scan kernels (gfx950).
//
//  * tagged words: a 64-bit word holding (32-bit call tag, 32-bit payload).
//    Tiles publish their chunk aggregates and inclusive prefixes as tagged
//    words written and read with relaxed agent-scope atomics; a reader
//    accepts a word only when its tag equals the current call's tag, so no
//    flag/payload ordering (and no L2 writeback or invalidate fence) is
//    needed, and the workspace never has to be cleared between calls.
//  * tile tickets: workgroups take tile indices from an atomic counter in
//    dispatch order, so a tile only ever waits on tiles whose workgroups
//    started before it (the single-pass decoupled look-back of Merrill and
//    Garland needs this for forward progress).  The workgroup that takes the
//    last ticket resets the counter for the next call.
//  * bounded waits: every cross-workgroup wait gives up after kSpinLimit
//    polls and raises bit 0 of the workspace error word instead of hanging.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mgs {

constexpr uint32_t kErrSpin = 1u;         // a look-back wait hit its spin limit
constexpr uint32_t kErrTicket = 2u;       // a ticket counter was not reset (workspace not zeroed)
constexpr uint32_t kSpinLimit = 1u << 20; // polls (each a memory round trip plus a short sleep)

// Workspace header (first 256 bytes of every workspace).
struct WsHeader {
    uint32_t ticket_fwd;
    uint32_t ticket_bwd;
    uint32_t err;
    uint32_t pad[61];
};
static_assert(sizeof(WsHeader) == 256, "header size");

__device__ __forceinline__ uint64_t tagged_load(const uint64_t *p)
{
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void tagged_store(uint64_t *p, uint32_t tag, float v)
{
    const uint64_t w = (static_cast<uint64_t>(tag) << 32) | static_cast<uint64_t>(__float_as_uint(v));
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool tag_is(uint64_t w, uint32_t tag)
{
    return static_cast<uint32_t>(w >> 32) == tag;
}

__device__ __forceinline__ float tag_value(uint64_t w)
{
    return __uint_as_float(static_cast<uint32_t>(w));
}

__device__ __forceinline__ void raise_error(uint32_t *err, uint32_t bits)
{
    __hip_atomic_fetch_or(err, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Block-wide: returns this workgroup's tile index (0 .. n_tiles-1), taken in
// dispatch order from *ctr.  `slot` is a __shared__ word.
__device__ __forceinline__ uint32_t take_ticket(uint32_t *ctr, uint32_t n_tiles, uint32_t *err,
                                                uint32_t *slot)
{
    if (threadIdx.x == 0) {
        uint32_t t = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (t == n_tiles - 1)
            __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (t >= n_tiles) {
            raise_error(err, kErrTicket);
            t %= n_tiles;
        }
        *slot = t;
    }
    __syncthreads();
    return *slot;
}

// Polls a tagged word until it carries `tag` or the spin limit is reached.
// Returns true when the word is ready.
__device__ __forceinline__ bool poll(const uint64_t *p, uint32_t tag, uint64_t &w)
{
    w = tagged_load(p);
    return tag_is(w, tag);
}

__device__ __forceinline__ void backoff()
{
    __builtin_amdgcn_s_sleep(1);
}

}  // namespace mgs
