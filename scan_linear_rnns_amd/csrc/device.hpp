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
//    Garland needs this for forward progress).  The same counter word holds
//    the launch epoch, which supplies the tag.
//  * bounded waits: every cross-workgroup wait gives up after kSpinLimit
//    polls and raises bit 0 of the workspace error word instead of hanging.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mgs {

constexpr uint32_t kErrSpin = 1u;         // a look-back wait hit its spin limit
constexpr uint32_t kErrTicket = 2u;       // a ticket counter was not reset (workspace not zeroed)
constexpr uint32_t kSpinLimit = 1u << 20; // polls (each a memory round trip plus a short sleep)

// Workspace header (first 256 bytes of every workspace).  `ticket` packs
// (epoch << 32) | count: every multi-tile launch on the workspace takes its
// tile indices from `count` and its tag from `epoch`, so tags differ between
// any two launches on one workspace -- also between replays of a captured
// graph -- and never equal 0 (the value of a zero-filled workspace).
struct WsHeader {
    unsigned long long ticket;
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

struct TileTicket {
    uint32_t tile;
    uint32_t tag;
};

// Block-wide: this workgroup's tile index (0 .. n_tiles-1), taken in dispatch
// order, and the launch's tag.  `slot` is two __shared__ words.  The
// workgroup that takes the last index starts the next epoch with count 0.
__device__ __forceinline__ TileTicket take_ticket(WsHeader *hd, uint32_t n_tiles, uint32_t *slot)
{
    if (threadIdx.x == 0) {
        const unsigned long long old =
            __hip_atomic_fetch_add(&hd->ticket, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        uint32_t cnt = static_cast<uint32_t>(old);
        const uint32_t epoch = static_cast<uint32_t>(old >> 32);
        if (cnt == n_tiles - 1)
            __hip_atomic_store(&hd->ticket, static_cast<unsigned long long>(epoch + 1u) << 32,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (cnt >= n_tiles) {
            raise_error(&hd->err, kErrTicket);
            cnt %= n_tiles;
        }
        slot[0] = cnt;
        slot[1] = epoch % 0xFFFFFFFEu + 1u;
    }
    __syncthreads();
    return TileTicket{slot[0], slot[1]};
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
