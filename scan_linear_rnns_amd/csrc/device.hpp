// device.hpp -- device-side building blocks shared by the scan kernels (gfx950).
//
//  * tagged words: a 64-bit word holding (32-bit call tag, 32-bit payload).
//    Tiles publish their chunk aggregates and inclusive prefixes as tagged
//    words with relaxed atomic stores (workgroup scope when every reader runs
//    on the writer's XCD, else agent scope; see tagged_store) and read them
//    with relaxed agent-scope atomic loads; a reader accepts a word only when
//    its tag equals the current call's tag, so no flag/payload ordering (and
//    no L2 writeback or invalidate fence) is needed, and the workspace never
//    has to be cleared between calls.
//  * launch epochs: every multi-tile launch draws its tag from a per-workspace
//    epoch counter on the device (see epoch_begin), so tags never repeat
//    between launches on one workspace, replays of a captured graph included.
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
// `spin_limit` and `fail_waits` are set by the host (0 in normal use) for
// tests of the failure path: a wait gives up after spin_limit polls (0: the
// built-in kSpinLimit), and with fail_waits every wait expects kNeverTag,
// which no launch publishes, so each one runs to its limit.  They sit in a
// cache line of their own, away from the ticket that every workgroup adds to
// at kernel start.
struct WsHeader {
    unsigned long long ticket;
    uint32_t err;
    uint32_t pad0[29];
    uint32_t spin_limit;   // byte 128
    uint32_t fail_waits;
    uint32_t pad1[30];
};
static_assert(sizeof(WsHeader) == 256, "header size");
constexpr uint32_t kNeverTag = 0xFFFFFFFFu;   // launch tags are 1 .. 2^32 - 2

// Output stores.  Every output element (and every chunk state a forward saves
// for its backward) is written exactly once and never read back by the kernel
// that writes it, so the stores carry the nontemporal hint: the lines drain to
// HBM while the kernel runs instead of staying dirty in L2 until the
// write-back at the end of the kernel, which the next kernel on the stream
// waits for.  Measured on the log-space pair at B=128, T=64, d=64: 8.4 -> 7.5 us.
__device__ __forceinline__ void store_out(float *p, float v) { __builtin_nontemporal_store(v, p); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// p 8-byte aligned
__device__ __forceinline__ void store_out2(float *p, float x, float y)
{
    const f32x2 v = {x, y};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x2 *>(p));
}

// p 16-byte aligned
__device__ __forceinline__ void store_out4(float *p, float x, float y, float z, float w)
{
    const f32x4 v = {x, y, z, w};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(p));
}

// Loads of an input that the kernel reads exactly once, at unit stride across
// the lanes of a wave: the nontemporal hint keeps these lines from displacing
// others in L2.  Measured: log-space backward at B=128, T=64, d=64
// 4.1 -> 3.9 us; the block-affine pair's vector inputs (b, h, dh) at k = 8
// 16.0 -> 15.4 us (lab shape) and 40.2 -> 38.6 us (B=16, T=1024).  Not for
// loads that read a line piecewise over several instructions (the block
// kernels' matrix rows and columns), which the hint slows down.
__device__ __forceinline__ float load_once(const float *p) { return __builtin_nontemporal_load(p); }

__device__ __forceinline__ uint64_t tagged_load(const uint64_t *p)
{
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Where a tagged word's readers run.  gfx950 deals the workgroups of a launch
// to its XCDs round robin by blockIdx (the XCC_ID hardware register of every
// workgroup equals blockIdx % 8 on an MI355X, checked on the device at 128 to
// 2048 workgroups), and the XCDs' L2 caches are not coherent with one another.
// An agent-scope load returns a line that is dirty in its own XCD's L2 and
// fetches any other line from memory; an agent-scope store writes through to
// memory.  When every reader of a word runs on its writer's XCD (`local`: the
// launch's tiles of one chain group lie a multiple of the device's XCD count
// apart in blockIdx; decided on the host), a workgroup-scope store, which
// leaves the line dirty in that L2, reaches the readers' agent-scope polls
// without the trip to memory: one hop between two workgroups of one XCD takes
// ~0.27 us so against ~0.47 us with an agent-scope store (~0.62 us between
// XCDs; ping-pong of a tagged word).  In every other launch the store is
// agent-scope.  Either way the tag, not the store's scope, tells a reader
// whether the word is current.

__device__ __forceinline__ void tagged_store(uint64_t *p, uint32_t tag, float v, bool local)
{
    const uint64_t w = (static_cast<uint64_t>(tag) << 32) | static_cast<uint64_t>(__float_as_uint(v));
    if (local)
        __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    else
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

// Launch tag for the decoupled look-back.  Thread 0 of every workgroup of a
// multi-tile launch adds 1 to the workspace's (epoch << 32 | count) word; the
// workgroup that brings the count to n_tiles starts the next epoch.  All
// workgroups of one launch therefore read the same epoch, and any two
// launches on one workspace (also replays of a captured graph) read different
// ones.  The atomic is issued right after the tile's input loads
// (epoch_begin) and its result is consumed only when the workgroup first
// publishes (epoch_end).  Loads complete in issue order within a wave, so an
// atomic issued ahead of the inputs -- every workgroup's thread 0 adding to
// the same word -- holds wave 0's inputs back until it returns (block-affine
// pair 37.1 -> 34.8 us when moved behind them).  The elementwise backward,
// whose work between its loads and its first publish is too short to hide
// the round trip, still issues it at kernel start.
//
// Tiles are indexed by blockIdx and wait only on tiles with a smaller index
// (forward) or a larger one whose blockIdx is smaller (backward, which numbers
// its tiles from the end of T).  Workgroups are dispatched in blockIdx order,
// so every tile a resident workgroup waits on has already been dispatched, and
// the lowest-numbered unfinished tile can always proceed: no deadlock, with no
// need to take tile indices from a counter.
// Taken after the tile's input loads (or at kernel start): the ticket word
// before thread 0's add, and the waits' settings (spin_limit, fail_waits; one load of a
// workgroup-uniform address, so a scalar load that vector loads do not queue
// behind), both consumed only at the tile's first publish.
struct Launch {
    unsigned long long old, cfg;
};

__device__ __forceinline__ Launch epoch_begin(WsHeader *hd)
{
    Launch l{0, *reinterpret_cast<const unsigned long long *>(&hd->spin_limit)};
    if (threadIdx.x == 0)
        l.old = __hip_atomic_fetch_add(&hd->ticket, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return l;
}

// Thread 0 only: turns epoch_begin's values into the words the workgroup
// shares through LDS -- w[0] the launch tag (starting the next epoch if this
// workgroup was the last of the launch to arrive), w[1] the tag the waits
// expect, w[2] their poll limit.
__device__ __forceinline__ void epoch_end(WsHeader *hd, const Launch &l, uint32_t n_tiles, uint32_t *w)
{
    const uint32_t cnt = static_cast<uint32_t>(l.old);
    const uint32_t epoch = static_cast<uint32_t>(l.old >> 32);
    if (cnt == n_tiles - 1)
        __hip_atomic_store(&hd->ticket, static_cast<unsigned long long>(epoch + 1u) << 32, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    if (cnt >= n_tiles) raise_error(&hd->err, kErrTicket);
    const uint32_t tag = epoch % 0xFFFFFFFEu + 1u;
    const uint32_t limit = static_cast<uint32_t>(l.cfg), fail = static_cast<uint32_t>(l.cfg >> 32);
    w[0] = tag;
    w[1] = fail ? kNeverTag : tag;
    w[2] = limit ? limit : kSpinLimit;
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
