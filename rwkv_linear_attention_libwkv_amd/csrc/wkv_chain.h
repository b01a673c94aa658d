// Plumbing of the single-pass chained scans (forward over time in the forward kernel,
// backward over time in the gradient kernel) for gfx950: tagged record words, the
// bounded waits, the search for the nearest inclusive record and the launch
// bookkeeping kept in the workspace's control block.
//
// Records.  Every tile publishes, per channel, the aggregate of the tile alone and then
// the inclusive value (everything from the scan's start up to and including the tile),
// each component as its own 64-bit word (value | tag << 32) with tag = (epoch << 2) |
// kind.  The epoch changes at every launch, so a word belongs to this launch exactly when
// its tag matches.  Words are written and read with device-scope atomics (single-copy
// atomic at 64 bits), so a reader never accepts a torn or stale value and needs no fence.
// A per-tile status word (the strongest kind published) lets a look-back inspect 64
// consecutive chunks of a group in one read; it is only a hint: every record word that
// is consumed is re-validated by its own tag.
//
// Launch bookkeeping.  Tiles take tickets from a counter, so every tile a tile waits on
// has already started; every workgroup counts itself done at its end, and the last one
// resets both counters and advances the epoch for the next launch (every other
// workgroup has read the epoch and taken its ticket by then).
//
// Giving up.  Every wait is bounded.  A tile whose wait gives up does not use a guessed
// state: it rebuilds the state it needs from what is certain without waiting (the
// nearest complete inclusive record, the complete aggregate records after it, and, for
// a tile whose record is missing, that tile's inputs read again from memory), so its
// results stay correct; the give-up word is raised as a diagnostic, and once it is up
// every other wait of the launch gives up at its next check.  The host can force this
// path for a number of launches (kCtrlForce) to test it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wkv_kernels.h"

namespace wkv {

constexpr uint32_t kKindAgg = 1u;
constexpr uint32_t kKindIncl = 2u;
constexpr uint32_t kMaxSpins = 1u << 18;
constexpr int kPollSleep = 2;  // s_sleep between polls (units of 64 clocks)

__device__ __forceinline__ void st_word(uint64_t* p, float v, uint32_t tag) {
    __hip_atomic_store(p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_word(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t word_tag(uint64_t w) { return (uint32_t)(w >> 32); }
__device__ __forceinline__ float word_val(uint64_t w) { return __uint_as_float((uint32_t)w); }

// Raise this launch's give-up word (once per wave) and report failure.
__device__ __forceinline__ bool raise_give_up(uint32_t* ctrl, uint32_t give_up_word, int lane) {
    if (lane == 0)
        __hip_atomic_store(&ctrl[kCtrlGiveUp], give_up_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return false;
}

// A wait stops after kMaxSpins polls, or once another tile of the launch gave up (checked
// before the first sleep and every 32 polls after it).
__device__ __forceinline__ bool must_stop(const uint32_t* ctrl, uint32_t give_up_word, uint32_t spin) {
    if (spin >= kMaxSpins) return true;
    return (spin & 31u) == 0u &&
           __hip_atomic_load(&ctrl[kCtrlGiveUp], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == give_up_word;
}

// Whether this launch runs every tile on the give-up path from the start (the host asked
// for it, or the tile's ticket showed the control block was not zero-filled).
__device__ __forceinline__ bool launch_forced(const uint32_t* ctrl) {
    return __builtin_amdgcn_readfirstlane(
               __hip_atomic_load(&ctrl[kCtrlForce], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) != 0u;
}

constexpr int kWindowWait = -1;      // no usable inclusive record in the window yet
constexpr int kWindowAllReady = -2;  // 64 aggregates and no inclusive record: look further

// One look at a window of 64 status words, lane l holding st, the status of chunk
// nearest + DIR * l (in_range: that chunk exists; avail: chunks of the window that exist).
// Returns the nearest chunk whose inclusive record is published while every chunk
// between it and the window's start has published at least its aggregate, or
// kWindowAllReady / kWindowWait.
template <int DIR>
__device__ __forceinline__ int scan_window(uint32_t st, bool in_range, int nearest, int avail, uint32_t tag_agg,
                                           uint32_t tag_incl) {
    const bool is_incl = in_range && st == tag_incl;
    const bool is_ready = is_incl || (in_range && st == tag_agg);
    const uint64_t incl = __ballot(is_incl);
    const uint64_t ready = __ballot(is_ready);
    if (incl) {
        const int d = __builtin_ctzll(incl);
        const uint64_t need = (d >= 63) ? ~0ull : ((2ull << d) - 1ull);
        return (ready & need) == need ? nearest + DIR * d : kWindowWait;
    }
    return (avail >= 64 && ready == ~0ull) ? kWindowAllReady : kWindowWait;
}

__device__ __forceinline__ uint32_t ld_status(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The nearest chunk, going from ci in direction DIR (-1: towards chunk 0, +1: towards
// chunk n_chunks - 1), whose inclusive record is published while every chunk between it
// and ci has published at least its aggregate.  Lane l inspects the status word of the
// l-th chunk of a window of 64; a window of 64 aggregates moves the search on by 64.
// Returns -1 after giving up (the give-up word raised).  status: this group's words.
template <int DIR>
__device__ __forceinline__ int find_inclusive(const uint32_t* status, int n_chunks, int ci, int lane,
                                              uint32_t tag_agg, uint32_t tag_incl, uint32_t* ctrl,
                                              uint32_t give_up_word) {
    int nearest = ci + DIR;  // chunk inspected by lane 0 in the current window
    for (;;) {
        const int pc = nearest + DIR * lane;
        const bool in_range = DIR < 0 ? pc >= 0 : pc < n_chunks;
        const int avail = DIR < 0 ? nearest + 1 : n_chunks - nearest;
        for (uint32_t spin = 0;; ++spin) {
            const uint32_t st = in_range ? ld_status(&status[pc]) : 0u;
            const int found = scan_window<DIR>(st, in_range, nearest, avail, tag_agg, tag_incl);
            if (found >= 0) return found;
            if (found == kWindowAllReady) break;
            if (must_stop(ctrl, give_up_word, spin)) {
                raise_give_up(ctrl, give_up_word, lane);
                return -1;
            }
            __builtin_amdgcn_s_sleep(kPollSleep);
        }
        nearest += 64 * DIR;
    }
}

// A ticket past the launch's tiles only comes from a ticket counter that was not zero
// before the launch (a workspace never zero-filled, or two launches sharing one at once).
// The n tickets of the launch are then still n consecutive numbers, so ticket mod n gives
// every tile to exactly one workgroup; such a workgroup runs its tile on the give-up path
// (nothing it could wait for is sure to exist) and flags the call with the mark a launch
// that gave up leaves, one epoch behind the counter, which the workspace query reports.
// Call with a wave-uniform ticket; every thread of the workgroup gets the same answer.
__device__ __forceinline__ void flag_stale_ticket(uint32_t* ctrl) {
    if (threadIdx.x == 0) {
        const uint32_t epoch = __hip_atomic_load(&ctrl[kCtrlEpoch], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&ctrl[kCtrlGiveUp], ((epoch - 1u) & kCtrlEpochMask) | kCtrlGiveUpMark, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
}
__device__ __forceinline__ uint32_t remap_ticket(uint32_t ticket, uint32_t n_tiles, uint32_t* ctrl, bool& forced) {
    if (ticket < n_tiles) return ticket;
    forced = true;
    flag_stale_ticket(ctrl);
    return ticket % n_tiles;
}

// End of a workgroup (one thread): count it done; the last one prepares the next launch.
// With `inherit`, a give-up of the launch before this one (the previous epoch) is carried
// over to this launch, so that the workspace reports it after a pair of dependent launches.
__device__ __forceinline__ void finish_tile(uint32_t* ctrl, uint32_t n_tiles, uint32_t epoch, bool inherit) {
    const uint32_t done = atomicAdd(&ctrl[kCtrlDone], 1u);
    if (done + 1u != n_tiles) return;
    const uint32_t force = __hip_atomic_load(&ctrl[kCtrlForce], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (force != 0u) __hip_atomic_store(&ctrl[kCtrlForce], force - 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (inherit) {
        const uint32_t prev = ((epoch - 1u) & kCtrlEpochMask) | kCtrlGiveUpMark;
        if (__hip_atomic_load(&ctrl[kCtrlGiveUp], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == prev)
            __hip_atomic_store(&ctrl[kCtrlGiveUp], epoch | kCtrlGiveUpMark, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    __hip_atomic_store(&ctrl[kCtrlTicket], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&ctrl[kCtrlDone], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&ctrl[kCtrlEpoch], (epoch + 1u) & kCtrlEpochMask, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace wkv
