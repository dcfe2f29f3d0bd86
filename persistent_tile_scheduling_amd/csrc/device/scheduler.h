// Persistent tile scheduler: where a worker's next output tile comes from.
//
// A worker is one resident workgroup that loops over output tiles. The tile
// body (loads, MFMA, epilogue) only ever sees a tile index; the scheduler is
// the single source of those indices, so static and dynamic runs share every
// other line of the kernel ("Advanced scheduling: Cluster Launch Control",
// section "When to use CLC": the mainloop and epilogue receive the current
// tile coordinate and do not know whether a formula or the hardware chose it).
//
// Static grid-stride: worker w runs tiles w, w+P, w+2P, ... ("Advanced
// scheduling: Cluster Launch Control", section "Limits of the static
// persistent scheduler"; CUTLASS Task Scheduling page "Schedules", section
// "Scheduling Shapes": the queue state is lowered to arithmetic).
//
// Dynamic claiming: MI355X has no launch queue a running workgroup can cancel
// entries from, so the claimable pool is an index range [0, T) handed out by
// one device-scope atomic counter. Mapping the pages' CLC request onto it:
//   * one lane issues the request (the pages: one thread submits try_cancel;
//     several issuers would each take a coordinate);
//   * the request for the next tile is issued before the current tile is
//     computed and its result is read only after the tile, so the atomic's
//     round trip hides behind the tile's work (section "Overlapping the
//     request with the current computation");
//   * the result reaches the other waves through an LDS slot and a barrier,
//     as the CLC response reaches the CTA through shared memory;
//   * a claim returning an index >= T is the failed request: the worker
//     finishes its current tile and leaves the loop, and never claims again
//     (section "One CLC request": after a failed request, asking again is
//     undefined, and there is no sentinel tile value).
// Every tile, the first included, comes from the counter, so a worker that
// starts late finds the pool already drained instead of owning tiles that
// wait for it (the launch tail of section "Limits of the static persistent
// scheduler"); every index is still handed out exactly once.
//
// Each worker ends on exactly one failed claim, so a run takes T + P claims.
// The counter resets itself: each worker, after its failed claim, increments
// an exit counter, and the worker that brings it to P (all claims are done)
// records the final claim value, zeroes both counters and counts the run.
// A run therefore needs no host-side reset and no memset node.
#pragma once

#include "common.h"

namespace pts {

enum : int { SCHED_STATIC = 0, SCHED_DYNAMIC = 1 };

// counters[0] claim counter, [1] exit counter, [2] final claim value of the
// last dynamic run, [3] dynamic runs completed.
struct TileScheduler {
    uint32_t *counters;
    int32_t num_tiles;
    int32_t num_workers;
    int32_t worker;
    int32_t mode;
    int32_t *slots; // two LDS words, alternating by tile sequence parity
    uint32_t pending; // claim result, held by the leader lane until published

    __device__ __forceinline__ int32_t claim()
    {
        uint32_t v = __hip_atomic_fetch_add(counters, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return v > 0x7FFFFFFFu ? 0x7FFFFFFF : (int32_t)v;
    }

    // First tile of this worker; all threads of the workgroup call it.
    __device__ __forceinline__ int32_t first(bool leader)
    {
        if (mode == SCHED_STATIC)
            return worker;
        if (leader)
            slots[0] = claim();
        barrier_lds();
        return uniform(slots[0]);
    }

    // Issue the request for the tile after the current one (leader only).
    __device__ __forceinline__ void claim_ahead(bool leader)
    {
        if (mode == SCHED_DYNAMIC && leader)
            pending = (uint32_t)claim();
    }

    // Make the pending claim visible to the workgroup. Must be followed by a
    // barrier_lds() before next() reads it. `seq` is the current tile's
    // position in this worker's sequence.
    __device__ __forceinline__ void publish(bool leader, int seq)
    {
        if (mode == SCHED_DYNAMIC && leader)
            slots[(seq + 1) & 1] = (int32_t)pending;
    }

    __device__ __forceinline__ int32_t next(int32_t current, int seq)
    {
        if (mode == SCHED_STATIC)
            return current + num_workers;
        return uniform(slots[(seq + 1) & 1]);
    }

    // End-of-kernel bookkeeping (leader only; after the worker's failed claim).
    __device__ __forceinline__ void finish(bool leader)
    {
        if (mode != SCHED_DYNAMIC || !leader)
            return;
        uint32_t old = __hip_atomic_fetch_add(counters + 1, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (old == (uint32_t)num_workers - 1u) {
            uint32_t final_claims = __hip_atomic_exchange(counters, 0u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(counters + 2, final_claims, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_add(counters + 3, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(counters + 1, 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
};

} // namespace pts
