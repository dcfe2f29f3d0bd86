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
//   * the request for the next tile is issued while the current tile is being
//     computed -- once its last ring stage is in LDS -- and its result is read
//     only when the tile's k loop is done (the kernels that load the next
//     tile during the epilogue) or while the accumulators are staged (the
//     others), so the atomic's round trip hides behind the last k-tile
//     (section "Overlapping the request with the current computation"; issued
//     at the tile's first k-tile instead, the round trip held up that tile's
//     load waits, since vmcnt counts in issue order);
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
// records the final claim total, zeroes the counters and counts the run.
// A run therefore needs no host-side reset and no memset node.
//
// MI355X-specific variant (per-XCD claiming): the eight XCDs have separate
// L2 caches, and one shared counter hands consecutive tiles to workers on
// different XCDs, so no L2 sees its neighbours' A and B panels. Instead each
// XCD owns a counter over the logical indices x, x+8, x+16, ... -- the tiles
// the static schedule deals to that XCD's workers, round by round, in compact
// blocks -- and its workers claim them in that order; once they are used up a
// worker claims from the other XCDs' sequences in turn (work stealing across
// XCDs); its loop ends only when every sequence is used up. Every position is
// still handed out exactly once.
//
// Non-persistent comparison point: one workgroup per tile (grid = T), which
// the hardware dispatches as compute units free up; each workgroup runs one
// tile and exits ("Schedules", section "Scheduling Shapes": the one-tile-per-
// CTA shape the persistent loop replaces).
#pragma once

#include "common.h"

namespace pts {

enum : int { SCHED_STATIC = 0, SCHED_DYNAMIC = 1, SCHED_DYNAMIC_XCD = 2, SCHED_NONPERSISTENT = 3 };

constexpr int NUM_XCD = 8;           // chiplets (XCDs) of an MI355X, each with its own L2
// Counter words. Counters that are hit at the same time sit in separate 4 KiB
// blocks, so their atomics are spread over memory channels instead of queueing
// at one.
constexpr int CTR_CLAIM = 0;         // single device-wide claim counter
constexpr int CTR_EXIT = 32;         // workers that have made their final claim
constexpr int CTR_FINAL = 64;        // total claims of the last dynamic run
constexpr int CTR_RUNS = 65;         // dynamic runs completed
constexpr int CTR_SYNC_STALLS = 66;  // stage-flag waits that ran out (0 unless the hand-off is broken)
constexpr int CTR_GATE = 96;         // scheduler probe: workers finished (late-worker gate)
constexpr int CTR_XCD_STRIDE = 1024; // per-XCD claim counter x at CTR_XCD_STRIDE * (x + 1)
constexpr int CTR_WORDS = CTR_XCD_STRIDE * (NUM_XCD + 1);

__host__ __device__ constexpr int ctr_xcd(int x) { return CTR_XCD_STRIDE * (x + 1); }

// Tiles are numbered along a locality-friendly order ("positions", see
// tile_position below); a scheduler hands out positions. Split [0, n) into
// `parts` contiguous nearly equal ranges; part p starts at part_begin(p).
__device__ __forceinline__ int part_begin(int n, int parts, int p)
{
    const int q = n / parts, rem = n % parts;
    return p * q + min(p, rem);
}

// Static grid-stride deals worker w the logical tiles w, w+P, w+2P, ...
// Workgroups are dispatched to the XCDs round-robin, so in every round of P
// logical tiles the workers of XCD x hold the logical tiles = x (mod 8).
// This bijection of each round onto itself gives those workers consecutive
// positions, i.e. one compact block of the output per XCD and round, whose
// A and B panels that XCD's L2 then shares. It only permutes which tile a
// logical index denotes; every position is still used exactly once. (The
// non-persistent schedule uses the same dealing with P = the number of
// workgroups resident at once.)
__device__ __forceinline__ int static_position(int t, int num_tiles, int round)
{
    const int num_workers = round;
    const int base = (t / num_workers) * num_workers;
    const int r = min(num_workers, num_tiles - base);
    const int u = t - base;
    return base + part_begin(r, NUM_XCD, u % NUM_XCD) + u / NUM_XCD;
}



// A worker's tile sequence. `claim` is the scheduler's own value (the
// logical index for static, the counter value for dynamic) and `pos` the
// tile position it denotes; pos >= num_tiles means there is no more work.
struct Claimed {
    int32_t claim;
    int32_t pos;
};

struct TileScheduler {
    uint32_t *counters;
    int32_t num_tiles;
    int32_t num_workers;
    int32_t round;    // static dealing width: P (static) or resident workgroups (non-persistent)
    int32_t worker;
    int32_t mode;
    int32_t *slots;   // four LDS words: two (claim, pos) pairs, alternating by tile parity
    int32_t xcd;      // this worker's XCD (dynamic XCD mode)
    uint32_t pending; // raw counter value of the request in flight (leader lane)

    __device__ __forceinline__ uint32_t atomic_take(int idx)
    {
        return __hip_atomic_fetch_add(counters + idx, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // Issue a request (leader lane only): one atomic on the single counter,
    // or on this XCD's counter. Its value is read only in resolve().
    __device__ __forceinline__ void issue()
    {
        pending = atomic_take(mode == SCHED_DYNAMIC ? CTR_CLAIM : ctr_xcd(xcd));
    }

    // XCD x's v-th claim is the logical index x + 8v: the same tiles, in the
    // same rounds, that the static schedule deals to XCD x's workers.
    __device__ __forceinline__ bool xcd_take(int x, uint32_t v, Claimed &out) const
    {
        const uint32_t t = (uint32_t)x + (uint32_t)NUM_XCD * v;
        if (v >= 0x1000000u || t >= (uint32_t)num_tiles)
            return false;
        out = Claimed{(int32_t)(x * 0x1000000 + v), static_position((int)t, num_tiles, round)};
        return true;
    }

    // Turn the request into a tile. Called by every lane of the leader's
    // wave (lane 0 holds `pending`); every lane returns the same result.
    // Single counter: the counter value is the position. Per-XCD counters:
    // this XCD's sequence first; once it is used up, lanes 1..7 look at the
    // other seven counters at once (a counter that shows its sequence used up
    // stays so) and the leader claims from the first, in turn from this XCD,
    // that may still have work; only when none has is the request failed.
    __device__ __forceinline__ Claimed resolve(int lane)
    {
        const uint32_t own = __builtin_amdgcn_readfirstlane(pending);
        if (mode == SCHED_DYNAMIC) {
            const int32_t c = own > 0x7FFFFFFFu ? 0x7FFFFFFF : (int32_t)own;
            return Claimed{c, c};
        }
        Claimed c{0x7FFFFFFF, num_tiles};
        if (xcd_take(xcd, own, c))
            return c;
        const int peek_x = (xcd + lane) % NUM_XCD;
        bool avail = false;
        if (lane >= 1 && lane < NUM_XCD) {
            const uint32_t seen =
                __hip_atomic_load(counters + ctr_xcd(peek_x), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            avail = (uint64_t)peek_x + (uint64_t)NUM_XCD * seen < (uint64_t)num_tiles;
        }
        uint64_t mask = __ballot(avail);
#pragma unroll 1
        while (mask != 0) {
            const int d = __builtin_ctzll(mask);
            mask &= mask - 1;
            const int x = (xcd + d) % NUM_XCD;
            uint32_t v = 0;
            if (lane == 0)
                v = atomic_take(ctr_xcd(x));
            if (xcd_take(x, __builtin_amdgcn_readfirstlane(v), c))
                return c;
        }
        return Claimed{0x7FFFFFFF, num_tiles};
    }

    // Resolve in the leader's wave, write the result to LDS slot `slot`
    // (lane 0), barrier, read it in every thread.
    __device__ __forceinline__ Claimed publish_and_read(int tid, int slot)
    {
        if (tid < 64) {
            const Claimed c = resolve(tid);
            if (tid == 0) {
                slots[2 * slot] = c.claim;
                slots[2 * slot + 1] = c.pos;
            }
        }
        barrier_lds();
        return Claimed{uniform(slots[2 * slot]), uniform(slots[2 * slot + 1])};
    }

    // First tile of this worker; all threads of the workgroup call it (thread
    // 0 is the leader).
    __device__ __forceinline__ Claimed first(int tid)
    {
        if (mode == SCHED_STATIC || mode == SCHED_NONPERSISTENT) {
            const int32_t t = worker;
            return Claimed{t, t < num_tiles ? static_position(t, num_tiles, round) : num_tiles};
        }
        if (tid == 0)
            issue();
        return publish_and_read(tid, 0);
    }

    // Issue the request for the tile after the current one (leader only).
    __device__ __forceinline__ bool claims() const { return mode == SCHED_DYNAMIC || mode == SCHED_DYNAMIC_XCD; }

    __device__ __forceinline__ void claim_ahead(bool leader)
    {
        if (claims() && leader)
            issue();
    }

    // The tile after `current` (all threads). For dynamic modes the pending
    // claim is resolved and published through LDS, which includes a barrier.
    // `seq` is the current tile's position in this worker's sequence.
    __device__ __forceinline__ Claimed next(Claimed current, int tid, int seq)
    {
        if (!claims())
            return next_computed(current);
        return publish_and_read(tid, (seq + 1) & 1);
    }

    // The same in two halves, for a caller that already has barriers to use:
    // stage_next (all threads; dynamic modes resolve the pending claim in the
    // leader's wave and write it to LDS), then, after at least one LDS
    // barrier, read_next (all).
    __device__ __forceinline__ void stage_next(int tid, int seq)
    {
        if (claims() && tid < 64) {
            const Claimed c = resolve(tid);
            if (tid == 0) {
                const int slot = (seq + 1) & 1;
                slots[2 * slot] = c.claim;
                slots[2 * slot + 1] = c.pos;
            }
        }
    }

    __device__ __forceinline__ Claimed read_next(Claimed current, int seq)
    {
        if (!claims())
            return next_computed(current);
        const int slot = (seq + 1) & 1;
        return Claimed{uniform(slots[2 * slot]), uniform(slots[2 * slot + 1])};
    }

    __device__ __forceinline__ Claimed next_computed(Claimed current) const
    {
        if (mode == SCHED_STATIC) {
            const int32_t t = current.claim + num_workers;
            return Claimed{t, t < num_tiles ? static_position(t, num_tiles, round) : num_tiles};
        }
        return Claimed{0x7FFFFFFF, num_tiles}; // non-persistent: one tile per workgroup
    }

    // End-of-kernel bookkeeping (leader only; after the worker's failed claim).
    // Relaxed ordering suffices: every claim of this worker has returned (its
    // value was read) before the exit increment is issued, so all claims of
    // all workers are performed before the last exit increment, and the
    // reset after it; device-scope atomics are performed at one coherent
    // point. The next launch on the stream sees the reset at the kernel
    // boundary. (Acquire/release here would add cache write-backs at exit.)
    __device__ __forceinline__ void finish(bool leader)
    {
        if (!claims() || !leader)
            return;
        uint32_t old = __hip_atomic_fetch_add(counters + CTR_EXIT, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (old == (uint32_t)num_workers - 1u) {
            uint32_t total = __hip_atomic_exchange(counters + CTR_CLAIM, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int x = 0; x < NUM_XCD; ++x)
                total += __hip_atomic_exchange(counters + ctr_xcd(x), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(counters + CTR_FINAL, total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_add(counters + CTR_RUNS, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(counters + CTR_EXIT, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
};

} // namespace pts
