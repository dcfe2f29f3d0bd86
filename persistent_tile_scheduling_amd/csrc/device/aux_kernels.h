// Auxiliary kernels: the grid-stride int16 copy, the scheduler probe and the
// matrix-unit ceiling probe.
#pragma once

#include "common.h"
#include "scheduler.h"

namespace pts {

// Grid-stride copy ("Schedules" page, section "Domains": thread index
// start = block * threads + thread, stride = grid * threads; an index is
// copied only while it is below the element count). Each lane moves 16 bytes
// (8 int16) per step; the n % 8 tail elements go to the first threads.
__global__ __launch_bounds__(256) void copy_int16_kernel(const int4 *__restrict__ src, int4 *__restrict__ dst,
                                                         int64_t nvec, const int16_t *__restrict__ src16,
                                                         int16_t *__restrict__ dst16, int64_t n)
{
    const int64_t start = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = start; i < nvec; i += step)
        dst[i] = src[i];
    const int64_t tail = nvec * 8 + start;
    if (start < 8 && tail < n)
        dst16[tail] = src16[tail];
}

// Scheduler probe: the tile scheduler of the GEMM kernel with a fixed busy
// wait standing in for a tile's work. One wave per worker.
//
// out_tiles[w * max_per_worker + i]: i-th tile of worker w (the logical
// index for static and single-counter claiming, the tile position for
// per-XCD claiming); out_counts[w]: how many. gate_worker (if >= 0) first waits until every other worker has
// finished -- the late-starting worker of "Advanced scheduling: Cluster Launch
// Control", section "Limits of the static persistent scheduler". The wait
// polls at most spin_limit times; on expiry status[0] = 1 and the worker goes
// on, so the kernel always ends.
//
// counters: CTR_WORDS words laid out as in TileScheduler, with CTR_GATE
// counting the workers that have finished
// (gate), reset by the gated worker once it passes.
__global__ __launch_bounds__(64) void sched_probe_kernel(int32_t num_tiles, int32_t num_workers, int32_t mode,
                                                         int32_t gate_worker, int64_t work_ticks,
                                                         int64_t spin_limit, int32_t *out_tiles,
                                                         int32_t *out_counts, int32_t max_per_worker,
                                                         uint32_t *counters, uint32_t *status)
{
    __shared__ int32_t slots[4];
    const bool leader = threadIdx.x == 0;
    const int w = blockIdx.x;

    if (w == gate_worker) {
        int64_t polls = 0;
        while (__hip_atomic_load(counters + CTR_GATE, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) <
                   (uint32_t)(num_workers - 1) &&
               polls < spin_limit) {
            __builtin_amdgcn_s_sleep(8);
            ++polls;
        }
        if (polls >= spin_limit && leader)
            __hip_atomic_store(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (leader)
            __hip_atomic_store(counters + CTR_GATE, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    TileScheduler sched{counters, num_tiles, num_workers, num_workers, w, mode, slots,
                        (int)(xcc_id_reg() % NUM_XCD), 0u};
    Claimed cur = sched.first((int)threadIdx.x);
    int seq = 0;
    while (cur.pos < num_tiles) {
        sched.claim_ahead(leader);
        if (leader && seq < max_per_worker)
            out_tiles[(int64_t)w * max_per_worker + seq] = mode == SCHED_DYNAMIC_XCD ? cur.pos : cur.claim;
        const uint64_t t0 = realtime();
        while ((int64_t)(realtime() - t0) < work_ticks)
            __builtin_amdgcn_s_sleep(1);
        barrier_lds();
        cur = sched.next(cur, (int)threadIdx.x, seq);
        ++seq;
    }
    if (leader)
        out_counts[w] = seq;
    wait_all();
    if (leader && gate_worker >= 0 && w != gate_worker)
        __hip_atomic_fetch_add(counters + CTR_GATE, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    sched.finish(leader);
}

// Matrix-unit ceiling probe: the default GEMM kernel's matrix work without
// its memory traffic. A workgroup is 8 waves (two per SIMD, as in the GEMM);
// each wave keeps a 128x64 block of fp32 accumulators (8 x 4 blocks of 16x16)
// and per step runs the 32 v_mfma_f32_16x16x32_bf16 of one k-step. Its 24
// operand fragments (two k-steps' worth of 8 A rows and 4 B columns) are read
// once from `frags` and alternate by step parity, so operand values change
// from one MFMA to the next as in the GEMM's k loop. Inside the loop there are
// no loads, LDS accesses or stores: the rate it reaches is the matrix units'
// rate under the chip's power limit with operands of the same values.
//
// frags: 8 waves x 24 fragments x 64 lanes x 16 bytes (8 bf16), fragment f of
// wave w at [(w * 24 + f) * 64 + lane]. out[block * 512 + thread]: the sum of
// that thread's 128 accumulators. stamps[block * 2 + {0, 1}]: shader-clock
// cycles and 100 MHz real-time ticks from the loop's start to its end, taken
// by the first wave.
__global__ __launch_bounds__(512) void mfma_ceiling_kernel(const bf16x8 *__restrict__ frags, float *__restrict__ out,
                                                           uint64_t *__restrict__ stamps, int32_t steps)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    bf16x8 a[2][8], b[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            a[h][i] = frags[(wave * 24 + h * 12 + i) * 64 + lane];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            b[h][j] = frags[(wave * 24 + h * 12 + 8 + j) * 64 + lane];
    }
    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    wait_all();
    const uint64_t c0 = shader_cycles(), t0 = realtime();
    for (int s = 0; s < steps; s += 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[h][j], a[h][i], acc[i][j], 0, 0, 0);
    }
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            sum += (acc[i][j][0] + acc[i][j][1]) + (acc[i][j][2] + acc[i][j][3]);
    const uint64_t c1 = shader_cycles(), t1 = realtime();
    out[(int64_t)blockIdx.x * 512 + threadIdx.x] = sum;
    if (threadIdx.x == 0) {
        stamps[2 * (int64_t)blockIdx.x] = c1 - c0;
        stamps[2 * (int64_t)blockIdx.x + 1] = t1 - t0;
    }
}

} // namespace pts
