/*
 * pts_gemm.h -- C ABI of the persistent-tile-scheduled bf16 GEMM for MI355X (gfx950).
 *
 * The library computes D = A * B for one problem or for a group of independent
 * problems in ONE persistent kernel launch. A fixed set of resident
 * workgroups ("workers") each loops over output tiles. Where a worker's next
 * tile comes from is the schedule:
 *
 *   - static grid-stride: worker w takes tiles w, w+P, w+2P, ... (P workers).
 *     This is the static persistent schedule of "Advanced scheduling: Cluster
 *     Launch Control", section "Limits of the static persistent scheduler",
 *     and the static persistent shape of the CUTLASS Task Scheduling page
 *     "Schedules", section "Scheduling Shapes".
 *   - dynamic work claiming: every tile, the first one included, is claimed
 *     from one device-wide atomic counter. The claim for the next tile is
 *     issued while the current tile is still being computed (once its last
 *     ring stage is loaded), and a claim that returns an index >= the tile
 *     count ends the worker's loop; it never claims again.
 *     This is the single-GPU analogue of the hardware work stealing in "Advanced
 *     scheduling: Cluster Launch Control", sections "One CLC request" and
 *     "Overlapping the request with the current computation".
 *
 * Both schedules run the same tile body (same loads, same MFMA order, same
 * epilogue), so for identical inputs they write bit-identical D; only the
 * source of the next tile coordinate differs ("Advanced scheduling: Cluster
 * Launch Control", section "When to use CLC").
 *
 * Operand layouts (the only ones supported):
 *   A: M x K, row-major,    A[i][k] = a[i * lda + k], bf16
 *   B: K x N, column-major, B[k][j] = b[j * ldb + k], bf16
 *   D: M x N, row-major,    D[i][j] = d[i * ldd + j], fp32 or bf16
 * Products are exact and accumulate in fp32 (MFMA). bf16 output rounds the
 * fp32 sum to nearest, ties to even. A tile sums its k-tiles in a rotated
 * order that starts at a k-tile fixed by the tile's position in the plan (so
 * that the compute dies do not all read the same k-slice at once): results
 * are deterministic, equal across schedules and worker counts, and differ
 * from a left-to-right fp32 sum only by rounding order.
 *
 * Memory: every pointer is device memory owned by the caller; the library
 * never allocates, frees or reads host copies of operand data. A plan owns a
 * few bytes of device memory of its own (tile metadata and the claim
 * counters), allocated in gemm_plan_create and freed in gemm_plan_destroy.
 *
 * Streams: `stream` arguments are hipStream_t values passed as void*
 * (NULL = the default stream). Every run is asynchronous on its stream.
 *
 * Threads and concurrency: a plan is not thread-safe, and one plan must not
 * have two runs in flight at once (its claim counter is per plan); create one
 * plan per concurrent stream instead. Runs of different plans may overlap.
 *
 * Errors: every call returns a gemm_status; gemm_last_error() returns a
 * message for the most recent failure on the calling thread.
 */
#ifndef PTS_GEMM_H
#define PTS_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_VALUE = 1, /* a NULL pointer, a bad size, stride or alignment */
    GEMM_ERR_UNSUPPORTED = 2,   /* a layout, dtype, tile or group count the library does not build */
    GEMM_ERR_OUT_OF_MEMORY = 3, /* the plan's own device memory could not be allocated */
    GEMM_ERR_HIP = 4,           /* a HIP runtime call failed (launch, copy, device query) */
    GEMM_ERR_TIMEOUT = 5        /* a bounded device-side wait ran out (probe kernel only) */
} gemm_status;

typedef enum { GEMM_DTYPE_BF16 = 0, GEMM_DTYPE_F32 = 1 } gemm_dtype;
typedef enum { GEMM_ROW_MAJOR = 0, GEMM_COL_MAJOR = 1 } gemm_layout;
/* STATIC: grid-stride. DYNAMIC: every tile claimed from one device-wide
 * counter. DYNAMIC_XCD: one counter per XCD (chiplet) over the tiles the
 * static schedule deals to that XCD (logical indices x, x+8, x+16, ...), so
 * the tiles in flight on an XCD share its L2; a worker whose XCD's sequence is
 * used up claims from the other XCDs' sequences in turn.
 * NONPERSISTENT: not a persistent kernel -- one workgroup per tile (grid =
 * tile count), dispatched by the hardware as compute units free up; the
 * comparison point the persistent schedules replace ("Schedules", section
 * "Scheduling Shapes"). num_workers must be 0 with it. */
typedef enum {
    GEMM_SCHEDULE_STATIC = 0,
    GEMM_SCHEDULE_DYNAMIC = 1,
    GEMM_SCHEDULE_DYNAMIC_XCD = 2,
    GEMM_SCHEDULE_NONPERSISTENT = 3
} gemm_schedule;

/* Largest group count one plan accepts: the per-problem operand pointers of a
 * run travel in the kernel's argument block. */
#define GEMM_MAX_GROUPS 64

/* One problem. m, n, k >= 0 and each below 2^31. ld = 0 selects the packed
 * value (lda = ldb = k, ldd = n). lda and ldb must be multiples of 8 (rows of
 * A and columns of B start 16-byte aligned) and >= k; ldd >= n. */
typedef struct {
    int64_t m, n, k;
    int64_t lda, ldb, ldd;
} gemm_shape;

/* Plan flags. */
#define GEMM_FLAG_NONE 0u
/*
 * Stage hand-off inside the k loop (persistent-kernel page, pipeline groups:
 * "FusedMerge" and "Merge" barrier layouts). By default one workgroup barrier
 * per ring stage serves as the stage's full and empty barrier at once. With
 * one of these flags the stages instead carry arrive counters in LDS, and a
 * wave waits only for the stage it needs next:
 *   GEMM_FLAG_STAGE_FLAGS_FUSED:  one full and one empty counter per stage
 *                                 (2 words per stage; all loads of a stage
 *                                 arrive on the one full counter);
 *   GEMM_FLAG_STAGE_FLAGS_MERGED: a full counter for A, a full counter for B,
 *                                 one empty counter (3 words per stage).
 * Results are bit-identical to the barrier form. Built for the 8-wave 16x16
 * two-stage kernel (the 256x256 default); other kernels, or both flags at
 * once, give GEMM_ERR_UNSUPPORTED. A device-side wait is bounded: one that runs
 * out is counted in out[4] of gemm_plan_read_counters, and that run's D is void.
 */
#define GEMM_FLAG_STAGE_FLAGS_FUSED 1u
#define GEMM_FLAG_STAGE_FLAGS_MERGED 2u
/*
 * Tile order of a grouped plan. By default the problems are laid out in the
 * tile space deepest first (descending number of k-tiles, ties in descriptor
 * order), so the costliest tiles are taken first and the cheap ones fill the
 * end of the run, whatever the schedule. With this flag the problems keep the
 * descriptor's order (the offsets-array order of the "Schedules" page,
 * section "Dynamic Domain"). Only the tile order changes: every tile is
 * computed once either way, traces report the descriptor's problem index.
 */
#define GEMM_FLAG_PROBLEM_ORDER_AS_GIVEN 4u
/*
 * Test only, with a stage-flag layout: every wait for a full counter asks for
 * one arrival more than can ever come, so every such wait runs out. Each wave
 * counts its first expired wait in out[4] of gemm_plan_read_counters and waits
 * no more; the kernel ends and D is void. It shows that the waits are bounded.
 */
#define GEMM_FLAG_DEBUG_STAGE_FLAG_STALL 8u
/*
 * Claim timing of the dynamic schedules (request-ahead off). By default a
 * worker asks for its next tile once the current tile's last stage is in LDS,
 * so the request's round trip overlaps the last k-tile (the Cluster Launch
 * Control page, section on overlapping the request with the current
 * computation). With this flag the request goes out only once the tile's
 * computation is done (after its k loop in the default 256x256 kernel with
 * bf16 output, which starts the next tile's loads before its epilogue; after
 * its epilogue in the other kernels) and the worker waits for the answer: the
 * baseline that shows what the overlap is worth. Results are identical; the
 * static and non-persistent schedules issue no requests and ignore it.
 */
#define GEMM_FLAG_CLAIM_AFTER_TILE 16u

/*
 * tile_m = tile_n = GEMM_TILE_AUTO: gemm_plan_create picks the output tile
 * from the problem sizes and the device: the first of 256x256, 256x128 and
 * 128x128 whose tile count (over all problems) reaches 55% of the compute
 * units, else 64x64, each with its default kernel. Large tiles read the least memory per
 * flop; a problem with too few of them leaves most of the chip idle. The other
 * kernel fields (tile_k, stages, load_path, waves, mfma) must then be 0 and no
 * stage-flag layout requested, else GEMM_ERR_INVALID_VALUE. This needs a
 * current HIP device (GEMM_ERR_HIP otherwise); gemm_plan_query_kernel reports
 * the tile chosen.
 */
#define GEMM_TILE_AUTO (-1)

typedef struct {
    int32_t group_count;       /* 1 = one GEMM; 2..GEMM_MAX_GROUPS = grouped, one launch */
    const gemm_shape *shapes;  /* host array[group_count]; copied by gemm_plan_create */
    int32_t layout_a;          /* GEMM_ROW_MAJOR */
    int32_t layout_b;          /* GEMM_COL_MAJOR */
    int32_t layout_d;          /* GEMM_ROW_MAJOR */
    int32_t dtype_a;           /* GEMM_DTYPE_BF16 */
    int32_t dtype_b;           /* GEMM_DTYPE_BF16 */
    int32_t dtype_acc;         /* GEMM_DTYPE_F32 */
    int32_t dtype_d;           /* GEMM_DTYPE_F32 or GEMM_DTYPE_BF16 */
    int32_t tile_m, tile_n;    /* output tile; 0 = 256, GEMM_TILE_AUTO = chosen by size. Built: 256x256,
                                  256x128, 128x128, 64x64 */
    int32_t tile_k;            /* k-tile depth of one LDS ring stage: 0 or 64 (the only depth built) */
    int32_t stages;            /* LDS ring stages: 0 or 2 (the only ring built) */
    int32_t load_path;         /* how a ring stage is filled: 0 or 1 = global->LDS loads (the only path) */
    int32_t waves;             /* waves per workgroup: 0 = default, 4 or 8. Built kernels:
                                    256x256: 8 waves (two per SIMD) with 16x16x32 MFMAs (default), or
                                             4 waves (one per SIMD) with 16x16x32 MFMAs;
                                    256x128: 8 waves, 16x16x32;
                                    128x128 and 64x64: 4 waves, 32x32x16 */
    int32_t mfma;              /* matrix instruction: 0 = the tile's kernel, 16 (16x16x32) or 32 (32x32x16),
                                  as listed above */
    int32_t schedule;          /* gemm_schedule */
    int32_t num_workers;       /* 0 = one per compute unit times occupancy, capped at the tile count */
    uint32_t flags;            /* GEMM_FLAG_* */
} gemm_desc;

typedef struct gemm_plan gemm_plan; /* opaque */

/* Device pointers of one problem. a and b must be 16-byte aligned; d at
 * least element aligned. A must be readable over (m-1)*lda + roundup(k, 8)
 * elements and B over (n-1)*ldb + roundup(k, 8): the last row of A (column
 * of B) is read in whole 16-byte chunks. Elements of D outside the m x n
 * region (row padding up to ldd) are never written. */
typedef struct {
    const void *a;
    const void *b;
    void *d;
} gemm_operands;

/* Message for a status code (static storage). The codes name the checks the
 * pages ask for before anything runs: a mismatched configuration is rejected
 * when it is put together, not at run time (CUTLASS Task Scheduling page
 * "Pipeline Groups", section "How member configs are merged"; "Introduction",
 * section "Authoring Lifecycle", step 6: validation before lowering). */
const char *gemm_status_string(gemm_status status);

/* Message describing the most recent failure on this thread ("" if none). */
const char *gemm_last_error(void);

/*
 * Validate a descriptor and build a plan on the current HIP device.
 * Everything checkable without the operand pointers is checked here (shapes,
 * strides, layouts, dtypes, tile size, worker count); on any error *out_plan is
 * set to NULL and nothing is allocated. The validation mirrors the pages'
 * rule that mismatched pipeline configurations are rejected when the group is
 * constructed (CUTLASS Task Scheduling page "Pipeline Groups", section "How
 * member configs are merged").
 */
gemm_status gemm_plan_create(const gemm_desc *desc, gemm_plan **out_plan);

/*
 * Run the plan: one persistent kernel launch on `stream` computing every
 * problem of the plan. This is the pages' persistent schedule: a fixed grid of
 * workers each running the work-tile loop, taking its next tile from the
 * queue at the end of every iteration ("Schedules", sections "Persistent
 * Scheduling" and "Scheduling Shapes"), the tile body being the GEMM
 * mainloop of "Pipeline Groups", section "Overview". `ops` is a host array of desc.group_count operand sets.
 * Returns GEMM_ERR_INVALID_VALUE for a NULL or misaligned pointer (nothing is
 * launched), GEMM_ERR_HIP if the launch fails. No element of any problem's D
 * may lie in another problem's D or in any problem's A or B (D blocks may
 * interleave inside one wider matrix, as column blocks do); overlapping
 * operands are not detected and give undefined results. Problems with m = 0 or n = 0
 * write nothing; k = 0 writes zeros. The run must be on the device the plan
 * was created on. The call enqueues that one kernel and nothing else (no
 * memset, copy or host synchronisation; the dynamic schedules' claim counters
 * are put back to zero by the kernel at the end of each run), so it may be
 * recorded into a HIP graph by stream capture and replayed; the operand
 * pointers are then fixed at capture time.
 */
gemm_status gemm_run(gemm_plan *plan, const gemm_operands *ops, void *stream);

/* Free the plan and its device memory (the claim counters and the problem
 * table, which the plan owns the way a pipeline group owns its shared barrier
 * storage: "Pipeline Groups", section "Setup"). NULL is a no-op. The caller
 * must ensure no run of the plan is still executing. GEMM_ERR_HIP if the
 * runtime refuses the free (the plan's host part is released regardless). */
gemm_status gemm_plan_destroy(gemm_plan *plan);

/* Tile count, worker count (grid size; the tile count for the non-persistent
 * schedule) and LDS bytes per workgroup of a plan: the size of the tile space
 * the work queue hands out and of the persistent grid that drains it
 * ("Schedules", section "Scheduling Shapes"; "Advanced scheduling: Cluster
 * Launch Control", section "Limits of the static persistent scheduler", whose
 * example has 12 tiles and 4 workers). Any output pointer may be NULL;
 * GEMM_ERR_INVALID_VALUE for a NULL plan. */
gemm_status gemm_plan_query(const gemm_plan *plan, int64_t *num_tiles, int32_t *num_workers,
                            int32_t *lds_bytes);

/* The kernel a plan runs: output tile (tile_m x tile_n, also when the
 * descriptor asked for GEMM_TILE_AUTO), k-tile depth, ring stages, waves per
 * workgroup and MFMA block edge (16 or 32). Any output pointer may be NULL;
 * GEMM_ERR_INVALID_VALUE for a NULL plan. */
gemm_status gemm_plan_query_kernel(const gemm_plan *plan, int32_t *tile_m, int32_t *tile_n, int32_t *tile_k,
                                   int32_t *stages, int32_t *waves, int32_t *mfma);

/*
 * Per-tile trace (test and benchmark use): which worker ran which tile, in
 * what order and when -- the record behind the exactly-once and launch-tail
 * statements of "Advanced scheduling: Cluster Launch Control", sections
 * "Limits of the static persistent scheduler" and "One CLC request" (the
 * 12-tile / 4-worker assignment table). After this call every run writes,
 * into `device_buf`, one record per tile followed by one record per worker:
 *
 *   struct { int32 tile, claim, worker, seq, group, row0, col0; uint32 xcc_id,
 *            cycles, pad; uint64 t_start, t_end; } -- 56 bytes, at index `tile`
 *   struct { uint64 t_start, t_end; int32 tiles, worker; uint32 hw_id, xcc_id; }
 *                                                  -- 32 bytes, at index `worker`
 *
 * `tile` is the tile's position in the plan's tile order (problems in turn,
 * deepest first unless GEMM_FLAG_PROBLEM_ORDER_AS_GIVEN; inside a problem,
 * groups of 8 tile rows walked column by column), `group` the problem's index
 * in the descriptor, `claim`
 * the scheduler's value that selected it (static: the logical grid-stride
 * index; dynamic: the counter value; per-XCD: XCD * 2^24 + counter value v,
 * i.e. logical index XCD + 8 v).
 * Times are the 100 MHz device real-time counter; seq is the tile's place in
 * its worker's sequence; hw_id is the wave's HW_ID register and xcc_id its
 * XCC (chiplet) id; `cycles` counts shader-clock cycles over the same span,
 * so cycles / (10 ns * (t_end - t_start)) is the clock in GHz.
 * `bytes` must be >= 56 * num_tiles + 32 * num_workers.
 * device_buf = NULL switches tracing off.
 */
gemm_status gemm_plan_set_trace(gemm_plan *plan, void *device_buf, size_t bytes);

/* Size of the scheduler's counter block: the plan's own, and the `counters`
 * array that pts_sched_probe takes. */
#define GEMM_SCHED_COUNTER_BYTES 36864

/*
 * Read the plan's scheduler counters (synchronizes the device): out[0] the
 * live claim counters, summed (0 between dynamic runs), out[1] the live exit counter
 * (0 between runs), out[2] the total number of claims in the last dynamic run
 * (single counter: tiles + workers, since every worker's loop ends on exactly
 * one failed claim), out[3] the number of dynamic runs completed, out[4] the
 * number of stage-flag waits that ran out since the plan was created (always 0
 * unless the stage hand-off is broken; see GEMM_FLAG_STAGE_FLAGS_FUSED).
 */
gemm_status gemm_plan_read_counters(const gemm_plan *plan, uint32_t out[5]);

/*
 * Test only: set the dynamic schedules' claim counters (synchronizes the
 * device), as if `value` claims had already been taken before the next run.
 * GEMM_SCHEDULE_DYNAMIC: the single counter, so that run processes exactly
 * the tiles value .. T-1 (value >= T: every worker's first claim fails and the
 * run writes nothing). GEMM_SCHEDULE_DYNAMIC_XCD: every XCD's counter, so each
 * XCD's sequence starts at its value-th entry. This replays the failed request
 * of "Advanced scheduling: Cluster Launch Control", section "One CLC request"
 * (a worker that finds the pool drained leaves its loop at once). The run's
 * self-reset puts the counters back to 0 afterwards. GEMM_ERR_INVALID_VALUE for
 * a NULL plan, another schedule, or value >= 2^24.
 */
gemm_status gemm_plan_preset_claims(gemm_plan *plan, uint32_t value);

/* Bytes of the per-GPU scratch array gemm_run_noalloc uses (the claim counter
 * block, then a table of GEMM_MAX_GROUPS problems). */
#define GEMM_NOALLOC_SCRATCH_BYTES 40960

/*
 * gemm_run without a plan and without allocating, for callers that cannot
 * call hipMalloc: code being recorded under HIP graph capture, tight serving
 * loops, harnesses that forbid device allocation.
 *
 * `desc` is validated exactly as by gemm_plan_create (same errors, same
 * tile, kernel and tile order) and `ops` / `stream` are as for gemm_run; the
 * result is bit-identical to gemm_run of a plan built from the same `desc`.
 * Instead of plan-owned memory the call uses a file-scope device array of
 * GEMM_NOALLOC_SCRATCH_BYTES bytes, one per GPU, kept until the process ends:
 * no hipMalloc, hipFree or other allocating call is made (the array's address
 * is looked up once per device, on the first call there). Limits: at most
 * GEMM_MAX_GROUPS problems (the scratch table's size; more give
 * GEMM_ERR_UNSUPPORTED), no trace. Each call enqueues two kernels on `stream`:
 * one that writes the problem table into the scratch and zeroes the claim
 * counters, then the GEMM. Every call on a GPU shares that GPU's scratch, so
 * calls that overlap on one GPU (two streams, or two host threads, without
 * ordering between them) race and their results are void: order them.
 */
gemm_status gemm_run_noalloc(const gemm_desc *desc, const gemm_operands *ops, void *stream);

/*
 * Grid-stride int16 copy dst[i] = src[i] for 0 <= i < n, 16 bytes per lane per
 * step ("Schedules", section "Domains": start = block * threads + thread,
 * step = grid * threads, indices >= n untouched). Used as the concurrent
 * HBM-bound load beside a GEMM. src and dst must be 16-byte aligned and must
 * not overlap. num_blocks = 0 picks one block per compute unit times 4.
 */
gemm_status pts_copy_int16(const void *src, void *dst, int64_t n, int32_t num_blocks, void *stream);

/*
 * A stream whose kernels run only on the first `cu_count` compute units of
 * the current device (hipExtStreamCreateWithCUMask), default priority. It
 * stands for "another kernel occupies part of the CUs" beside a GEMM ("Advanced
 * scheduling: Cluster Launch Control", section "Limits of the static
 * persistent scheduler"): a copy launched on it holds those CUs, so GEMM
 * workers placed there start late. 1 <= cu_count <= compute units, else
 * GEMM_ERR_INVALID_VALUE; *out_stream is NULL on error. Destroy it with
 * pts_stream_destroy (NULL is a no-op) once its work has finished.
 */
gemm_status pts_stream_create_cu_masked(int32_t cu_count, void **out_stream);
gemm_status pts_stream_destroy(void *stream);

/*
 * Scheduler probe: runs the tile scheduler alone, with `work_ns` of busy-wait
 * standing in for each tile's work, one 64-thread workgroup per worker.
 * out_tiles[w * max_per_worker + i] receives the i-th tile worker w processed
 * and out_counts[w] how many; both are device arrays of num_workers rows.
 * gate_worker >= 0 holds that worker back until all others have finished
 * (bounded by spin_limit polls; on expiry out_status[0] = 1), which replays a
 * worker that starts late. out_tiles holds the logical index (static) or
 * counter value (dynamic) of each tile, or its position (per-XCD claiming).
 * counters: device array of GEMM_SCHED_COUNTER_BYTES bytes, zeroed by the
 * caller before the first call (the claim counters reset themselves at the
 * end of every call); 4-byte aligned.
 * out_status: device array of 1 uint32.
 */
gemm_status pts_sched_probe(int32_t num_tiles, int32_t num_workers, int32_t schedule,
                            int32_t gate_worker, int64_t work_ns, int64_t spin_limit,
                            int32_t *out_tiles, int32_t *out_counts, int32_t max_per_worker,
                            uint32_t *counters, uint32_t *out_status, void *stream);

/*
 * Matrix-unit ceiling probe: the default GEMM kernel's MFMA work (8 waves per
 * workgroup, each running the 32 v_mfma_f32_16x16x32_bf16 of one k-step of a
 * 128x64 accumulator block per step) with no memory traffic inside its loop,
 * for measuring what the matrix units sustain under the power limit beside
 * the GEMM ("Pipeline Groups", section "Overview": the MMA consumer alone,
 * with its loaders and store taken away). One launch does
 * blocks x 8 x steps x 32 x 16384 FLOP; num_blocks = 0 runs one workgroup per
 * compute unit, and steps = 1024 then matches the FLOP of one 8192^3 GEMM.
 * frags: device array of PTS_MFMA_CEILING_FRAG_BYTES bytes (bf16 operand
 * fragments, read once), 16-byte aligned. out: device array of
 * num_blocks x 512 floats (per thread, the sum of its accumulators: with every
 * fragment element 1.0 each is 4096 x steps). stamps: device array of
 * num_blocks x 2 uint64 (shader cycles, then 100 MHz ticks, of each
 * workgroup's loop). steps must be even and >= 2, num_blocks in [0, 65536];
 * GEMM_ERR_INVALID_VALUE otherwise, with nothing launched.
 */
#define PTS_MFMA_CEILING_FRAG_BYTES 196608
gemm_status pts_mfma_ceiling(const void *frags, float *out, uint64_t *stamps, int32_t num_blocks, int32_t steps,
                             void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PTS_GEMM_H */
