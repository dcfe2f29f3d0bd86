// Persistent bf16 GEMM kernel for gfx950: D = A * B, fp32 accumulate.
//
// Dataflow (CUTLASS Task Scheduling page "Pipeline Groups", section
// "Overview": the GEMM mainloop is the canonical Merge -- smem_a and smem_b are
// filled by their loaders, consumed together by the MMA into the
// accumulator, which the store writes to D):
//
//   HBM --(128-bit global->LDS loads)--> LDS ring of STAGES stages (A and B)
//       --(ds_read_b128 fragments)--> v_mfma_f32_32x32x16_bf16 or
//           v_mfma_f32_16x16x32_bf16, fp32 accumulators in registers
//       --(masked epilogue, fp32 or bf16 round-to-nearest-even)--> D
//
// Workgroup: WAVES_M x WAVES_N waves (2 x 2, or 2 x 4 for two waves per SIMD);
// each wave owns a (BM/WAVES_M) x (BN/WAVES_N) block of the output tile and,
// for every k-tile, issues its share of the ring stage's loads. Load and compute overlap through the ring: while stage s is
// consumed, the loads for the k-tile STAGES-1 ahead are in flight. The
// hand-off of a stage (producer commit -> consumer wait, consumer release ->
// producer acquire, in the pages' acquire/commit/wait/release terms of the
// "Introduction" page, section "Core Terms") is: wait for this wave's own
// loads of the stage (vmcnt), then one workgroup barrier, which also proves
// every wave has finished reading the stage that the next loads overwrite.
//
// Per persistent tile the accumulators restart from zero, the MFMA analogue
// of resetting scale_d per work tile ("Resources" page, per-work-tile state).
// The k loop is the schedule's domain loop; with one k-tile it is both the
// first and the last iteration ("Schedules" page, section "First, Last, and
// Periodic Iteration").
//
// Ragged edges: rows of A beyond M and columns of B beyond N are read from
// the last valid row/column (values land only in output elements that the
// epilogue masks off); k beyond K is zeroed in LDS after the last k-tile's
// loads land, so out-of-range k contributes exactly 0. The epilogue writes
// only i < M, j < N ("Schedules" page, section "Domains": in-range indices
// only).
#pragma once

#include "common.h"
#include "scheduler.h"

namespace pts {

#ifndef PTS_MAX_GROUPS
#define PTS_MAX_GROUPS 64
#endif

// One problem of a (grouped) run; plan-owned device table.
struct GroupDesc {
    int32_t m, n, k;
    int32_t tiles_n;     // ceil(n / BN)
    int32_t tile_begin;  // index of the problem's first tile in the run's tile space
    int32_t num_k_tiles; // ceil(k / BK)
    int32_t index;       // the problem's index in the plan descriptor (tile order may differ)
    int32_t band_rows;   // tile rows per band of the tile order (raster_tile)
    int64_t lda, ldb, ldd;
};

struct TileTrace {
    int32_t tile, claim, worker, seq, group, row0, col0;
    uint32_t xcc_id;
    uint32_t cycles; // shader-clock cycles from t_start to t_end (clock = cycles / elapsed)
    uint32_t pad;
    uint64_t t_start, t_end;
};
static_assert(sizeof(TileTrace) == 56, "trace record layout");

struct WorkerTrace {
    uint64_t t_start, t_end;
    int32_t tiles, worker;
    uint32_t hw_id, xcc_id;
};
static_assert(sizeof(WorkerTrace) == 32, "trace record layout");

struct GemmArgs {
    const GroupDesc *groups;
    uint32_t *counters;
    uint8_t *trace; // TileTrace[total_tiles] then WorkerTrace[num_workers], or null
    int32_t group_count;
    int32_t total_tiles;
    int32_t num_workers;
    int32_t schedule;
    int32_t round;     // static dealing width (see static_position)
    int32_t full_excess; // test only: added to every stage-flag full target (0 in normal runs)
    int32_t k_phase_row; // k-tiles between successive tile rows' k starts (see k_phase)
    int32_t claim_late;  // 1: the next tile is requested after this tile's epilogue, not before it
    uint64_t d_vec_ok; // bit g: problem g's D rows start 16-byte aligned (whole-chunk stores)
    const uint16_t *a[PTS_MAX_GROUPS];
    const uint16_t *b[PTS_MAX_GROUPS];
    void *d[PTS_MAX_GROUPS];
};

// How a ring stage is handed from its loads to its readers and back.
enum : int {
    SYNC_BARRIER = 0, // one workgroup barrier per stage serves as full and empty
    SYNC_FUSED = 1,   // per stage: one full and one empty arrive counter (2 words per stage)
    SYNC_MERGED = 2   // per stage: full for A, full for B, one empty (3 words per stage)
};

// LOAD_PATH: how a ring stage is filled (one path is built).
enum : int {
    LOAD_DMA = 0 // global -> LDS loads (buffer_load ... lds), no registers
};

// The matrix instruction: a 32x32 output block per 16-deep k-step, or a 16x16
// block per 32-deep k-step. Both take one 16-byte fragment per lane for each
// operand (8 consecutive k of one row of A / column of B) and do the same
// work per cycle; the 16x16 form needs two waves per SIMD to issue at full
// rate and draws less power per operation, so it holds a higher clock.
template <int MB> struct Mfma;
template <> struct Mfma<32> {
    using Acc = f32x16;
    static constexpr int KM = 16;
    static __device__ __forceinline__ Acc run(bf16x8 x, bf16x8 y, Acc c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c, 0, 0, 0);
    }
};
template <> struct Mfma<16> {
    using Acc = f32x4;
    static constexpr int KM = 32;
    static __device__ __forceinline__ Acc run(bf16x8 x, bf16x8 y, Acc c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, c, 0, 0, 0);
    }
    // The same instruction at a fixed place in the stream: these statements
    // keep their program order with each other and with every memory access
    // (the "memory" clobber), so a hand-placed interleaving of MFMAs, fragment
    // reads and loads is issued as written. The accumulator stays in AGPRs
    // with srcC tied to the destination.
    static __device__ __forceinline__ void run_fixed(bf16x8 x, bf16x8 y, Acc &c)
    {
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(x), "v"(y) : "memory");
    }
};

// WAVES_M x WAVES_N waves per workgroup, one wave tile each. 2 x 2 gives one
// wave per SIMD (512 registers each); 2 x 4 gives two waves per SIMD (256
// registers each), so one wave's LDS and memory waits overlap the other's
// MFMAs. MB is the matrix instruction's output block edge (32 or 16).
// SYNC is the stage hand-off (a compile-time choice, so the default barrier
// form carries none of the counter code).
template <int BM_, int BN_, int BK_, int STAGES_, bool OUT_BF16_, int LOAD_PATH_ = LOAD_DMA, int WAVES_M_ = 2,
          int WAVES_N_ = 2, int MB_ = 32, int SYNC_ = SYNC_BARRIER>
struct GemmConfig {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_;
    static constexpr int SYNC = SYNC_;
    static constexpr bool OUT_BF16 = OUT_BF16_;
    static constexpr int LOAD_PATH = LOAD_PATH_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, WAVES = WAVES_M * WAVES_N, THREADS = 64 * WAVES;
    static constexpr int WAVES_PER_SIMD = WAVES / 4;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N; // wave tile
    static constexpr int MB = MB_;                               // MFMA output block edge
    using Op = Mfma<MB>;
    using Acc = typename Op::Acc;                                // one block's accumulators per lane
    static constexpr int MI = WTM / MB, NI = WTN / MB;           // MFMA blocks per wave
    static constexpr int KSTEPS = BK / Op::KM;                   // MFMA k-steps per k-tile
    static constexpr int KCHUNKS = Op::KM / 8;                   // 16-byte chunks per row per k-step
    static constexpr int ROW_BYTES = BK * 2;                     // one row of A (column of B) per k-tile
    static constexpr int CHUNKS = BK / 8;                        // 16-byte chunks per row
    static constexpr int A_BYTES = BM * ROW_BYTES, B_BYTES = BN * ROW_BYTES;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int ROWS_PER_LOAD = 1024 / ROW_BYTES;       // rows one wave-wide 16 B/lane load covers
    static constexpr int A_LOADS = A_BYTES / 1024 / WAVES;       // per wave (= per thread) per stage
    static constexpr int B_LOADS = B_BYTES / 1024 / WAVES;
    static constexpr int LOADS = A_LOADS + B_LOADS;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    static_assert(BK == 32 || BK == 64, "k-tile");
    static_assert(WTM % MB == 0 && WTN % MB == 0 && KSTEPS >= 1, "wave tile");
    static_assert(A_LOADS >= 1 && B_LOADS >= 1 && A_BYTES % (1024 * WAVES) == 0 && B_BYTES % (1024 * WAVES) == 0,
                  "stage must split into whole 1 KiB wave loads");
    static_assert(STAGES >= 2 && (STAGES - 2) * LOADS <= 63, "vmcnt range");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS capacity");
};

// LDS layout of one operand tile in a stage: row r (a row of A or a column of
// B) holds its BK k-values in CHUNKS 16-byte chunks; logical chunk c sits at
// physical position c ^ swz(r), chosen so that one wave-wide 16-byte-per-lane
// fragment read takes the LDS's full width, measured with the LDS bank
// conflict counter (a read of 64 consecutive 16-byte chunks is active 4
// cycles and conflict-free; the same amount read in a conflicting pattern
// takes 8).
//   16x16x32 operands (MB = 16): lane l reads row l % 16, chunk 4 ks + l / 16.
//     swz = (r >> 1) & 7 measures conflict-free; r ^ (r >> 3 & 1), which
//     spreads any 16 consecutive lanes over distinct bank groups, measures
//     4 conflict cycles per read.
//   32x32x16 operands (MB = 32): lane l reads row l % 32, chunk l / 32 (+2 ks).
//     r ^ (r >> 3 & 1) measures conflict-free; (r >> 2) & 7 does not.
// swz depends on r mod 16 (mod 32 for MB = 32) only, so a lane's fragment
// offsets repeat every MB rows and the per-block differences become
// instruction immediates.
template <int BK, int MB>
__device__ __forceinline__ int lds_swizzle(int r)
{
    if constexpr (BK == 64 && MB == 16)
        return (r >> 1) & 7;
    else if constexpr (BK == 64)
        return (r ^ ((r >> 3) & 1)) & 7;
    else
        return ((r >> 1) ^ ((r >> 3) & 1)) & 3;
}

template <class C>
__device__ __forceinline__ int lds_offset(int r, int c)
{
    return r * C::ROW_BYTES + ((c ^ lds_swizzle<C::BK, C::MB>(r)) << 4);
}

// Wait until this wave's loads of the oldest in-flight stage have landed,
// given how many younger stages (each C::LOADS loads) are still in flight.
// Global->LDS loads complete in issue order, so vmcnt(younger * LOADS) does it.
template <class C, int N>
__device__ __forceinline__ void wait_stage_loads(int younger)
{
    if constexpr (N <= 0) {
        wait_vmcnt<0>();
    } else {
        if (younger >= N)
            wait_vmcnt<N * C::LOADS>();
        else
            wait_stage_loads<C, N - 1>(younger);
    }
}

template <class C>
struct TileCtx {
    int group;     // index in the plan's tile order (selects the operand pointers)
    int problem;   // index in the plan descriptor
    int row0, col0, vm, vn; // tile origin and valid extent
    int k, nk;
    int kt0; // first k-tile of the tile's k order (see k_phase)
    int64_t lda, ldb, ldd;
    const uint16_t *a;
    const uint16_t *b;
    void *d;
    bool vec_ok;
};

// The kernel's argument block, read in place through the kernarg segment
// pointer: indexing its per-problem pointer arrays with a tile-dependent
// problem index then compiles to scalar loads instead of a private copy.
typedef const __attribute__((address_space(4))) GemmArgs *KernArgs;

__device__ __forceinline__ KernArgs kernel_args()
{
    return (KernArgs)__builtin_amdgcn_kernarg_segment_ptr();
}

// Tile order inside one problem, in three levels:
//   * a block: RASTER_ROWS tile rows by RASTER_COLS tile columns, walked
//     column by column (32 consecutive positions, what one die's workers run
//     in one round of the static dealing: a compact block whose A and B
//     panels that die's L2 shares);
//   * a stripe: RASTER_COLS columns of a band of `band` tile rows, its
//     blocks one below the other;
//   * a band: `band` tile rows (a multiple of RASTER_ROWS), its stripes left
//     to right.
// With band = RASTER_ROWS a stripe is one block and a band is walked column
// by column. A problem whose B does not fit the memory-side cache takes wider
// bands (the plan sets `band` per problem): successive rounds then walk along
// one band, whose A panels every round of it reads again while each B panel
// is needed by one round only, so the A band stays cached and B streams past
// once per band instead of once per group of RASTER_ROWS rows. Partial
// bands, stripes and blocks at the edges keep the same order. This is an
// order, not a change of work: every tile has exactly one position.
constexpr int RASTER_ROWS = 8;
constexpr int RASTER_COLS = 4;

__device__ __forceinline__ void raster_tile(int local, int tiles_m, int tiles_n, int band, int &tm, int &tn)
{
    const int first_row = local / (band * tiles_n) * band;
    const int band_rows = min(band, tiles_m - first_row);
    const int in_band = local - first_row * tiles_n;
    const int stripe = in_band / (band_rows * RASTER_COLS);
    const int stripe_cols = min(RASTER_COLS, tiles_n - stripe * RASTER_COLS);
    const int in_stripe = in_band - stripe * band_rows * RASTER_COLS;
    const int block = in_stripe / (RASTER_ROWS * stripe_cols);
    const int block_rows = min(RASTER_ROWS, band_rows - block * RASTER_ROWS);
    const int in_block = in_stripe - block * RASTER_ROWS * stripe_cols;
    tm = first_row + block * RASTER_ROWS + in_block % block_rows;
    tn = stripe * RASTER_COLS + in_block / block_rows;
}

// Where a tile's k loop starts. Each compute die (XCD) works on a compact
// block of tiles whose A and B panels its L2 shares: RASTER_ROWS tile rows by
// a few tile columns. Within a block, the tiles of one tile row start at the
// same k-tile, so they read each A k-slice together; successive rows start
// `row_step` k-tiles apart, so the tiles of one column meet each B k-slice
// one after another, the first bringing it into L2 for the rest, and the
// block's requests at any moment spread over more of the L2. (The plan sets
// row_step to 0 for runs of many rounds, where the workers of a die drift
// apart and the extra offset only breaks the sharing.) Across blocks the
// start is rotated by K_PHASE k-tiles per block, so the dies do not all
// request the same k-slice of memory at once. Each tile still sums every
// k-tile exactly once, in an order fixed by its position and the problem set
// alone, so every schedule and worker count computes the same bits. A block
// is K_PHASE_BLOCK consecutive positions: what the static dealing gives one
// die per round with one workgroup on each of the 256 compute units (32 per
// die). Where a problem's tiles start at a multiple of 8, position % 8 is the
// tile's row inside its raster group (elsewhere it is just another fixed
// offset).
constexpr int K_PHASE = 8;
constexpr int K_PHASE_BLOCK = 32;

__device__ __forceinline__ int k_phase(int pos, int nk, int row_step)
{
    return nk > 0 ? (((pos / K_PHASE_BLOCK) % NUM_XCD) * K_PHASE + (pos % RASTER_ROWS) * row_step) % nk : 0;
}

// The plan's problem table is never written while a kernel runs: read it
// through the constant address space, so a uniform index becomes scalar loads.
typedef const __attribute__((address_space(4))) GroupDesc *ConstGroups;

// Lane l of every wave holds problem l's first tile (or INT32_MAX past the
// last problem): read once per worker, it turns the tile -> problem search
// into one ballot (at most 64 problems, one per lane).
__device__ __forceinline__ int load_group_begin(KernArgs args, int lane)
{
    const ConstGroups groups = (ConstGroups)args->groups;
    return lane < args->group_count ? groups[lane].tile_begin : 0x7FFFFFFF;
}

template <class C>
__device__ __forceinline__ TileCtx<C> decode_tile(KernArgs args, int t, int group_begin)
{
    // problem: the last g with tile_begin <= t (offsets are non-decreasing)
    const int g = __builtin_popcountll(__ballot(group_begin <= t)) - 1;
    const ConstGroups gp = (ConstGroups)args->groups + g;
    GroupDesc gd;
    gd.m = gp->m;
    gd.n = gp->n;
    gd.k = gp->k;
    gd.tiles_n = gp->tiles_n;
    gd.tile_begin = gp->tile_begin;
    gd.num_k_tiles = gp->num_k_tiles;
    gd.lda = gp->lda;
    gd.ldb = gp->ldb;
    gd.ldd = gp->ldd;
    const int local = t - gd.tile_begin;
    int tm, tn;
    raster_tile(local, (gd.m + C::BM - 1) / C::BM, gd.tiles_n, gp->band_rows, tm, tn);
    TileCtx<C> c;
    c.group = g;
    c.problem = gp->index;
    c.row0 = tm * C::BM;
    c.col0 = tn * C::BN;
    c.vm = min(C::BM, gd.m - c.row0);
    c.vn = min(C::BN, gd.n - c.col0);
    c.k = gd.k;
    c.nk = gd.num_k_tiles;
    c.kt0 = k_phase(t, c.nk, args->k_phase_row);
    c.lda = gd.lda;
    c.ldb = gd.ldb;
    c.ldd = gd.ldd;
    c.a = args->a[g];
    c.b = args->b[g];
    c.d = args->d[g];
    c.vec_ok = (args->d_vec_ok >> g) & 1;
    return c;
}

// The order of a k-step's MFMAs over its MI x NI blocks: rows in turn, each
// row's columns ascending on even rows and descending on odd ones, so every
// MFMA shares an operand with the one before it (the row's A fragment inside
// a row, the last column's B fragment across a row change). Under the power
// limit that is worth about 2% of clock against rows all walked the same way
// (measured on an MFMA-only stream of this kernel's shape; with no operand
// shared between neighbours, 3% less again).
template <int NI>
__device__ __forceinline__ constexpr int serpentine_col_of(int mi, int nn)
{
    return (mi & 1) ? NI - 1 - nn : nn;
}

template <class C>
struct Mainloop {
    uint8_t *smem;
    int wave, lane, wm, wn;
    // Operand tiles as buffer descriptors (scalar registers); each load
    // address is descriptor + this thread's 32-bit byte offset + the k-tile's
    // byte offset (a scalar).
    u32x4 a_rsrc, b_rsrc;
    uint32_t a_off[C::A_LOADS];
    uint32_t b_off[C::B_LOADS];

    // logical k-chunk carried by the i-th load of lane ln (same for A and B)
    __device__ __forceinline__ int load_chunk(int i, int nloads, int ln) const
    {
        const int r = (wave * nloads + i) * C::ROWS_PER_LOAD + ln / C::CHUNKS;
        return (ln % C::CHUNKS) ^ lds_swizzle<C::BK, C::MB>(r);
    }
    __device__ __forceinline__ int load_chunk(int i, int nloads) const { return load_chunk(i, nloads, lane); }

    // Paired loads (two waves per SIMD, two ring stages): on a full tile the
    // first wave of each SIMD issues its own loads and those of its partner
    // (wave + 4), whose rows are the same plus a fixed row shift, while the
    // partner only computes. A wave stalled on issuing loads then always has
    // a partner on its SIMD that keeps the matrix unit busy. Edge tiles, whose
    // rows are clamped per lane, load as usual.
    static constexpr bool PAIRED = C::WAVES == 8 && C::STAGES == 2 && C::LOAD_PATH == LOAD_DMA;
    // One wave per SIMD with 16x16 blocks: the hand-laid k loop below.
    static constexpr bool SINGLE = C::WAVES == 4 && C::MB == 16;
    bool full_tile;
    uint32_t a_shift, b_shift; // byte shift from a wave's rows to its partner's

    // The k loop visits k-tiles in the tile's rotated order: iteration kt
    // holds k-tile phys(kt). Every k offset and every "is this the partial
    // last k-tile" test goes through it.
    int kt0, nk_all;
    static __device__ __forceinline__ constexpr int serpentine_col(int mi, int nn)
    {
        return serpentine_col_of<C::NI>(mi, nn);
    }
    __device__ __forceinline__ int phys(int kt) const
    {
        const int p = kt + kt0;
        return p >= nk_all ? p - nk_all : p;
    }
    __device__ __forceinline__ bool is_tail(int kt, int k) const { return (k % C::BK) != 0 && phys(kt) == nk_all - 1; }

    __device__ __forceinline__ void setup(const TileCtx<C> &t)
    {
        kt0 = t.kt0;
        nk_all = t.nk;
        a_rsrc = buffer_rsrc(t.a + (int64_t)t.row0 * t.lda);
        b_rsrc = buffer_rsrc(t.b + (int64_t)t.col0 * t.ldb);
        full_tile = t.vm == C::BM && t.vn == C::BN;
        a_shift = (uint32_t)(4 * C::A_LOADS * C::ROWS_PER_LOAD * t.lda * 2);
        b_shift = (uint32_t)(4 * C::B_LOADS * C::ROWS_PER_LOAD * t.ldb * 2);
        const int ln = lane;
        const int rl = ln / C::CHUNKS;
#pragma unroll
        for (int i = 0; i < C::A_LOADS; ++i) {
            const int r = (wave * C::A_LOADS + i) * C::ROWS_PER_LOAD + rl;
            a_off[i] = (uint32_t)((int64_t)min(r, t.vm - 1) * t.lda * 2) + load_chunk(i, C::A_LOADS, ln) * 16;
        }
#pragma unroll
        for (int i = 0; i < C::B_LOADS; ++i) {
            const int r = (wave * C::B_LOADS + i) * C::ROWS_PER_LOAD + rl;
            b_off[i] = (uint32_t)((int64_t)min(r, t.vn - 1) * t.ldb * 2) + load_chunk(i, C::B_LOADS, ln) * 16;
        }
        if constexpr (SINGLE) {
            // last 16-byte chunk start inside the rows' readable extent, as a
            // byte limit on the k-tile offset of each load's chunk
            const int klast = ((t.k + 7) & ~7) - 8;
#pragma unroll
            for (int p = 0; p < 2; ++p)
                k_lim[p] = (klast - load_chunk(p, C::A_LOADS, ln) * 8) * 2;
        }
    }

    // The one-wave layout's loads. A load's chunk offset is clamped to the
    // last chunk start inside the rows: for every k-tile but a last one that
    // ends inside a k-tile this is the chunk itself, for that one it is what
    // the tail form computes. So one branch-free form serves every k-tile,
    // and a load past the last k-tile is masked off instead of branched over.
    // The logical chunk of load i depends on i only through its parity (the
    // swizzle repeats every 16 rows and a load covers 8), for A and B alike.
    int k_lim[2];
    __device__ __forceinline__ void issue_masked(int i, int kt, int stage, bool on)
    {
        static_assert(C::A_LOADS == C::B_LOADS && C::A_LOADS % 2 == 0 && C::ROWS_PER_LOAD == 8, "chunk parity");
        const bool is_a = i < C::A_LOADS;
        const int j = is_a ? i : i - C::A_LOADS;
        const uint32_t region = is_a ? 0u : (uint32_t)C::A_BYTES;
        const uint32_t wbase =
            opaque_s((uint32_t)(stage * C::STAGE_BYTES) + region + (uint32_t)(wave * C::A_LOADS * 1024));
        const uint32_t off = (is_a ? a_off[j] : b_off[j]) + (uint32_t)min(phys(kt) * C::BK * 2, k_lim[j & 1]);
        dma_load16_if(lds_address(smem + wbase + j * 1024), off, is_a ? a_rsrc : b_rsrc, on);
    }

    // Issue load number `i` (0 .. LOADS-1; A loads first) of this wave's share
    // of k-tile kt into ring stage `stage`: one wave-wide 16-byte-per-lane
    // global->LDS load fills 1 KiB of the stage.
    // Load number i of this wave's share, into the LDS slot of wave `lds_wave`
    // (this wave, or its partner with PARTNER), rows shifted by the partner
    // shift in the latter case.
    template <bool TAIL, bool PARTNER = false>
    __device__ __forceinline__ void issue_one(int i, int kt, int stage, int k)
    {
        const bool is_a = i < C::A_LOADS;
        const int j = is_a ? i : i - C::A_LOADS;
        const int nl = is_a ? C::A_LOADS : C::B_LOADS;
        const int lds_wave = PARTNER ? wave + 4 : wave;
        const uint32_t region = is_a ? 0u : (uint32_t)C::A_BYTES;
        const uint32_t wbase =
            opaque_s((uint32_t)(stage * C::STAGE_BYTES) + region + (uint32_t)(lds_wave * nl * 1024));
        uint32_t off = is_a ? a_off[j] : b_off[j];
        uint32_t soff = (uint32_t)phys(kt) * C::BK * 2;
        if constexpr (TAIL) {
            // last 16-byte chunk start inside the rows' readable extent
            const int klast = ((k + 7) & ~7) - 8;
            const int c = load_chunk(j, nl);
            off = off - c * 16 + min(phys(kt) * C::BK + c * 8, klast) * 2;
            soff = 0;
        }
        if constexpr (PARTNER)
            soff = uniform(soff + (is_a ? a_shift : b_shift));
        dma_load16(lds_address(smem + wbase + j * 1024), off, is_a ? a_rsrc : b_rsrc, soff);
    }

    template <bool TAIL>
    __device__ __forceinline__ void issue(int kt, int stage, int k)
    {
        if constexpr (PAIRED) {
            if (full_tile) {
                if (wave < 4) {
#pragma unroll
                    for (int i = 0; i < C::LOADS; ++i)
                        issue_one<TAIL>(i, kt, stage, k);
#pragma unroll
                    for (int i = 0; i < C::LOADS; ++i)
                        issue_one<TAIL, true>(i, kt, stage, k);
                }
                return;
            }
        }
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i)
            issue_one<TAIL>(i, kt, stage, k);
    }

    __device__ __forceinline__ void issue_any(int kt, int stage, int k, int nk)
    {
        (void)nk;
        if (is_tail(kt, k))
            issue<true>(kt, stage, k);
        else
            issue<false>(kt, stage, k);
    }

    __device__ __forceinline__ void zero_chunk_tail(uint8_t *slot, int k0, int k)
    {
        if (k0 + 8 <= k)
            return;
        u16x8 v = *(u16x8 *)slot;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (k0 + e >= k)
                v[e] = 0;
        *(u16x8 *)slot = v;
    }

    // Zero the k >= K part of the chunks this thread loaded into `stage`
    // (last k-tile only; this thread's loads of the stage have landed).
    // The chunks a wave zeroes are the ones it loaded: with paired loads on a
    // full tile, the first wave of each SIMD zeroes its own and its partner's
    // (after its own load wait covered both) and the partner zeroes none.
    __device__ __forceinline__ void zero_k_tail(int kt, int stage, int k)
    {
        if constexpr (PAIRED) {
            if (full_tile) {
                if (wave < 4) {
                    zero_k_tail_of(wave, kt, stage, k);
                    zero_k_tail_of(wave + 4, kt, stage, k);
                }
                return;
            }
        }
        zero_k_tail_of(wave, kt, stage, k);
    }
    __device__ __forceinline__ void zero_k_tail_of(int w, int kt, int stage, int k)
    {
        uint8_t *sa = smem + stage * C::STAGE_BYTES;
        uint8_t *sb = sa + C::A_BYTES;
        const int koff = phys(kt) * C::BK;
        // the logical chunks of wave w's slots equal this wave's (the swizzle
        // depends on the row modulo 16 and the partner shift is a multiple of 16)
#pragma unroll
        for (int i = 0; i < C::A_LOADS; ++i)
            zero_chunk_tail(sa + (w * C::A_LOADS + i) * 1024 + lane * 16, koff + load_chunk(i, C::A_LOADS) * 8, k);
#pragma unroll
        for (int i = 0; i < C::B_LOADS; ++i)
            zero_chunk_tail(sb + (w * C::B_LOADS + i) * 1024 + lane * 16, koff + load_chunk(i, C::B_LOADS) * 8, k);
    }

    // Byte offset, inside an MB-row block, of this lane's fragment for k-step
    // ks: row lane%MB, logical chunk KCHUNKS*ks + lane/MB.
    uint32_t frag_off[C::KSTEPS];

    __device__ __forceinline__ void setup_fragments()
    {
        const int lr = lane % C::MB, lk = lane / C::MB;
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks)
            frag_off[ks] =
                (uint32_t)(lr * C::ROW_BYTES + (((C::KCHUNKS * ks + lk) ^ lds_swizzle<C::BK, C::MB>(lr)) << 4));
    }

    struct Frags {
        bf16x8 a[C::MI];
        bf16x8 b[C::NI];
    };

    // ds_read_b128 of this wave's A and B fragments for k-step ks of `stage`.
    __device__ __forceinline__ void load_frags(int stage, int ks, Frags &f) const
    {
        const uint32_t sbase = opaque_s((uint32_t)(stage * C::STAGE_BYTES));
        const uint8_t *sa = smem + sbase + wm * C::WTM * C::ROW_BYTES;
        const uint8_t *sb = smem + sbase + C::A_BYTES + wn * C::WTN * C::ROW_BYTES;
#pragma unroll
        for (int mi = 0; mi < C::MI; ++mi)
            f.a[mi] = *(const bf16x8 *)(sa + frag_off[ks] + mi * C::MB * C::ROW_BYTES);
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni)
            f.b[ni] = *(const bf16x8 *)(sb + frag_off[ks] + ni * C::MB * C::ROW_BYTES);
    }

    // MI x NI MFMAs of one k-step. The B fragment is the MFMA's first
    // operand: the result block is D^T, so each lane ends up holding groups of
    // 4 consecutive columns of one row (what the epilogue wants).
    static __device__ __forceinline__ void mma(const Frags &f, typename C::Acc (&acc)[C::MI][C::NI])
    {
#pragma unroll
        for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
            for (int nn = 0; nn < C::NI; ++nn) {
                const int ni = serpentine_col(mi, nn);
                acc[mi][ni] = C::Op::run(f.b[ni], f.a[mi], acc[mi][ni]);
            }
    }

    // Ask the scheduler to interleave the next k-step's fragment reads with
    // this k-step's MFMAs (one read after each MFMA, the rest of the MFMAs
    // after), so LDS latency hides behind matrix work.
    static __device__ __forceinline__ void interleave_reads_with_mfma()
    {
        constexpr int READS = C::MI + C::NI, MFMAS = C::MI * C::NI;
        constexpr int PAIRS = READS < MFMAS ? READS : MFMAS;
#pragma unroll
        for (int i = 0; i < PAIRS; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); // DS read
        }
        if constexpr (MFMAS > PAIRS)
            __builtin_amdgcn_sched_group_barrier(0x008, MFMAS - PAIRS, 0);
        if constexpr (READS > PAIRS)
            __builtin_amdgcn_sched_group_barrier(0x100, READS - PAIRS, 0);
    }

    // ---- stage flags --------------------------------------------------------
    // The pages' per-stage full and empty barriers, as arrive counters in LDS
    // in place of the workgroup barrier (two-stage paired loop only). Every use
    // of a stage adds exactly FLAG_UNIT to each of its words: the loading waves
    // split it on full (all 8 waves load on an edge tile, the first 4 on a full
    // tile), every wave adds 1 to empty once it has issued its last read of the
    // stage. The counters only grow, so a wave waits for "at least the count of
    // this use" and no reset is needed between tiles: `uses` counts this
    // worker's earlier fills of each stage. LDS operations of one wave are
    // performed in order, so an arrive issued after a wave's reads (or after its
    // load wait) is seen only after them.
    static constexpr uint32_t FLAG_UNIT = C::WAVES;
    // polls of a bounded wait: with the sleep and the LDS round trip each, a few
    // million cycles (milliseconds), far beyond any legitimate wait
    static constexpr uint32_t SPIN_LIMIT = 1u << 15;
    // word offsets (+ stage); the fused layout uses the full and empty words only
    static constexpr int W_FULL = 0, W_FULL_B = 2, W_EMPTY = 4;
    __attribute__((address_space(3))) uint32_t *sflags;
    uint32_t *stall_ctr; // device counter of waits that ran out
    static constexpr int sync = C::SYNC;
    uint32_t uses0, uses1;
    uint32_t full_excess; // added to every full target; nonzero only to test the bounded wait
    bool broken; // a wait ran out: stop waiting (the plan's stall counter says the result is void)

    __device__ __forceinline__ uint32_t use_of(int kt) const { return ((kt & 1) ? uses1 : uses0) + (uint32_t)(kt >> 1); }
    __device__ __forceinline__ void count_uses(int nk)
    {
        uses0 += (uint32_t)((nk + 1) >> 1);
        uses1 += (uint32_t)(nk >> 1);
    }
    __device__ __forceinline__ bool loads_this_tile() const { return !(PAIRED && full_tile) || wave < 4; }

    __device__ __forceinline__ void arrive(int word, uint32_t n)
    {
        asm volatile("" ::: "memory");
        if (lane == 0)
            __hip_atomic_fetch_add(sflags + word, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        asm volatile("" ::: "memory");
    }

    // Bounded wait until word >= target (modulo 2^32). A wait that runs out
    // (only a broken protocol could cause it) counts itself in the plan's stall
    // counter and makes this wave stop waiting, so the kernel always ends.
    __device__ __forceinline__ void wait_count(int word, uint32_t target)
    {
        asm volatile("" ::: "memory");
        for (uint32_t i = 0; !broken; ++i) {
            const uint32_t v = __builtin_amdgcn_readfirstlane(
                __hip_atomic_load(sflags + word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
            if ((int32_t)(v - target) >= 0)
                break;
            if (i == SPIN_LIMIT) {
                broken = true;
                if (lane == 0)
                    __hip_atomic_fetch_add(stall_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        asm volatile("" ::: "memory");
    }

    // Flag form of stage_ready(kt): the loading waves wait for their own loads
    // of kt, zero its k tail, and arrive on full; then every wave waits for the
    // full count of this use.
    __device__ __forceinline__ void stage_ready_flags(int kt, const TileCtx<C> &t)
    {
        const int s = kt & 1;
        const uint32_t target = FLAG_UNIT * (use_of(kt) + 1) + full_excess;
        if (loads_this_tile()) {
            const uint32_t share = PAIRED && full_tile ? 2u : 1u;
            if (sync == SYNC_MERGED && !is_tail(kt, t.k)) {
                // A was issued before B (paired: own A, own B, partner A,
                // partner B), so with B_LOADS younger loads left all A has landed
                wait_vmcnt<C::B_LOADS>();
                arrive(W_FULL + s, share);
                wait_vmcnt<0>();
                arrive(W_FULL_B + s, share);
            } else {
                wait_vmcnt<0>();
                if (is_tail(kt, t.k))
                    zero_k_tail(kt, s, t.k);
                arrive(W_FULL + s, share);
                if (sync == SYNC_MERGED)
                    arrive(W_FULL_B + s, share);
            }
        }
        wait_count(W_FULL + s, target);
        if (sync == SYNC_MERGED)
            wait_count(W_FULL_B + s, target);
    }

    // Every wave has issued its last read of k-tile kt's stage.
    __device__ __forceinline__ void release_stage(int kt) { arrive(W_EMPTY + (kt & 1), 1u); }

    // Before loading k-tile kt + 2 into kt's stage: every wave has released kt.
    __device__ __forceinline__ void wait_stage_empty(int kt)
    {
        if (loads_this_tile())
            wait_count(W_EMPTY + (kt & 1), FLAG_UNIT * (use_of(kt) + 1));
    }

    // Wait for this wave's loads of k-tile kt, fix its k tail, then meet the
    // other waves: after this barrier every wave's loads of kt have landed and
    // every wave has finished reading the stage that k-tile kt + STAGES - 1
    // will overwrite.
    __device__ __forceinline__ void stage_ready(int kt, const TileCtx<C> &t)
    {
        wait_stage_loads<C, C::STAGES - 2>(min(C::STAGES - 2, t.nk - 1 - kt));
        if (is_tail(kt, t.k))
            zero_k_tail(kt, kt % C::STAGES, t.k);
        barrier_lds();
    }

    // The tile's k loop. `on_last_stage` runs (in every wave) once the last
    // k-tile's stage is ready and no further load of this tile is waited for
    // with vmcnt, so a memory operation it issues overlaps the last k-tile's
    // MFMAs and the epilogue without any load wait stalling on it.
    //
    // `pre` >= 0: the tile's first two stages were issued before this call
    // (during the previous tile's epilogue), followed by `pre` stores of
    // this thread (the first stage wait leaves both in flight); -1: nothing
    // was issued yet. Only the 16x16 barrier-hand-off loops take it.
    template <class Hook>
    __device__ __forceinline__ void run(const TileCtx<C> &t, typename C::Acc (&acc)[C::MI][C::NI], Hook &&on_last_stage,
                                        int pre = -1)
    {
        static_assert(C::STAGES == 2 && C::LOAD_PATH == LOAD_DMA, "the built k loops use a two-stage ring");
        if constexpr (C::MB == 16 && C::WAVES == 4)
            run_single(t, acc, on_last_stage, pre);
        else if constexpr (C::MB == 16 && C::SYNC == SYNC_BARRIER)
            run_straight(t, acc, on_last_stage, pre);
        else if constexpr (C::MB == 16)
            run_burst_rolling(t, acc, on_last_stage);
        else
            run_burst(t, acc, on_last_stage);
    }

    // ---- rolling fragments (16x16 blocks) ----------------------------------
    // A 16x16 k-step needs MI + NI fragments; two whole sets do not fit two
    // waves per SIMD. Instead the A fragments roll: after row mi's NI MFMAs,
    // A[mi] is dead and its registers receive A[mi] of the next k-step; the B
    // fragments of the next k-step go to a second B set, read during the
    // first NI rows. One A set and two B sets are live.
    // The last ROLL_SPARE rows of A have a second register set: odd k-steps
    // use it, so the next k-step's fragments of those rows can be read early
    // (after rows MI - 2 ROLL_SPARE ..) instead of after their own MFMAs, and
    // a k-step's last read of its stage is issued ROLL_SPARE rows before the
    // k-step ends. The stage barrier that follows k-step 0 waits for that read:
    // one spare row (4 registers) took 2232 -> 2197 cycles per k-tile; two or
    // three were no better or worse.
    static constexpr int ROLL_SPARE = 1 < C::MI / 2 ? 1 : C::MI / 2;
    struct RollFrags {
        bf16x8 a[C::MI];
        bf16x8 ax[ROLL_SPARE > 0 ? ROLL_SPARE : 1];
        bf16x8 b[2][C::NI];
    };

    __device__ __forceinline__ const uint8_t *a_base(int stage) const
    {
        return smem + opaque_s((uint32_t)(stage * C::STAGE_BYTES)) + wm * C::WTM * C::ROW_BYTES;
    }
    __device__ __forceinline__ const uint8_t *b_base(int stage) const
    {
        return smem + opaque_s((uint32_t)(stage * C::STAGE_BYTES)) + C::A_BYTES + wn * C::WTN * C::ROW_BYTES;
    }

    __device__ __forceinline__ void read_all(int stage, int ks, RollFrags &f, int bset) const
    {
        const uint8_t *sa = a_base(stage), *sb = b_base(stage);
#pragma unroll
        for (int mi = 0; mi < C::MI; ++mi)
            f.a[mi] = *(const bf16x8 *)(sa + frag_off[ks] + mi * C::MB * C::ROW_BYTES);
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni)
            f.b[bset][ni] = *(const bf16x8 *)(sb + frag_off[ks] + ni * C::MB * C::ROW_BYTES);
    }

    // One k-step from (f.a, f.b[BS]) while reading k-step (stage, ks) into
    // f.a (rolling) and f.b[BS ^ 1].
    template <int BS>
    __device__ __forceinline__ void rolling_step(RollFrags &f, typename C::Acc (&acc)[C::MI][C::NI], int stage,
                                                 int ks) const
    {
        static_assert(C::NI <= C::MI, "B reads ride on the first NI rows");
        constexpr int SP = ROLL_SPARE, FIRST_EARLY = C::MI - 2 * SP;
        static_assert(SP >= 0 && FIRST_EARLY >= 0, "spare rows");
        const uint8_t *sa = a_base(stage), *sb = b_base(stage);
#pragma unroll
        for (int mi = 0; mi < C::MI; ++mi) {
            const bool spare_row = mi >= C::MI - SP;
#pragma unroll
            for (int nn = 0; nn < C::NI; ++nn) {
                const int ni = serpentine_col(mi, nn);
                acc[mi][ni] = C::Op::run(f.b[BS][ni], (BS == 1 && spare_row) ? f.ax[mi - (C::MI - SP)] : f.a[mi],
                                         acc[mi][ni]);
            }
            if (!spare_row)
                f.a[mi] = *(const bf16x8 *)(sa + frag_off[ks] + mi * C::MB * C::ROW_BYTES);
            if (mi < C::NI)
                f.b[BS ^ 1][mi] = *(const bf16x8 *)(sb + frag_off[ks] + mi * C::MB * C::ROW_BYTES);
            if (mi >= FIRST_EARLY && mi < FIRST_EARLY + SP) {
                // row r = MI - SP + j of the next k-step, into the set it will use
                const int j = mi - FIRST_EARLY, r = C::MI - SP + j;
                const bf16x8 v = *(const bf16x8 *)(sa + frag_off[ks] + r * C::MB * C::ROW_BYTES);
                if (BS == 0)
                    f.ax[j] = v;
                else
                    f.a[r] = v;
            }
        }
        static_for<C::MI>([](auto row) {
            constexpr int mi = decltype(row)::value;
            constexpr int reads = (mi < C::MI - SP ? 1 : 0) + (mi < C::NI ? 1 : 0) +
                                  (mi >= FIRST_EARLY && mi < FIRST_EARLY + SP ? 1 : 0);
            __builtin_amdgcn_sched_group_barrier(0x008, C::NI, 0); // the row's MFMAs
            if constexpr (reads > 0)
                __builtin_amdgcn_sched_group_barrier(0x100, reads, 0); // its reads
        });
    }

    // The loads and stage barriers of run_burst_rolling without its fragment
    // reads and MFMAs (same calls in the same order, so every wave meets the
    // same barriers).
    template <class Hook>
    __device__ __forceinline__ void run_rolling_idle(const TileCtx<C> &t, Hook &on_last_stage, int pre = -1)
    {
        const int nk = t.nk;
        // an idle wave exists only in an edge tile (every wave loads LOADS per stage)
        first_stages<false>(t, pre);
        if (nk == 1)
            on_last_stage();
        for (int kt = 0; kt + 1 < nk; ++kt) {
            stage_ready(kt + 1, t);
            if (kt + 2 < nk)
                issue_any(kt + 2, kt & 1, t.k, nk);
            if (kt + 2 == nk)
                on_last_stage();
        }
    }

    template <class Hook>
    __device__ __forceinline__ void run_burst_rolling(const TileCtx<C> &t, typename C::Acc (&acc)[C::MI][C::NI],
                                                      Hook &on_last_stage)
    {
        static_assert(C::KSTEPS % 2 == 0, "B sets alternate by k-step parity");
        const int nk = t.nk;
        if (nk == 0) {
            on_last_stage();
            return;
        }
        if constexpr (C::SYNC == SYNC_BARRIER) {
            // A wave whose whole wave tile lies outside the valid rows or
            // columns of an edge tile computes nothing: it only loads and meets
            // the stage barriers, so edge tiles really are cheaper (its partner
            // on the SIMD gets the matrix unit to itself).
            if (wm * C::WTM >= t.vm || wn * C::WTN >= t.vn) {
                run_rolling_idle(t, on_last_stage);
                return;
            }
        }
        // With stage flags the tile's first two fills need no empty wait: the
        // previous tile's staging barrier came after every release.
        constexpr bool flags = C::SYNC != SYNC_BARRIER;
        issue_any(0, 0, t.k, nk);
        if (flags)
            stage_ready_flags(0, t);
        else
            stage_ready(0, t);
        if (1 < nk)
            issue_any(1, 1, t.k, nk);
        if (nk == 1)
            on_last_stage();
        RollFrags f;
        read_all(0, 0, f, 0);
        for (int kt = 0; kt < nk; ++kt) {
            const int stage = kt & 1;
#pragma unroll
            for (int ks = 0; ks + 1 < C::KSTEPS; ++ks) {
                if (ks & 1)
                    rolling_step<1>(f, acc, stage, ks + 1);
                else
                    rolling_step<0>(f, acc, stage, ks + 1);
            }
            if (flags)
                release_stage(kt);
            if (kt + 1 < nk) {
                if (flags) {
                    stage_ready_flags(kt + 1, t);
                    if (kt + 2 < nk)
                        wait_stage_empty(kt);
                } else {
                    stage_ready(kt + 1, t);
                }
                if (kt + 2 < nk)
                    issue_any(kt + 2, stage, t.k, nk);
                if (kt + 2 == nk)
                    on_last_stage();
            }
            // The last k-step reads k-step 0 of the next k-tile's stage (past
            // the last k-tile: a stage nobody writes any more; unused).
            rolling_step<(C::KSTEPS - 1) & 1>(f, acc, stage ^ 1, 0);
        }
        count_uses(nk);
    }

    // ---- the straightened k loop (8 waves, 16x16 blocks, barrier hand-off) ----
    // The same k-tiles as run_burst_rolling, in the same order with the same
    // loads, barriers and MFMAs, but a k-tile that needs nothing special -- its
    // successor's stage is not the partial k-tile, it issues loads, and those
    // loads are not the partial k-tile's -- runs a body with no test at all:
    // k-step 0, the stage barrier, the loads of k-tile kt + 2, k-step 1. The
    // few k-tiles that need more (the partial one's load and k-tail zeroing,
    // the last two, where loads stop and the next claim goes out) take the
    // general body. Full and edge tiles are separate instances, so the
    // paired-load choice is fixed per instance.

    // This wave's loads of k-tile kt into ring stage `stage`: the k-tile's
    // byte offset is one scalar for all of them, each LDS destination the
    // stage base plus a constant.
    template <bool FULL>
    __device__ __forceinline__ void issue_fast(int kt, int stage)
    {
        const uint32_t soff = (uint32_t)phys(kt) * (uint32_t)(C::BK * 2);
        const uint32_t base = opaque_s(lds_address(smem) + (uint32_t)(stage * C::STAGE_BYTES));
        if constexpr (FULL && PAIRED) {
            if (wave < 4) {
                const uint32_t a0 = base + (uint32_t)(wave * C::A_LOADS * 1024);
                const uint32_t b0 = base + (uint32_t)(C::A_BYTES + wave * C::B_LOADS * 1024);
                issue_set<0>(a0, a_off, a_rsrc, soff);
                issue_set<0>(b0, b_off, b_rsrc, soff);
                issue_set<4 * C::A_LOADS * 1024>(a0, a_off, a_rsrc, uniform((int)(soff + a_shift)));
                issue_set<4 * C::B_LOADS * 1024>(b0, b_off, b_rsrc, uniform((int)(soff + b_shift)));
            }
        } else {
            issue_set<0>(base + (uint32_t)(wave * C::A_LOADS * 1024), a_off, a_rsrc, soff);
            issue_set<0>(base + (uint32_t)(C::A_BYTES + wave * C::B_LOADS * 1024), b_off, b_rsrc, soff);
        }
    }

    template <int EXTRA, int N>
    static __device__ __forceinline__ void issue_set(uint32_t lds_base, const uint32_t (&off)[N], u32x4 rsrc,
                                                     uint32_t soff)
    {
        static_for<N>([&](auto j) {
            constexpr int J = decltype(j)::value;
            dma_load16_at<EXTRA + J * 1024>(lds_base, off[J], rsrc, soff);
        });
    }

    // One k-tile with nothing special about it.
    template <bool FULL>
    __device__ __forceinline__ void straight_ktile(RollFrags &f, typename C::Acc (&acc)[C::MI][C::NI], int kt)
    {
        const int stage = kt & 1;
        rolling_step<0>(f, acc, stage, 1);
        // k-tile kt + 1's loads (this wave's) have landed; every wave is past
        // its reads of stage kt
        wait_vmcnt<0>();
        barrier_lds();
        issue_fast<FULL>(kt + 2, stage);
        rolling_step<1>(f, acc, stage ^ 1, 0);
    }

    // One k-tile of the general body (the loop body of run_burst_rolling).
    template <class Hook>
    __device__ __forceinline__ void general_ktile(RollFrags &f, typename C::Acc (&acc)[C::MI][C::NI], int kt,
                                                  const TileCtx<C> &t, Hook &on_last_stage)
    {
        const int nk = t.nk;
        const int stage = kt & 1;
        rolling_step<0>(f, acc, stage, 1);
        if (kt + 1 < nk) {
            stage_ready(kt + 1, t);
            if (kt + 2 < nk)
                issue_any(kt + 2, stage, t.k, nk);
            if (kt + 2 == nk)
                on_last_stage();
        }
        rolling_step<1>(f, acc, stage ^ 1, 0);
    }

    // The first two stages of a tile: issued here, or (`pre` >= 0) issued
    // already, during the previous tile's epilogue and ahead of its D stores.
    // pre = the number of stores each thread issued after them when that is
    // exactly STORES (the previous tile was a full tile), else 0: the wait for
    // stage 0 then leaves stage 1's loads and those stores in flight.
    static constexpr int STORES = C::BM * C::BN * (C::OUT_BF16 ? 2 : 4) / 16 / C::THREADS; // 16-byte stores per thread
    template <bool FULL>
    __device__ __forceinline__ void first_stages(const TileCtx<C> &t, int pre)
    {
        const int nk = t.nk;
        // this wave's loads of one stage: 2 LOADS for a loading wave of a
        // paired full tile (none for its partner), LOADS otherwise
        constexpr int STAGE_LOADS = (FULL && PAIRED) ? 2 * C::LOADS : C::LOADS;
        if (pre < 0) {
            issue_any(0, 0, t.k, nk);
            wait_vmcnt<0>();
        } else if (pre == STORES && nk > 1) {
            // (kernels whose count does not fit the counter never pass pre > 0)
            if constexpr (STAGE_LOADS + STORES <= 63)
                wait_vmcnt<STAGE_LOADS + STORES>();
            else
                wait_vmcnt<0>();
        } else if (pre == STORES) {
            if constexpr (STORES <= 63)
                wait_vmcnt<STORES>();
            else
                wait_vmcnt<0>();
        } else {
            wait_vmcnt<0>();
        }
        if (is_tail(0, t.k))
            zero_k_tail(0, 0, t.k);
        barrier_lds();
        if (pre < 0 && 1 < nk)
            issue_any(1, 1, t.k, nk);
    }

    // Both first stages of tile t, ahead of the previous tile's D stores.
    __device__ __forceinline__ void issue_first_two(const TileCtx<C> &t)
    {
        if (t.nk > 0)
            issue_any(0, 0, t.k, t.nk);
        if (t.nk > 1)
            issue_any(1, 1, t.k, t.nk);
    }

    template <bool FULL, class Hook>
    __device__ __forceinline__ void run_straight_t(const TileCtx<C> &t, typename C::Acc (&acc)[C::MI][C::NI],
                                                   Hook &on_last_stage, int pre = -1)
    {
        static_assert(C::KSTEPS == 2 && C::STAGES == 2, "two k-steps per k-tile, two stages");
        const int nk = t.nk;
        // the loop iteration whose k-tile is the partial last one (phys = nk - 1), or -1
        const int tail_it = (t.k % C::BK) != 0 ? nk - 1 - kt0 : -1;
        first_stages<FULL>(t, pre);
        if (nk == 1)
            on_last_stage();
        RollFrags f;
        read_all(0, 0, f, 0);
        int kt = 0;
        while (kt < nk) {
            // straight k-tiles need kt + 2 < nk, kt + 2 != tail_it and kt + 1 != tail_it
            int end = nk - 2;
            if (kt <= tail_it - 2)
                end = min(end, tail_it - 2);
            else if (kt == tail_it - 1)
                end = kt;
            for (; kt < end; ++kt)
                straight_ktile<FULL>(f, acc, kt);
            if (kt >= nk)
                break;
            general_ktile(f, acc, kt, t, on_last_stage);
            ++kt;
        }
    }

    template <class Hook>
    __device__ __forceinline__ void run_straight(const TileCtx<C> &t, typename C::Acc (&acc)[C::MI][C::NI],
                                                 Hook &on_last_stage, int pre = -1)
    {
        if (t.nk == 0) {
            on_last_stage();
            return;
        }
        // A wave whose whole wave tile lies outside the valid rows or columns of
        // an edge tile computes nothing: it only loads and meets the stage
        // barriers.
        if (wm * C::WTM >= t.vm || wn * C::WTN >= t.vn) {
            run_rolling_idle(t, on_last_stage, pre);
            return;
        }
        if (full_tile)
            run_straight_t<true>(t, acc, on_last_stage, pre);
        else
            run_straight_t<false>(t, acc, on_last_stage, pre);
    }

    // ---- one wave per SIMD (16x16 blocks) ------------------------------------
    // A wave owns 128x128 of the tile: 64 MFMAs per k-step, 16 fragment reads,
    // 256 accumulators (all AGPRs), and both fragment sets fit in registers.
    // With no second wave on the SIMD to cover a stall, the k-step is laid out
    // by hand: the next k-step's fragment reads and, in the second k-step of a
    // k-tile, this wave's loads of k-tile kt + 2 are spread between the MFMAs,
    // so neither LDS nor the load queue ever holds up the matrix unit in one
    // burst. The reads end well before the k-step does, so the stage barrier
    // finds them complete.
    static constexpr int S_MFMAS = C::MI * C::NI;
    static constexpr int S_READS = C::MI + C::NI;
    static constexpr int READ_EVERY = 3; // one read after every third MFMA
    static constexpr int LOAD_EVERY = 3; // one load after every third MFMA (16 loads over 48 of 64)

    // Fragment read r of a k-step, in the order the next k-step first needs
    // them: A0, B0 .. B(NI-1), A1 .. A(MI-1).
    __device__ __forceinline__ void read_frag(Frags &f, int r, const uint8_t *sa, const uint8_t *sb,
                                              uint32_t foff) const
    {
        if (r == 0)
            f.a[0] = *(const bf16x8 *)(sa + foff);
        else if (r <= C::NI)
            f.b[r - 1] = *(const bf16x8 *)(sb + foff + (r - 1) * C::MB * C::ROW_BYTES);
        else
            f.a[r - C::NI] = *(const bf16x8 *)(sa + foff + (r - C::NI) * C::MB * C::ROW_BYTES);
    }

    // One k-step from `cur`, reading k-step rks of stage rstage into `nxt`.
    // With LOADS, this wave's loads of k-tile lkt go into stage lstage between
    // the MFMAs, masked off unless `on`.
    template <bool LOADS>
    __device__ __forceinline__ void single_step(const Frags &cur, Frags &nxt, typename C::Acc (&acc)[C::MI][C::NI],
                                                int rstage, int rks, int lkt, int lstage, bool on)
    {
        static_assert(S_READS * READ_EVERY <= S_MFMAS && C::LOADS * LOAD_EVERY <= S_MFMAS, "slots");
        const uint8_t *sa = a_base(rstage), *sb = b_base(rstage);
        const uint32_t foff = frag_off[rks];
#pragma unroll
        for (int x = 0; x < S_MFMAS; ++x) {
            const int mi = x / C::NI, ni = serpentine_col(mi, x % C::NI);
            C::Op::run_fixed(cur.b[ni], cur.a[mi], acc[mi][ni]);
            if (x % READ_EVERY == 0 && x / READ_EVERY < S_READS)
                read_frag(nxt, x / READ_EVERY, sa, sb, foff);
            if (LOADS && x % LOAD_EVERY == LOAD_EVERY - 1 && x / LOAD_EVERY < C::LOADS)
                issue_masked(x / LOAD_EVERY, lkt, lstage, on);
        }
    }

    // The same k-step for a k-tile with nothing special about it (the loads,
    // if any, are of a whole k-tile): the k-tile's byte offset is one scalar
    // for all of this wave's loads and each LDS destination is the stage base
    // plus a constant, so a load costs three instructions and no mask. One
    // wave per SIMD issues at most one instruction per issue cycle, and the
    // masked form's ten per load no longer fit between the MFMAs.
    template <bool LOADS>
    __device__ __forceinline__ void single_step_fast(const Frags &cur, Frags &nxt,
                                                     typename C::Acc (&acc)[C::MI][C::NI], int rstage, int rks,
                                                     uint32_t lbase, uint32_t soff)
    {
        static_assert(C::A_LOADS == C::B_LOADS, "A and B slots side by side");
        const uint8_t *sa = a_base(rstage), *sb = b_base(rstage);
        const uint32_t foff = frag_off[rks];
#pragma unroll
        for (int x = 0; x < S_MFMAS; ++x) {
            const int mi = x / C::NI, ni = serpentine_col(mi, x % C::NI);
            C::Op::run_fixed(cur.b[ni], cur.a[mi], acc[mi][ni]);
            if (x % READ_EVERY == 0 && x / READ_EVERY < S_READS)
                read_frag(nxt, x / READ_EVERY, sa, sb, foff);
            if (LOADS && x % LOAD_EVERY == LOAD_EVERY - 1 && x / LOAD_EVERY < C::LOADS) {
                const int i = x / LOAD_EVERY;
                const bool is_a = i < C::A_LOADS;
                const int j = is_a ? i : i - C::A_LOADS;
                dma_load16_imm(lbase, (is_a ? 0 : C::A_BYTES) + j * 1024, is_a ? a_off[j] : b_off[j],
                               is_a ? a_rsrc : b_rsrc, soff);
            }
        }
    }

    // LDS address of this wave's first A slot in `stage` (its B slots start
    // A_BYTES further on).
    __device__ __forceinline__ uint32_t single_lbase(int stage) const
    {
        return opaque_s(lds_address(smem) + (uint32_t)(stage * C::STAGE_BYTES + wave * C::A_LOADS * 1024));
    }

    // Every k-tile has the same shape: k-step 0 (reading k-step 1), the
    // barrier that readies k-tile kt + 1, k-step 1 (reading k-step 0 of kt + 1
    // and loading kt + 2). A k-tile that needs nothing special -- kt + 2 < nk,
    // and neither kt + 1 nor kt + 2 is the partial k-tile -- runs the straight
    // form (no tests, unmasked loads); the others run the general form, where
    // past the end the reads fetch a stage nobody uses and the loads are
    // masked off. Both issue the same loads, barriers and MFMAs in the same
    // order, so the result does not depend on which form ran.
    template <class Hook>
    __device__ __forceinline__ void run_single(const TileCtx<C> &t, typename C::Acc (&acc)[C::MI][C::NI],
                                               Hook &on_last_stage, int pre = -1)
    {
        static_assert(C::STAGES == 2 && C::KSTEPS == 2 && C::LOAD_PATH == LOAD_DMA && !PAIRED, "one-wave layout");
        const int nk = t.nk;
        if (nk == 0) {
            on_last_stage();
            return; // the accumulators keep their zeros
        }
        first_stages<false>(t, pre);
        if (nk == 1)
            on_last_stage();
        Frags f0, f1;
        load_frags(0, 0, f0);
        // The zeros must reach the accumulators before the first MFMA reads
        // them, and the compiler does not see the MFMAs as such: pin the
        // zeroing here and leave the write-to-read latency.
#pragma unroll
        for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni)
                asm volatile("" : "+a"(acc[mi][ni]));
        asm volatile("s_nop 4" ::: "memory");
        // the loop iteration whose k-tile is the partial one (phys = nk - 1), or -1
        const int tail_it = (t.k % C::BK) != 0 ? nk - 1 - kt0 : -1;
        int kt = 0;
        while (kt < nk) {
            // straight k-tiles need kt + 2 < nk, kt + 2 != tail_it and kt + 1 != tail_it
            int end = nk - 2;
            if (kt <= tail_it - 2)
                end = min(end, tail_it - 2);
            else if (kt == tail_it - 1)
                end = kt;
            for (; kt < end; ++kt) {
                const int stage = kt & 1;
                single_step_fast<false>(f0, f1, acc, stage, 1, 0, 0);
                wait_vmcnt<0>();
                barrier_lds();
                single_step_fast<true>(f1, f0, acc, stage ^ 1, 0, single_lbase(stage),
                                       (uint32_t)phys(kt + 2) * (uint32_t)(C::BK * 2));
            }
            if (kt >= nk)
                break;
            const int stage = kt & 1;
            single_step<false>(f0, f1, acc, stage, 1, 0, 0, false);
            if (kt + 1 < nk)
                stage_ready(kt + 1, t);
            if (kt + 2 == nk)
                on_last_stage();
            single_step<true>(f1, f0, acc, stage ^ 1, 0, kt + 2, stage, kt + 2 < nk);
            ++kt;
        }
        // The accumulators were last written by MFMAs the compiler sees only
        // as assembly: leave the matrix unit's result latency before anything
        // reads them.
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    }

    // ---- global->LDS path -------------------------------------------------
    // Two stages: the loads of k-tile kt+2 can only start once every wave has
    // left stage kt, i.e. at the barrier that ends k-tile kt; they are issued
    // there in one burst.
    template <class Hook>
    __device__ __forceinline__ void run_burst(const TileCtx<C> &t, typename C::Acc (&acc)[C::MI][C::NI], Hook &on_last_stage)
    {
        const int nk = t.nk;
        if (nk == 0) {
            on_last_stage();
            return;
        }
        const int pro = min(C::STAGES - 1, nk);
        for (int s = 0; s < pro; ++s)
            issue_any(s, s, t.k, nk);
        stage_ready(0, t);
        if (C::STAGES - 1 < nk)
            issue_any(C::STAGES - 1, C::STAGES - 1, t.k, nk);
        if (nk == 1)
            on_last_stage();
        Frags f[2];
        load_frags(0, 0, f[0]);
        for (int kt = 0; kt < nk; ++kt) {
            const int stage = kt % C::STAGES;
#pragma unroll
            for (int ks = 0; ks + 1 < C::KSTEPS; ++ks) {
                load_frags(stage, ks + 1, f[(ks + 1) & 1]);
                mma(f[ks & 1], acc);
                interleave_reads_with_mfma();
            }
            if (kt + 1 < nk) {
                // k-tile kt+1's stage: ready, then its first fragments, while
                // the last k-step of kt runs from registers.
                stage_ready(kt + 1, t);
                if (kt + C::STAGES < nk)
                    issue_any(kt + C::STAGES, stage, t.k, nk);
                if (kt + 2 == nk)
                    on_last_stage();
                load_frags((kt + 1) % C::STAGES, 0, f[C::KSTEPS & 1]);
            }
            // one MFMA site for the last k-step keeps the accumulators in one
            // register class across the loop
            mma(f[(C::KSTEPS - 1) & 1], acc);
        }
    }
};

// Epilogue: accumulators -> LDS -> D.
//
// With the B fragment as the MFMA's first operand, lane l of an MB x MB block
// (mi, ni) holds, for q = 0 .. MB/8 - 1, the four consecutive columns
// 8q + 4(l/MB) .. +3 of row l%MB in acc[4q .. 4q+3] (32x32: q = 0..3; 16x16:
// q = 0 only, l/16 = 0..3). Each wave writes those 4-element groups
// as fp32 into a row-major staging tile in LDS (the ring is idle once the k
// loop has ended; LDS stores take the accumulator registers directly); then
// the workgroup stores the tile row by row, 4 elements per lane, converting
// to bf16 there when D is bf16, so each wave writes whole contiguous row
// segments of D. Rows are padded by 16 bytes so the rows a wave writes in
// one instruction fall in distinct LDS banks.
// Only rows < M and columns < N of the problem are written ("Schedules" page,
// section "Domains": an index is stored only while it is in range).
// D is written once and never read back by the kernel, so its vector stores
// are non-temporal: they do not displace the A and B lines that the tiles in
// flight on the same die still share in its L2.
template <class C>
struct Epilogue {
    static constexpr int ES = C::OUT_BF16 ? 2 : 4;   // bytes per element of D
    static constexpr int PITCH = C::BN * 4 + 16;     // staged row, fp32
    // 256-row tiles are staged in two halves to fit LDS
    static constexpr int PASSES = (C::BM * PITCH > 150 * 1024) ? 2 : 1;
    static constexpr int PASS_ROWS = C::BM / PASSES;         // staged rows per pass
    static constexpr int WAVE_ROWS = C::WTM / PASSES;        // a wave's rows per pass
    static constexpr int MI_PASS = C::MI / PASSES;
    static constexpr int CHUNKS_ROW = C::BN / 4;             // 4-element groups per row
    static constexpr int LDS_BYTES = PASS_ROWS * PITCH;
    static constexpr int ITERS = PASS_ROWS * CHUNKS_ROW / C::THREADS; // groups per thread per pass
    static constexpr int BATCH = ITERS < 4 ? ITERS : 4; // staged groups read ahead of their stores
    static_assert(C::MI % PASSES == 0, "passes split the wave's row blocks");
    static_assert(LDS_BYTES <= 150 * 1024, "epilogue staging must fit LDS");
};

// `on_staged` runs once, after the first pass's accumulators are written to
// LDS and before the barrier that publishes them, so an LDS write it makes is
// visible to every wave after that barrier.
template <class C, class Hook>
__device__ __forceinline__ void store_epilogue(const TileCtx<C> &t, const typename C::Acc (&acc)[C::MI][C::NI],
                                               int wm, int wn, int lane, int tid, uint8_t *smem, Hook &&on_staged)
{
    using E = Epilogue<C>;
    // per-tile addresses from opaque indices (see store_epilogue_wide)
    lane = (int)opaque_v((uint32_t)lane);
    tid = (int)opaque_v((uint32_t)tid);
    const int lr = lane % C::MB, lc = (lane / C::MB) * 4;
    constexpr int QS = C::MB * C::MB / 256; // 4-element groups per lane per block
    static_assert(sizeof(typename C::Acc) == QS * 16, "accumulator groups");
    uint8_t *const tile_base = (uint8_t *)t.d + ((int64_t)t.row0 * t.ldd + t.col0) * E::ES;
    // (one wave per SIMD only: with two waves per SIMD the batched form came out
    // slower, its extra registers spilling around the tile loop)
    const bool full = C::WAVES == 4 && C::LOAD_PATH == LOAD_DMA && t.vec_ok && t.vm == C::BM && t.vn == C::BN;
#pragma unroll
    for (int pass = 0; pass < E::PASSES; ++pass) {
        // accumulators of this pass's row blocks -> LDS
#pragma unroll
        for (int m = 0; m < E::MI_PASS; ++m) {
            const int mi = pass * E::MI_PASS + m;
            const int sr = wm * E::WAVE_ROWS + m * C::MB + lr;
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni) {
#pragma unroll
                for (int q = 0; q < QS; ++q) {
                    const int c = wn * C::WTN + ni * C::MB + 8 * q + lc;
                    *(f32x4 *)(smem + sr * E::PITCH + c * 4) =
                        f32x4{acc[mi][ni][4 * q + 0], acc[mi][ni][4 * q + 1], acc[mi][ni][4 * q + 2],
                              acc[mi][ni][4 * q + 3]};
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (pass == 0)
            on_staged();
        barrier_lds();
        // LDS -> D, one 4-element group per lane per step
        constexpr int TOTAL = E::PASS_ROWS * E::CHUNKS_ROW;
        if (full) {
            // Full tile, vector-store rows: no masks, and the staged reads go
            // out BATCH at a time ahead of their conversions and stores, so
            // the LDS latency is paid once per batch instead of once per group
            // (with one wave per SIMD nothing else hides it).
            static_assert(TOTAL == E::ITERS * C::THREADS && E::ITERS % E::BATCH == 0, "store batches");
#pragma unroll
            for (int it0 = 0; it0 < TOTAL / C::THREADS; it0 += E::BATCH) {
                f32x4 v32[E::BATCH];
#pragma unroll
                for (int b = 0; b < E::BATCH; ++b) {
                    const int idx = tid + (it0 + b) * C::THREADS;
                    v32[b] = *(const f32x4 *)(smem + (idx / E::CHUNKS_ROW) * E::PITCH + (idx % E::CHUNKS_ROW) * 16);
                }
#pragma unroll
                for (int b = 0; b < E::BATCH; ++b) {
                    const int idx = tid + (it0 + b) * C::THREADS;
                    const int sr = idx / E::CHUNKS_ROW;
                    const int c = (idx % E::CHUNKS_ROW) * 4;
                    // opaque: formed here, not hoisted into registers held across the passes
                    const int i = (int)opaque_v(
                        (uint32_t)((sr / E::WAVE_ROWS) * C::WTM + pass * E::WAVE_ROWS + (sr % E::WAVE_ROWS)));
                    uint8_t *dst = tile_base + ((int64_t)i * t.ldd + c) * E::ES;
                    if constexpr (C::OUT_BF16) {
                        bf16x4 v;
                        v[0] = (__bf16)v32[b][0];
                        v[1] = (__bf16)v32[b][1];
                        v[2] = (__bf16)v32[b][2];
                        v[3] = (__bf16)v32[b][3];
                        __builtin_nontemporal_store(v, (bf16x4 *)dst);
                    } else {
                        __builtin_nontemporal_store(v32[b], (f32x4 *)dst);
                    }
                }
            }
            if (pass + 1 < E::PASSES)
                barrier_lds();
            continue;
        }
#pragma unroll 2
        for (int idx = tid; idx < TOTAL; idx += C::THREADS) {
            const int sr = idx / E::CHUNKS_ROW;
            const int c = (idx % E::CHUNKS_ROW) * 4;
            // staged row -> tile row
            const int i = (sr / E::WAVE_ROWS) * C::WTM + pass * E::WAVE_ROWS + (sr % E::WAVE_ROWS);
            if (i >= t.vm || c >= t.vn)
                continue;
            const f32x4 v32 = *(const f32x4 *)(smem + sr * E::PITCH + c * 4);
            uint8_t *dst = tile_base + ((int64_t)i * t.ldd + c) * E::ES;
            if constexpr (C::OUT_BF16) {
                bf16x4 v;
                v[0] = (__bf16)v32[0];
                v[1] = (__bf16)v32[1];
                v[2] = (__bf16)v32[2];
                v[3] = (__bf16)v32[3];
                if (t.vec_ok && c + 3 < t.vn) {
                    __builtin_nontemporal_store(v, (bf16x4 *)dst);
                } else {
                    for (int e = 0; e < 4 && c + e < t.vn; ++e)
                        ((__bf16 *)dst)[e] = v[e];
                }
            } else {
                const f32x4 v = v32;
                if (t.vec_ok && c + 3 < t.vn) {
                    __builtin_nontemporal_store(v, (f32x4 *)dst);
                } else {
                    for (int e = 0; e < 4 && c + e < t.vn; ++e)
                        ((float *)dst)[e] = v[e];
                }
            }
        }
        if (pass + 1 < E::PASSES)
            barrier_lds();
    }
}

// Epilogue of the two-waves-per-SIMD kernels: accumulators -> LDS -> D with
// the output type already in LDS (bf16 output). Each lane converts its
// 4-column groups to bf16 (round to nearest even, the same conversion as at a
// store) and writes them into a row-major staging tile, which fits LDS in one
// pass. Then each thread reads all its staged 16-byte chunks ahead of their
// stores, so the LDS latency is paid once instead of once per chunk (the
// fragment and accumulator registers are free by then).
// Full tiles with 16-byte-aligned rows store whole chunks with no masks; edge
// tiles store only rows < M and columns < N.
template <class C>
struct WideEpilogue {
    static constexpr int ES = C::OUT_BF16 ? 2 : 4;                       // bytes per element of D
    static constexpr int PITCH = C::BN * ES + 16;                        // staged row, padded
    static constexpr int PASSES = (C::BM * PITCH > 150 * 1024) ? 2 : 1;
    static constexpr int PASS_ROWS = C::BM / PASSES;
    static constexpr int WAVE_ROWS = C::WTM / PASSES;
    static constexpr int MI_PASS = C::MI / PASSES;
    static constexpr int CHUNK = 16 / ES;                                // elements per 16-byte chunk
    static constexpr int CHUNKS_ROW = C::BN / CHUNK;
    static constexpr int ITERS = PASS_ROWS * CHUNKS_ROW / C::THREADS;    // chunks per thread per pass
    // every chunk read ahead of its store (8 at a time measured 1-3% slower with
    // two waves per SIMD); at most 16 (64 registers) at a time
    static constexpr int BATCH = ITERS < 16 ? ITERS : 16;
    static constexpr int LDS_BYTES = PASS_ROWS * PITCH;
    static_assert(C::MB == 16 && C::MI % PASSES == 0, "16x16 blocks, passes split the row blocks");
    static_assert(PASS_ROWS * CHUNKS_ROW == ITERS * C::THREADS, "whole chunks per thread");
    static_assert(LDS_BYTES <= 150 * 1024, "staging must fit LDS");
};

// `on_staged` runs once, after the first pass's values are in LDS and before
// the barrier that publishes them.
template <class C, class Hook>
__device__ __forceinline__ void store_epilogue_wide(const TileCtx<C> &t, const typename C::Acc (&acc)[C::MI][C::NI],
                                                    int wm, int wn, int lane, int tid, uint8_t *smem,
                                                    Hook &&on_staged)
{
    using E = WideEpilogue<C>;
    // The thread's staging and store addresses are formed here, per tile,
    // from indices the compiler cannot see through: hoisted out of the tile
    // loop they would stay live across the k loop, where every register is
    // taken, and go to scratch.
    lane = (int)opaque_v((uint32_t)lane);
    tid = (int)opaque_v((uint32_t)tid);
    const int lr = lane % 16, lc = (lane / 16) * 4;
    uint8_t *const tile_base = (uint8_t *)t.d + ((int64_t)t.row0 * t.ldd + t.col0) * E::ES;
    const bool full = t.vec_ok && t.vm == C::BM && t.vn == C::BN;
#pragma unroll
    for (int pass = 0; pass < E::PASSES; ++pass) {
        // this pass's accumulators, converted, -> LDS
#pragma unroll
        for (int m = 0; m < E::MI_PASS; ++m) {
            const int mi = pass * E::MI_PASS + m;
            const int sr = wm * E::WAVE_ROWS + m * 16 + lr;
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni) {
                const int c = wn * C::WTN + ni * 16 + lc;
                uint8_t *dst = smem + sr * E::PITCH + c * E::ES;
                const typename C::Acc &v = acc[mi][ni];
                if constexpr (C::OUT_BF16) {
                    bf16x4 h;
                    h[0] = (__bf16)v[0];
                    h[1] = (__bf16)v[1];
                    h[2] = (__bf16)v[2];
                    h[3] = (__bf16)v[3];
                    *(bf16x4 *)dst = h;
                } else {
                    *(f32x4 *)dst = f32x4{v[0], v[1], v[2], v[3]};
                }
                // one block at a time: accumulators held in AGPRs are read
                // into VGPRs only as each block is staged
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (pass == 0)
            on_staged();
        barrier_lds();
        // LDS -> D: the chunks read BATCH at a time ahead of their stores
#pragma unroll
        for (int it0 = 0; it0 < E::ITERS; it0 += E::BATCH) {
            u32x4 chunk[E::BATCH];
#pragma unroll
            for (int b = 0; b < E::BATCH; ++b) {
                const int idx = tid + (it0 + b) * C::THREADS;
                chunk[b] = *(const u32x4 *)(smem + (idx / E::CHUNKS_ROW) * E::PITCH + (idx % E::CHUNKS_ROW) * 16);
            }
#pragma unroll
            for (int b = 0; b < E::BATCH; ++b) {
                const int idx = tid + (it0 + b) * C::THREADS;
                const int sr = idx / E::CHUNKS_ROW;
                const int i = (sr / E::WAVE_ROWS) * C::WTM + pass * E::WAVE_ROWS + (sr % E::WAVE_ROWS);
                const int c = (idx % E::CHUNKS_ROW) * E::CHUNK;
                uint8_t *dst = tile_base + ((int64_t)i * t.ldd + c) * E::ES;
                if (full) {
                    __builtin_nontemporal_store(chunk[b], (u32x4 *)dst);
                } else if (i < t.vm && c < t.vn) {
                    if (t.vec_ok && c + E::CHUNK <= t.vn) {
                        __builtin_nontemporal_store(chunk[b], (u32x4 *)dst);
                    } else {
                        // the row's last partial chunk (or unaligned rows): element by element
                        const u32x4 w = chunk[b];
                        for (int e = 0; e < E::CHUNK && c + e < t.vn; ++e) {
                            if constexpr (C::OUT_BF16)
                                ((uint16_t *)dst)[e] = (uint16_t)(w[e / 2] >> (16 * (e % 2)));
                            else
                                ((uint32_t *)dst)[e] = w[e];
                        }
                    }
                }
            }
        }
        if (pass + 1 < E::PASSES)
            barrier_lds();
    }
}

// bf16 D of the 16x16 barrier-hand-off kernels, staged per wave: each wave
// turns one 16-row block of its wave tile at a time around in a private LDS
// area of its own (beside the ring, so the next tile's first stages can load
// meanwhile) and stores it as whole rows. Converted to bf16 (round to nearest
// even, the same as a store would) and paired up across lanes (below), the
// block row's columns go to the wave's area in 16-byte chunks; each lane then
// reads 16-byte chunks back, WTN * 2 / 16 to a row, and one store writes
// 64 / (WTN * 2 / 16) rows x WTN * 2 contiguous bytes. No workgroup barrier
// is needed: only the wave itself uses its area, and a wave's LDS operations
// are performed in order. Only rows < M and columns < N are written (the
// element-wise path for a chunk that crosses column N or a row that is not
// 16-byte aligned).
template <class C>
struct WaveEpilogue {
    static constexpr int ROW_BYTES = C::WTN * 2;                // a staged row of bf16 D
    static constexpr int AREA = C::MB * ROW_BYTES;              // one wave's area
    static constexpr int LDS_BYTES = C::WAVES * AREA;
    static constexpr int CHUNKS_ROW = C::WTN * 2 / 16;          // 16-byte chunks per wave-tile row
    static constexpr int ROWS = 64 / CHUNKS_ROW;                // rows per read (one chunk per lane)
    static constexpr int READS = C::MB / ROWS;                  // reads (and stores) per row block
    static_assert(C::MB == 16 && C::OUT_BF16 && 64 % CHUNKS_ROW == 0 && C::MB % ROWS == 0, "wave-staged bf16 D");
    static_assert(C::NI % 2 == 0 && CHUNKS_ROW == 2 * C::NI, "blocks staged in pairs");
    static_assert(C::MI * READS == C::BM * C::BN * 2 / 16 / C::THREADS, "every thread stores the same count");
    // Chunk c of staged row r sits at position c ^ (r mod CHUNKS_ROW). With
    // it both the 16-byte writes below (16 rows, one chunk per 16 lanes) and
    // the 16-byte reads (ROWS rows, CHUNKS_ROW chunks each) measure
    // conflict-free with the LDS bank conflict counter; a row pitch padded by
    // 16 bytes, the usual remedy, leaves the reads at 4 conflict cycles each.
    static __device__ __forceinline__ int pos(int r, int c) { return c ^ (r & (CHUNKS_ROW - 1)); }
};

// The bf16 bits of two fp32 values (round to nearest even), lo in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2 h;
    h[0] = (__bf16)lo;
    h[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, h);
}

// D of a full wave tile, staged per wave in 16-row slices through LDS and
// stored as 16-byte chunks. A lane holds 4 consecutive columns of one row of
// each 16x16 block (lane l: row l % 16, columns 4 (l / 16) ..): two
// v_permlane16_swap per pair of neighbouring blocks give every lane 8
// consecutive columns (16-lane group g: block ni + (g & 1), columns
// 8 (g >> 1) ..), which it writes to LDS in one 16-byte store.
template <class C>
__device__ __forceinline__ void store_epilogue_wave(const TileCtx<C> &t, const typename C::Acc (&acc)[C::MI][C::NI],
                                                    int wm, int wn, int lane, int wave, uint8_t *area_base)
{
    using E = WaveEpilogue<C>;
    lane = (int)opaque_v((uint32_t)lane);
    uint8_t *const area = area_base + wave * E::AREA;
    const int lr = lane % 16, g = lane / 16;
    const int rr = lane / E::CHUNKS_ROW, cc = lane % E::CHUNKS_ROW; // this lane's chunk of a read
    const int row = wm * C::WTM + rr, col = wn * C::WTN + cc * 8;     // in the tile
    uint8_t *const base = (uint8_t *)t.d + ((int64_t)(t.row0 + row) * t.ldd + t.col0 + col) * 2;
    const bool full = t.vec_ok && t.vm == C::BM && t.vn == C::BN;
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi) {
#pragma unroll
        for (int ni = 0; ni < C::NI; ni += 2) {
            const typename C::Acc &x = acc[mi][ni], &y = acc[mi][ni + 1];
            // groups 0..3 end up with columns 0-7 of x, 0-7 of y, 8-15 of x, 8-15 of y
            const auto s0 = __builtin_amdgcn_permlane16_swap(pack_bf16x2(x[0], x[1]), pack_bf16x2(y[0], y[1]),
                                                             false, false);
            const auto s1 = __builtin_amdgcn_permlane16_swap(pack_bf16x2(x[2], x[3]), pack_bf16x2(y[2], y[3]),
                                                             false, false);
            const u32x4 w = {s0[0], s1[0], s0[1], s1[1]};
            const int c = 2 * (ni + (g & 1)) + (g >> 1);
            *(u32x4 *)(area + lr * E::ROW_BYTES + (E::pos(lr, c) << 4)) = w;
        }
        wave_lds_exchange();
        u32x4 chunk[E::READS];
#pragma unroll
        for (int j = 0; j < E::READS; ++j) {
            const int r = j * E::ROWS + rr;
            chunk[j] = *(const u32x4 *)(area + r * E::ROW_BYTES + (E::pos(r, cc) << 4));
        }
        wave_lds_exchange();
#pragma unroll
        for (int j = 0; j < E::READS; ++j) {
            uint8_t *const dst = base + ((int64_t)(mi * C::MB + j * E::ROWS) * t.ldd) * 2;
            if (full) {
                __builtin_nontemporal_store(chunk[j], (u32x4 *)dst);
            } else {
                const int i = row + mi * C::MB + j * E::ROWS;
                if (i < t.vm && col < t.vn) {
                    if (t.vec_ok && col + 8 <= t.vn) {
                        __builtin_nontemporal_store(chunk[j], (u32x4 *)dst);
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (col + e < t.vn)
                                ((uint16_t *)dst)[e] = (uint16_t)(chunk[j][e / 2] >> (16 * (e % 2)));
                    }
                }
            }
        }
    }
}

// fp32 D of the 8-wave 16x16 barrier-hand-off kernels, staged per wave like
// bf16 D above, in 8-row halves of each 16-row block (a whole fp32 block row
// per wave beside the ring would need all 160 KiB of LDS). A lane's 4 fp32
// of a block are one 16-byte chunk already; the lanes of the half's rows write
// them, then every lane reads 16-byte chunks back, WTN * 4 / 16 to a row.
// Chunk c of staged row r sits at c ^ (r mod chunks per row): with it the
// half-wave 16-byte writes and the 16-byte reads both measure conflict-free
// with the LDS bank conflict counter. Only rows < M and columns < N are
// written.
template <class C>
struct WaveEpilogueF32 {
    static constexpr int ROW_BYTES = C::WTN * 4;                // a staged row of fp32 D
    static constexpr int HALF = C::MB / 2;                      // rows staged at a time
    static constexpr int AREA = HALF * ROW_BYTES;               // one wave's area
    static constexpr int LDS_BYTES = C::WAVES * AREA;
    static constexpr int CHUNKS_ROW = C::WTN * 4 / 16;          // 16-byte chunks per wave-tile row
    static constexpr int ROWS = 64 / CHUNKS_ROW;                // rows per read (one chunk per lane)
    static constexpr int READS = HALF / ROWS;                   // reads (and stores) per half
    static_assert(C::MB == 16 && !C::OUT_BF16 && 64 % CHUNKS_ROW == 0 && HALF % ROWS == 0, "wave-staged fp32 D");
    static_assert(CHUNKS_ROW == 4 * C::NI, "a lane's block chunk: 4 per 16x16 block row");
    static_assert(C::MI * 2 * READS == C::BM * C::BN * 4 / 16 / C::THREADS, "every thread stores the same count");
    static __device__ __forceinline__ int pos(int r, int c) { return c ^ (r & (CHUNKS_ROW - 1)); }
};

template <class C>
__device__ __forceinline__ void store_epilogue_wave_f32(const TileCtx<C> &t,
                                                        const typename C::Acc (&acc)[C::MI][C::NI], int wm, int wn,
                                                        int lane, int wave, uint8_t *area_base)
{
    using E = WaveEpilogueF32<C>;
    lane = (int)opaque_v((uint32_t)lane);
    uint8_t *const area = area_base + wave * E::AREA;
    const int lr = lane % 16, g = lane / 16;
    const int rr = lane / E::CHUNKS_ROW, cc = lane % E::CHUNKS_ROW; // this lane's chunk of a read
    const int row = wm * C::WTM + rr, col = wn * C::WTN + cc * 4;     // in the tile
    uint8_t *const base = (uint8_t *)t.d + ((int64_t)(t.row0 + row) * t.ldd + t.col0 + col) * 4;
    const bool full = t.vec_ok && t.vm == C::BM && t.vn == C::BN;
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (lr / E::HALF == h) {
                const int sr = lr % E::HALF;
#pragma unroll
                for (int ni = 0; ni < C::NI; ++ni)
                    *(f32x4 *)(area + sr * E::ROW_BYTES + (E::pos(sr, 4 * ni + g) << 4)) = acc[mi][ni];
            }
            wave_lds_exchange();
            f32x4 chunk[E::READS];
#pragma unroll
            for (int j = 0; j < E::READS; ++j) {
                const int r = j * E::ROWS + rr;
                chunk[j] = *(const f32x4 *)(area + r * E::ROW_BYTES + (E::pos(r, cc) << 4));
            }
            wave_lds_exchange();
#pragma unroll
            for (int j = 0; j < E::READS; ++j) {
                const int dr = mi * C::MB + h * E::HALF + j * E::ROWS;   // row offset from `row`
                uint8_t *const dst = base + ((int64_t)dr * t.ldd) * 4;
                if (full) {
                    __builtin_nontemporal_store(chunk[j], (f32x4 *)dst);
                } else {
                    const int i = row + dr;
                    if (i < t.vm && col < t.vn) {
                        if (t.vec_ok && col + 4 <= t.vn) {
                            __builtin_nontemporal_store(chunk[j], (f32x4 *)dst);
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (col + e < t.vn)
                                    ((float *)dst)[e] = chunk[j][e];
                        }
                    }
                }
            }
        }
    }
}

template <class C, bool USED>
constexpr int wave_epilogue_lds_bytes()
{
    if constexpr (!USED)
        return 0;
    else if constexpr (C::OUT_BF16)
        return WaveEpilogue<C>::LDS_BYTES;
    else
        return WaveEpilogueF32<C>::LDS_BYTES;
}

template <class C, bool WIDE>
constexpr int epilogue_lds_bytes()
{
    if constexpr (WIDE)
        return WideEpilogue<C>::LDS_BYTES;
    else
        return Epilogue<C>::LDS_BYTES;
}

template <class C>
__global__ __attribute__((amdgpu_flat_work_group_size(C::THREADS, C::THREADS),
                          amdgpu_waves_per_eu(C::WAVES_PER_SIMD, C::WAVES_PER_SIMD)))
void gemm_persistent_kernel(const GemmArgs args_by_value)
{
    (void)args_by_value;
    const KernArgs args = kernel_args();
    const int group_begin = load_group_begin(args, (int)(threadIdx.x & 63));
    // settle the load here, so no wait for it lands inside the tile loop
    // (where it would also wait for the previous tile's stores)
    wait_vmcnt<0>();
    // the two-waves-per-SIMD 16x16 kernels stage bf16 D as bf16 (WideEpilogue);
    // with the barrier hand-off they, and the one-wave-per-SIMD 16x16 kernel,
    // stage it per wave, beside the ring, and load the next tile's first
    // stages during the epilogue (WaveEpilogue; fp32 D of the two-wave ones
    // in half blocks, WaveEpilogueF32)
    constexpr bool WIDE_EPI = C::WAVES == 8 && C::MB == 16 && C::OUT_BF16;
    constexpr bool SINGLE_EPI = C::WAVES == 4 && C::MB == 16 && C::OUT_BF16;
    constexpr bool F32_EPI = C::WAVES == 8 && C::MB == 16 && !C::OUT_BF16;
    constexpr bool PREFETCH = (WIDE_EPI || SINGLE_EPI || F32_EPI) && C::SYNC == SYNC_BARRIER;
    constexpr int EPI_BYTES = PREFETCH ? 0 : epilogue_lds_bytes<C, WIDE_EPI>();
    constexpr int WAVE_EPI_BYTES = wave_epilogue_lds_bytes<C, PREFETCH>();
    constexpr int SMEM_BYTES = (C::LDS_BYTES > EPI_BYTES ? C::LDS_BYTES : EPI_BYTES) + WAVE_EPI_BYTES;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM_BYTES];
    __shared__ int32_t sched_slots[4];
    __shared__ uint32_t stage_flags[6];

    const int tid = threadIdx.x;
    const int wave = uniform(tid >> 6);
    const int lane = tid & 63;
    const bool leader = tid == 0;

    Mainloop<C> ml;
    ml.smem = smem;
    ml.wave = wave;
    ml.lane = lane;
    ml.wm = wave / C::WAVES_N;
    ml.wn = wave % C::WAVES_N;
    ml.setup_fragments();
    ml.sflags = (__attribute__((address_space(3))) uint32_t *)stage_flags;
    ml.stall_ctr = args->counters + CTR_SYNC_STALLS;
    ml.uses0 = ml.uses1 = 0;
    ml.full_excess = C::SYNC != SYNC_BARRIER ? (uint32_t)args->full_excess : 0u;
    ml.broken = false;
    if (tid < 6)
        stage_flags[tid] = 0;
    barrier_lds();

    TileScheduler sched{args->counters, args->total_tiles, args->num_workers, args->round, (int)blockIdx.x,
                        args->schedule, sched_slots, (int)(xcc_id_reg() % NUM_XCD), 0u};
    uint8_t *const trace = args->trace;
    const int total_tiles = args->total_tiles;
    const bool tracing = trace != nullptr;
    const uint64_t t_worker0 = tracing ? realtime() : 0;

    // Request-ahead off (a measurement baseline): no claim before the epilogue.
    const bool claim_late = args->claim_late != 0;
    Claimed cur = sched.first(tid);
    int seq = 0;
    if constexpr (PREFETCH) {
        // Tile i's epilogue overlaps tile i + 1's first loads: once the k loop
        // is done (every wave past its last read of the ring: the barrier
        // below, which also publishes the next claim) the next tile is decoded
        // and both of its first stages are loaded while this tile's D is
        // staged per wave and stored; the next tile then waits for its stage 0
        // only, with this tile's stores still in flight.
        // (the lane index is recomputed where needed: kept live across the k
        // loop it is spilled where no register is spare, and its reload's
        // wait would also wait for the next tile's loads)
        TileCtx<C> tc{};
        if (cur.pos < total_tiles) {
            tc = decode_tile<C>(args, cur.pos, group_begin);
            ml.lane = (int)lane_id();
            ml.setup(tc);
        }
        int pre = -1;
        while (cur.pos < total_tiles) {
            const uint64_t t_tile0 = tracing ? realtime() : 0;
            const uint64_t c_tile0 = tracing ? shader_cycles() : 0;
            typename C::Acc acc[C::MI][C::NI];
#pragma unroll
            for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < C::NI; ++ni)
                    acc[mi][ni] = typename C::Acc{};
            auto claim = [&] {
                if (!claim_late)
                    sched.claim_ahead(leader);
            };
            ml.run(tc, acc, claim, pre);
            if (claim_late)
                sched.claim_ahead(leader);
            sched.stage_next(tid, seq);
            barrier_lds();
            const Claimed next = sched.read_next(cur, seq);
            TileCtx<C> tn{};
            if (next.pos < total_tiles) {
                tn = decode_tile<C>(args, next.pos, group_begin);
                ml.lane = (int)lane_id();
                ml.setup(tn);
                ml.issue_first_two(tn);
            }
            if constexpr (C::OUT_BF16)
                store_epilogue_wave<C>(tc, acc, ml.wm, ml.wn, (int)lane_id(), wave, smem + C::LDS_BYTES);
            else
                store_epilogue_wave_f32<C>(tc, acc, ml.wm, ml.wn, (int)lane_id(), wave, smem + C::LDS_BYTES);
            pre = (tc.vec_ok && tc.vm == C::BM && tc.vn == C::BN) ? Mainloop<C>::STORES : 0;
            if (tracing && leader) {
                TileTrace r;
                r.tile = cur.pos;
                r.claim = cur.claim;
                r.worker = blockIdx.x;
                r.seq = seq;
                r.group = tc.problem;
                r.row0 = tc.row0;
                r.col0 = tc.col0;
                r.xcc_id = xcc_id_reg();
                r.t_start = t_tile0;
                r.t_end = realtime();
                r.cycles = (uint32_t)(shader_cycles() - c_tile0);
                r.pad = 0;
                ((TileTrace *)trace)[cur.pos] = r;
                // (the record's stores are younger still: the next tile's
                // stage-0 wait then waits for a little more, never for less)
            }
            tc = tn;
            cur = next;
            ++seq;
        }
        wait_vmcnt<0>();
    }
    while (!PREFETCH && cur.pos < total_tiles) {
        const uint64_t t_tile0 = tracing ? realtime() : 0;
        const uint64_t c_tile0 = tracing ? shader_cycles() : 0;
        const TileCtx<C> tc = decode_tile<C>(args, cur.pos, group_begin);
        // Every per-lane value of the k loop is formed per tile from a lane
        // index the compiler cannot see through: hoisted out of the tile loop
        // it would stay live across every k loop, where no register is spare,
        // and go to scratch.
        ml.lane = (int)opaque_v((uint32_t)lane);

        typename C::Acc acc[C::MI][C::NI];
#pragma unroll
        for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni)
                acc[mi][ni] = typename C::Acc{};

        ml.setup(tc);
        // The request for the next tile goes out once this tile's last stage
        // is in LDS: its round trip overlaps the last k-tile and the epilogue,
        // and no load wait of this tile is held up by it.
        ml.run(tc, acc, [&] {
            if (!claim_late)
                sched.claim_ahead(leader);
        });
        // every wave has finished reading the ring before it is reused for staging
        barrier_raw();
        // The next tile's claim is resolved while the accumulators are staged
        // (its request went out a k-tile ago) and published by the staging
        // barrier, so no wave waits on it after the stores.
        auto stage = [&] {
            if (!claim_late)
                sched.stage_next(tid, seq);
        };
        if constexpr (WIDE_EPI)
            store_epilogue_wide<C>(tc, acc, ml.wm, ml.wn, lane, tid, smem, stage);
        else
            store_epilogue<C>(tc, acc, ml.wm, ml.wn, lane, tid, smem, stage);

        if (tracing && leader) {
            TileTrace r;
            r.tile = cur.pos;
            r.claim = cur.claim;
            r.worker = blockIdx.x;
            r.seq = seq;
            r.group = tc.problem;
            r.row0 = tc.row0;
            r.col0 = tc.col0;
            r.xcc_id = xcc_id_reg();
            r.t_start = t_tile0;
            r.t_end = realtime();
            r.cycles = (uint32_t)(shader_cycles() - c_tile0);
            r.pad = 0;
            ((TileTrace *)trace)[cur.pos] = r;
        }
        // The D stores stay in flight into the next tile's prologue (the first
        // stage wait covers them: loads complete in issue order and an older
        // store only makes a vmcnt wait stricter). Staging reads must be done
        // in every wave before the next tile's loads overwrite the ring.
        wait_lgkmcnt0();
        barrier_raw();
        if (claim_late) {
            // ask only now, and wait for the answer (resolved and published
            // through LDS with a barrier)
            sched.claim_ahead(leader);
            cur = sched.next(cur, tid, seq);
        } else {
            cur = sched.read_next(cur, seq);
        }
        ++seq;
    }

    if (tracing && leader) {
        WorkerTrace r;
        r.t_start = t_worker0;
        r.t_end = realtime();
        r.tiles = seq;
        r.worker = blockIdx.x;
        r.hw_id = hw_id_reg();
        r.xcc_id = xcc_id_reg();
        ((WorkerTrace *)(trace + (size_t)total_tiles * sizeof(TileTrace)))[blockIdx.x] = r;
    }
    sched.finish(leader);
}

} // namespace pts
