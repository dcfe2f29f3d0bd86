// Host side of the C ABI declared in include/pts_gemm.h: plan validation,
// tile-space construction, plan-owned device memory, and kernel launches.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#define PTS_MAX_GROUPS GEMM_MAX_GROUPS
#include "pts_gemm.h"

#include "device/aux_kernels.h"
#include "device/gemm_kernel.h"

namespace {

thread_local std::string g_last_error;

gemm_status fail(gemm_status s, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

gemm_status hip_fail(hipError_t e, const char *what)
{
    return fail(GEMM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// One compiled kernel configuration.
struct KernelEntry {
    int bm, bn, bk, stages;
    bool out_bf16;
    int load_path;
    int waves;
    int mfma;
    int sync;
    const void *fn;
    int lds_bytes;
};

template <int BM, int BN, int BK, int S, bool BF16, int LP = pts::LOAD_DMA, int WM = 2, int WN = 2, int MB = 32,
          int SYNC = pts::SYNC_BARRIER>
KernelEntry make_entry()
{
    using C = pts::GemmConfig<BM, BN, BK, S, BF16, LP, WM, WN, MB, SYNC>;
    return KernelEntry{BM, BN, BK, S, BF16, LP, C::WAVES, MB, SYNC, (const void *)&pts::gemm_persistent_kernel<C>,
                       C::LDS_BYTES};
}

const std::vector<KernelEntry> &kernel_table()
{
    static const std::vector<KernelEntry> table = {
        // The first entry of a (tile, output type) pair is its default. For
        // 256x256 that is 8 waves (two per SIMD) with global->LDS loads and
        // 16x16x32 MFMAs: the fastest measured on 8192^3 (one wave per SIMD
        // leaves the LDS reads latency-bound; the 16x16 instruction holds a
        // higher clock than the 32x32 one under the power limit).
        make_entry<256, 256, 64, 2, true, pts::LOAD_DMA, 2, 4, 16>(),
        make_entry<256, 256, 64, 2, false, pts::LOAD_DMA, 2, 4, 16>(),
        // one wave per SIMD, 128x128 each (the hand-laid k loop)
        make_entry<256, 256, 64, 2, true, pts::LOAD_DMA, 2, 2, 16>(),
        make_entry<256, 256, 64, 2, false, pts::LOAD_DMA, 2, 2, 16>(),
        // 256x128: the default kernel on half the columns, its 8 waves as 4x2
        // (64x64 each: fewer fragment reads per MFMA than 2x4's 128x32, +5%
        // at 8192^3), for problems with too few 256x256 tiles
        make_entry<256, 128, 64, 2, true, pts::LOAD_DMA, 4, 2, 16>(),
        make_entry<256, 128, 64, 2, false, pts::LOAD_DMA, 4, 2, 16>(),
        make_entry<128, 128, 64, 2, true>(),  make_entry<128, 128, 64, 2, false>(),
        make_entry<64, 64, 64, 2, true>(),    make_entry<64, 64, 64, 2, false>(),
        // the default kernel with the stage hand-off through LDS arrive counters
        make_entry<256, 256, 64, 2, true, pts::LOAD_DMA, 2, 4, 16, pts::SYNC_FUSED>(),
        make_entry<256, 256, 64, 2, false, pts::LOAD_DMA, 2, 4, 16, pts::SYNC_FUSED>(),
        make_entry<256, 256, 64, 2, true, pts::LOAD_DMA, 2, 4, 16, pts::SYNC_MERGED>(),
        make_entry<256, 256, 64, 2, false, pts::LOAD_DMA, 2, 4, 16, pts::SYNC_MERGED>(),
    };
    return table;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

} // namespace

// Everything a run needs except device memory: built and validated on the
// host by build_core, which allocates nothing on the device.
struct PlanCore {
    int device = 0;
    int32_t group_count = 0;
    gemm_shape shapes[GEMM_MAX_GROUPS];       // ld values resolved, in tile order
    int32_t order[GEMM_MAX_GROUPS];           // tile-order slot -> descriptor problem index
    pts::GroupDesc groups[GEMM_MAX_GROUPS];   // the device table's contents, in tile order
    int32_t dtype_d = GEMM_DTYPE_F32;
    int32_t schedule = GEMM_SCHEDULE_STATIC;
    int32_t round = 0;
    int32_t k_phase_row = 0; // k-tiles between tile rows' k starts in a die's block
    int32_t full_excess = 0; // test only (GEMM_FLAG_DEBUG_STAGE_FLAG_STALL)
    int32_t claim_late = 0;  // GEMM_FLAG_CLAIM_AFTER_TILE
    KernelEntry kernel{};
    int64_t total_tiles = 0;
    int32_t workers = 0;
};

struct gemm_plan {
    PlanCore core;
    void *d_mem = nullptr;                  // the one device allocation (counters, then the group table)
    pts::GroupDesc *d_groups = nullptr;
    uint32_t *d_counters = nullptr;
    void *trace = nullptr;
    size_t trace_bytes = 0;
};

namespace {

// Output tile for GEMM_TILE_AUTO: the first of 256x256, 256x128, 128x128
// whose tile count (over all problems) reaches 55% of the compute units, else
// 64x64. Larger tiles read less memory per flop, but a problem with too few of
// them leaves most of the chip idle for the whole run; on bf16 squares from
// 1024^3 to 6144^3 this rule picks the fastest of the four tiles.
void pick_auto_tile(const gemm_desc *desc, int cus, int &tm, int &tn)
{
    static const int cand[3][2] = {{256, 256}, {256, 128}, {128, 128}};
    for (const auto &c : cand) {
        int64_t tiles = 0;
        for (int g = 0; g < desc->group_count; ++g) {
            const gemm_shape &s = desc->shapes[g];
            if (s.m > 0 && s.n > 0)
                tiles += ((s.m + c[0] - 1) / c[0]) * ((s.n + c[1] - 1) / c[1]);
        }
        if (20 * tiles >= 11 * (int64_t)cus) {
            tm = c[0];
            tn = c[1];
            return;
        }
    }
    tm = tn = 64;
}

// Tile rows per band of a problem's tile order (the device's raster_tile). A
// band of 8 tile rows walks every column for each group of 8 tile rows, so B
// is read again per group unless the memory-side cache (256 MiB on MI355X,
// shared by the dies) keeps it. When B takes more than half of that cache the
// band widens to the most tile rows, a multiple of 8 up to 64, whose A panels
// fit in three quarters of it: they stay cached while B streams past once per
// band. At 16384 x 16384 x 8192 (48 rows): +6.5%; 32 rows +5%, 24 +4%, 16
// +1.5%, 64 (A band 256 MiB) +1.5%. Where B fits, the narrow band (0.5-0.9%
// better there).
constexpr int64_t WIDE_BAND_B_BYTES = (int64_t)128 << 20;
constexpr int64_t BAND_A_BYTES = (int64_t)192 << 20;
static int32_t band_rows_for(const gemm_shape &s, int tile_m)
{
    if ((int64_t)s.n * s.k * 2 <= WIDE_BAND_B_BYTES || s.k == 0)
        return 8;
    const int64_t rows = BAND_A_BYTES / ((int64_t)tile_m * s.k * 2) / 8 * 8;
    return (int32_t)std::min<int64_t>(64, std::max<int64_t>(8, rows));
}

// Validate a descriptor and lay out its tile space (the plan's host part).
// Allocates no device memory; needs the current HIP device for the compute
// unit count and the kernel's occupancy.
gemm_status build_core(const gemm_desc *desc, PlanCore &core)
{
    if (desc == nullptr)
        return fail(GEMM_ERR_INVALID_VALUE, "desc is NULL");
    if (desc->group_count < 1)
        return fail(GEMM_ERR_INVALID_VALUE, "group_count must be >= 1 (got %d)", desc->group_count);
    if (desc->group_count > GEMM_MAX_GROUPS)
        return fail(GEMM_ERR_UNSUPPORTED, "group_count %d exceeds GEMM_MAX_GROUPS (%d)", desc->group_count,
                    GEMM_MAX_GROUPS);
    if (desc->shapes == nullptr)
        return fail(GEMM_ERR_INVALID_VALUE, "shapes is NULL");
    if (desc->layout_a != GEMM_ROW_MAJOR || desc->layout_b != GEMM_COL_MAJOR || desc->layout_d != GEMM_ROW_MAJOR)
        return fail(GEMM_ERR_UNSUPPORTED, "layouts must be A row-major, B column-major, D row-major");
    if (desc->dtype_a != GEMM_DTYPE_BF16 || desc->dtype_b != GEMM_DTYPE_BF16 || desc->dtype_acc != GEMM_DTYPE_F32)
        return fail(GEMM_ERR_UNSUPPORTED, "A and B must be bf16 and the accumulator fp32");
    if (desc->dtype_d != GEMM_DTYPE_F32 && desc->dtype_d != GEMM_DTYPE_BF16)
        return fail(GEMM_ERR_UNSUPPORTED, "D must be fp32 or bf16");
    if (desc->schedule < GEMM_SCHEDULE_STATIC || desc->schedule > GEMM_SCHEDULE_NONPERSISTENT)
        return fail(GEMM_ERR_INVALID_VALUE,
                    "schedule must be static (0), dynamic (1), dynamic per XCD (2) or non-persistent (3)");
    if (desc->schedule == GEMM_SCHEDULE_NONPERSISTENT && desc->num_workers > 0)
        return fail(GEMM_ERR_INVALID_VALUE, "the non-persistent schedule launches one workgroup per tile");
    if (desc->num_workers < 0)
        return fail(GEMM_ERR_INVALID_VALUE, "num_workers must be >= 0");
    if ((desc->flags & ~(GEMM_FLAG_STAGE_FLAGS_FUSED | GEMM_FLAG_STAGE_FLAGS_MERGED |
                         GEMM_FLAG_PROBLEM_ORDER_AS_GIVEN | GEMM_FLAG_DEBUG_STAGE_FLAG_STALL |
                         GEMM_FLAG_CLAIM_AFTER_TILE)) != 0 ||
        (desc->flags & (GEMM_FLAG_STAGE_FLAGS_FUSED | GEMM_FLAG_STAGE_FLAGS_MERGED)) ==
            (GEMM_FLAG_STAGE_FLAGS_FUSED | GEMM_FLAG_STAGE_FLAGS_MERGED))
        return fail(GEMM_ERR_UNSUPPORTED, "unknown flags 0x%x (the two stage-flag layouts exclude each other)",
                    desc->flags);
    const uint32_t sync_flags = desc->flags & (GEMM_FLAG_STAGE_FLAGS_FUSED | GEMM_FLAG_STAGE_FLAGS_MERGED);
    const int32_t sync = sync_flags == GEMM_FLAG_STAGE_FLAGS_FUSED    ? pts::SYNC_FUSED
                         : sync_flags == GEMM_FLAG_STAGE_FLAGS_MERGED ? pts::SYNC_MERGED
                                                                      : pts::SYNC_BARRIER;
    if ((desc->flags & GEMM_FLAG_DEBUG_STAGE_FLAG_STALL) != 0 && sync == pts::SYNC_BARRIER)
        return fail(GEMM_ERR_INVALID_VALUE, "the stall test flag needs a stage-flag layout");
    const bool auto_tile = desc->tile_m == GEMM_TILE_AUTO || desc->tile_n == GEMM_TILE_AUTO;
    if (auto_tile && (desc->tile_m != desc->tile_n || desc->tile_k != 0 || desc->stages != 0 ||
                      desc->load_path != 0 || desc->waves != 0 || desc->mfma != 0 || sync != pts::SYNC_BARRIER))
        return fail(GEMM_ERR_INVALID_VALUE,
                    "an automatic tile takes no other kernel choice (tile_m = tile_n = GEMM_TILE_AUTO, the rest 0)");
    // the device is queried only once everything checkable without it has passed
    int cus = 0;
    auto query_device = [&]() -> hipError_t {
        hipError_t qe = hipGetDevice(&core.device);
        if (qe == hipSuccess)
            qe = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, core.device);
        return qe;
    };
    int tm = desc->tile_m == 0 ? 256 : desc->tile_m;
    int tn = desc->tile_n == 0 ? 256 : desc->tile_n;
    if (auto_tile) {
        const hipError_t qe = query_device();
        if (qe != hipSuccess)
            return hip_fail(qe, "querying the compute unit count");
        pick_auto_tile(desc, cus, tm, tn);
    }
    const bool out_bf16 = desc->dtype_d == GEMM_DTYPE_BF16;
    const KernelEntry *entry = nullptr;
    if (desc->tile_k < 0 || desc->stages < 0 || desc->load_path < 0 || desc->load_path > 1 ||
        (desc->waves != 0 && desc->waves != 4 && desc->waves != 8) ||
        (desc->mfma != 0 && desc->mfma != 16 && desc->mfma != 32))
        return fail(GEMM_ERR_INVALID_VALUE,
                    "tile_k and stages must be >= 0, load_path 0 or 1, waves 0, 4 or 8, mfma 0, 16 or 32");
    for (const KernelEntry &k : kernel_table())
        if (k.bm == tm && k.bn == tn && k.out_bf16 == out_bf16 && (desc->tile_k == 0 || k.bk == desc->tile_k) &&
            (desc->stages == 0 || k.stages == desc->stages) &&
            (desc->load_path == 0 || k.load_path == desc->load_path - 1) &&
            (desc->waves == 0 || k.waves == desc->waves) && (desc->mfma == 0 || k.mfma == desc->mfma) &&
            k.sync == sync) {
            entry = &k;
            break;
        }
    if (entry == nullptr && sync != pts::SYNC_BARRIER)
        return fail(GEMM_ERR_UNSUPPORTED, "stage flags are built for the 8-wave 16x16 two-stage 256x256 kernel only");
    if (entry == nullptr)
        return fail(GEMM_ERR_UNSUPPORTED, "tile %dx%d (k %d, %d stages, load path %d, %d waves, mfma %d) is not built",
                    tm, tn, desc->tile_k, desc->stages, desc->load_path, desc->waves, desc->mfma);

    pts::GroupDesc groups[GEMM_MAX_GROUPS];
    gemm_shape shapes[GEMM_MAX_GROUPS];
    int64_t tiles = 0;
    for (int g = 0; g < desc->group_count; ++g) {
        gemm_shape s = desc->shapes[g];
        if (s.m < 0 || s.n < 0 || s.k < 0 || s.m > INT32_MAX || s.n > INT32_MAX || s.k > INT32_MAX)
            return fail(GEMM_ERR_INVALID_VALUE, "problem %d: m, n, k must be in [0, 2^31)", g);
        if (s.lda == 0) s.lda = s.k;
        if (s.ldb == 0) s.ldb = s.k;
        if (s.ldd == 0) s.ldd = s.n;
        if (s.lda < s.k || s.ldb < s.k || s.ldd < s.n || s.lda < 0 || s.ldb < 0 || s.ldd < 0)
            return fail(GEMM_ERR_INVALID_VALUE, "problem %d: leading dimension smaller than the packed extent", g);
        if ((s.lda % 8) != 0 || (s.ldb % 8) != 0)
            return fail(GEMM_ERR_INVALID_VALUE,
                        "problem %d: lda (%lld) and ldb (%lld) must be multiples of 8 elements (16-byte rows)", g,
                        (long long)s.lda, (long long)s.ldb);
        // load offsets inside one tile are 32-bit byte offsets from the tile's origin
        if ((int64_t)(tm - 1) * s.lda * 2 + (s.k + 8) * 2 >= ((int64_t)1 << 31) ||
            (int64_t)(tn - 1) * s.ldb * 2 + (s.k + 8) * 2 >= ((int64_t)1 << 31))
            return fail(GEMM_ERR_UNSUPPORTED, "problem %d: lda/ldb too large for 32-bit tile offsets", g);
        shapes[g] = s;
        pts::GroupDesc &gd = groups[g];
        gd.m = (int32_t)s.m;
        gd.n = (int32_t)s.n;
        gd.k = (int32_t)s.k;
        gd.tiles_n = (int32_t)ceil_div(s.n, tn);
        gd.tile_begin = 0;
        gd.num_k_tiles = (int32_t)ceil_div(s.k, entry->bk);
        gd.index = g;
        gd.band_rows = band_rows_for(s, tm);
        gd.lda = s.lda;
        gd.ldb = s.ldb;
        gd.ldd = s.ldd;
        if (s.m > 0 && s.n > 0)
            tiles += ceil_div(s.m, tm) * ceil_div(s.n, tn);
        if (tiles >= (int64_t)1 << 27)
            return fail(GEMM_ERR_UNSUPPORTED, "more than 2^27 output tiles");
    }
    // Tile order: deepest problems first (a tile's cost grows with its
    // k-tiles), so the long tiles start early and the short ones fill the end
    // of the run; the descriptor's order on request. Positions are then
    // counted in that order (the prefix sums of "Schedules", section
    // "Dynamic Domains").
    core.group_count = desc->group_count;
    for (int g = 0; g < desc->group_count; ++g)
        core.order[g] = g;
    if ((desc->flags & GEMM_FLAG_PROBLEM_ORDER_AS_GIVEN) == 0)
        std::stable_sort(core.order, core.order + desc->group_count,
                         [&](int32_t x, int32_t y) { return groups[x].num_k_tiles > groups[y].num_k_tiles; });
    int64_t begin = 0;
    for (int i = 0; i < desc->group_count; ++i) {
        const int32_t p = core.order[i];
        core.groups[i] = groups[p];
        core.groups[i].tile_begin = (int32_t)begin;
        core.shapes[i] = shapes[p];
        if (shapes[p].m > 0 && shapes[p].n > 0)
            begin += ceil_div(shapes[p].m, tm) * ceil_div(shapes[p].n, tn);
    }

    hipError_t e = auto_tile ? hipSuccess : query_device();
    if (e != hipSuccess)
        return hip_fail(e, "querying the compute unit count");
    int occ = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, entry->fn, entry->waves * 64, 0);
    if (e != hipSuccess)
        return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
    if (occ < 1)
        return fail(GEMM_ERR_UNSUPPORTED, "kernel cannot be resident on this device");
    const int64_t resident = (int64_t)cus * occ;
    int64_t workers = desc->num_workers > 0 ? desc->num_workers : std::min<int64_t>(tiles, resident);
    int64_t round = workers;
    if (desc->schedule == GEMM_SCHEDULE_NONPERSISTENT) {
        workers = tiles;
        round = std::min<int64_t>(tiles, resident);
    }
    if (tiles == 0)
        workers = round = 0;
    if (workers > 65535 * 16)
        return fail(GEMM_ERR_INVALID_VALUE, "num_workers too large");

    core.dtype_d = desc->dtype_d;
    core.schedule = desc->schedule;
    core.kernel = *entry;
    core.total_tiles = tiles;
    core.workers = (int32_t)workers;
    core.round = (int32_t)round;
    // Tile rows of a die's block start their k loops 2 k-tiles apart for runs
    // of up to 4 rounds of the resident workgroups (measured: +0.7-0.9% at 4
    // rounds; -2.5 to -4.6% for the dynamic schedules at 9 and 16, where the
    // workers of a die drift apart). A function of the problem set and the
    // device only, so every schedule and worker count sums in the same order.
    core.k_phase_row = tiles <= 4 * resident ? 2 : 0;
    core.full_excess = (desc->flags & GEMM_FLAG_DEBUG_STAGE_FLAG_STALL) != 0 ? 1 : 0;
    core.claim_late = (desc->flags & GEMM_FLAG_CLAIM_AFTER_TILE) != 0 ? 1 : 0;
    return GEMM_OK;
}

// The kernel argument block of one run: per-run operand checks, then the
// plan's values. `groups` and `counters` are the device table and counter
// block the kernel reads.
gemm_status fill_args(const PlanCore &core, const gemm_operands *ops, pts::GemmArgs &args)
{
    if (ops == nullptr)
        return fail(GEMM_ERR_INVALID_VALUE, "ops is NULL");
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    if (dev != core.device)
        return fail(GEMM_ERR_INVALID_VALUE, "plan was created on device %d, current device is %d", core.device, dev);
    memset(&args, 0, sizeof args);
    const size_t esize_d = core.dtype_d == GEMM_DTYPE_BF16 ? 2 : 4;
    for (int g = 0; g < core.group_count; ++g) {
        // slot g of the tile order holds descriptor problem p
        const int p = core.order[g];
        const gemm_shape &s = core.shapes[g];
        const gemm_operands &o = ops[p];
        const bool has_tiles = s.m > 0 && s.n > 0;
        if (has_tiles) {
            if (o.d == nullptr || (s.k > 0 && (o.a == nullptr || o.b == nullptr)))
                return fail(GEMM_ERR_INVALID_VALUE, "problem %d: NULL operand pointer", p);
            if (s.k > 0 && (((uintptr_t)o.a % 16) != 0 || ((uintptr_t)o.b % 16) != 0))
                return fail(GEMM_ERR_INVALID_VALUE, "problem %d: A and B must be 16-byte aligned", p);
            if (((uintptr_t)o.d % esize_d) != 0)
                return fail(GEMM_ERR_INVALID_VALUE, "problem %d: D must be element aligned", p);
        }
        args.a[g] = (const uint16_t *)o.a;
        args.b[g] = (const uint16_t *)o.b;
        args.d[g] = o.d;
        // rows of D start 16-byte aligned: the epilogue may store whole 16-byte chunks
        if (((uintptr_t)o.d % 16) == 0 && ((size_t)s.ldd * esize_d) % 16 == 0)
            args.d_vec_ok |= (uint64_t)1 << g;
    }
    args.group_count = core.group_count;
    args.total_tiles = (int32_t)core.total_tiles;
    args.num_workers = core.workers;
    args.schedule = core.schedule;
    args.round = core.round;
    args.full_excess = core.full_excess;
    args.k_phase_row = core.k_phase_row;
    args.claim_late = core.claim_late;
    return GEMM_OK;
}

gemm_status launch_gemm(const PlanCore &core, pts::GemmArgs &args, void *stream)
{
    void *kargs[] = {&args};
    hipError_t e = hipLaunchKernel(core.kernel.fn, dim3(core.workers), dim3(core.kernel.waves * 64), kargs, 0,
                                   (hipStream_t)stream);
    if (e != hipSuccess)
        return hip_fail(e, "hipLaunchKernel");
    return GEMM_OK;
}

} // namespace

// ---- the no-allocation entry point's scratch ---------------------------------
// gemm_run_noalloc takes no plan: the device memory its kernels need beyond
// the caller's operands (the claim counter block, then the problem table) is
// this file-scope array, one copy per GPU, held until the process ends. Host
// code never uses its name as an address: the per-device address comes from
// hipGetSymbolAddress (scratch_address below).
constexpr size_t NOALLOC_TABLE_OFFSET = GEMM_SCHED_COUNTER_BYTES;
static_assert(NOALLOC_TABLE_OFFSET + sizeof(pts::GroupDesc) * GEMM_MAX_GROUPS <= GEMM_NOALLOC_SCRATCH_BYTES,
              "scratch holds the counter block and a full problem table");
static __device__ __align__(256) uint8_t scratch[GEMM_NOALLOC_SCRATCH_BYTES];

// The setup kernel's argument block: the problem table travels by value.
struct NoallocSetup {
    pts::GroupDesc groups[GEMM_MAX_GROUPS];
    uint8_t *scratch; // the device's scratch address
    int32_t group_count;
};
static_assert(sizeof(NoallocSetup) <= 4096, "kernel argument block limit");

// Writes the run's problem table into the scratch and zeroes the claim and
// exit counters (they start each run at zero; the GEMM kernel also resets them
// at its end, but a scratch shared by every call must not rely on the last
// call having finished normally). Vector stores only.
__global__ __launch_bounds__(64) void noalloc_setup_kernel(const NoallocSetup args_by_value)
{
    (void)args_by_value;
    typedef const __attribute__((address_space(4))) NoallocSetup *Args;
    const Args args = (Args)__builtin_amdgcn_kernarg_segment_ptr();
    const int t = threadIdx.x;
    uint8_t *const base = args->scratch;
    uint32_t *const ctr = (uint32_t *)base;
    pts::GroupDesc *const table = (pts::GroupDesc *)(base + NOALLOC_TABLE_OFFSET);
    // the table as 32-bit words (a GroupDesc is 14 words)
    typedef const __attribute__((address_space(4))) uint32_t *ArgWords;
    static_assert(sizeof(pts::GroupDesc) % 4 == 0, "table of whole words");
    const ArgWords src = (ArgWords)&args->groups[0];
    uint32_t *const dst = (uint32_t *)table;
    const int words = args->group_count * (int)(sizeof(pts::GroupDesc) / 4);
    for (int i = t; i < words; i += 64)
        dst[i] = src[i];
    if (t == 0) {
        ctr[pts::CTR_CLAIM] = 0u;
        ctr[pts::CTR_EXIT] = 0u;
    }
    if (t < pts::NUM_XCD)
        ctr[pts::ctr_xcd(t)] = 0u;
}

namespace {

constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_scratch_mutex;
uint8_t *g_scratch_address[NOALLOC_MAX_DEVICES] = {};

// The scratch array's address on `device`, which must be the current device:
// looked up once per device (hipGetSymbolAddress), then kept.
gemm_status scratch_address(int device, uint8_t **out)
{
    if (device < 0 || device >= NOALLOC_MAX_DEVICES)
        return fail(GEMM_ERR_UNSUPPORTED, "device %d: gemm_run_noalloc serves devices 0..%d", device,
                    NOALLOC_MAX_DEVICES - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_address[device] == nullptr) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return hip_fail(e, "hipGetSymbolAddress of the scratch array");
        if (p == nullptr || ((uintptr_t)p % 256) != 0)
            return fail(GEMM_ERR_HIP, "scratch array at an unexpected address %p", p);
        g_scratch_address[device] = (uint8_t *)p;
    }
    *out = g_scratch_address[device];
    return GEMM_OK;
}

} // namespace

extern "C" {

const char *gemm_status_string(gemm_status s)
{
    switch (s) {
    case GEMM_OK: return "success";
    case GEMM_ERR_INVALID_VALUE: return "invalid value";
    case GEMM_ERR_UNSUPPORTED: return "unsupported configuration";
    case GEMM_ERR_OUT_OF_MEMORY: return "out of device memory";
    case GEMM_ERR_HIP: return "HIP runtime error";
    case GEMM_ERR_TIMEOUT: return "device-side wait timed out";
    }
    return "unknown status";
}

const char *gemm_last_error(void) { return g_last_error.c_str(); }

gemm_status gemm_plan_create(const gemm_desc *desc, gemm_plan **out_plan)
{
    if (out_plan == nullptr)
        return fail(GEMM_ERR_INVALID_VALUE, "out_plan is NULL");
    *out_plan = nullptr;
    auto plan = new (std::nothrow) gemm_plan();
    if (plan == nullptr)
        return fail(GEMM_ERR_OUT_OF_MEMORY, "host allocation failed");
    gemm_status st = build_core(desc, plan->core);
    if (st != GEMM_OK) {
        delete plan;
        return st;
    }
    // one device block: the counters first (4 KiB aligned words), then the group table
    const size_t cbytes = sizeof(uint32_t) * pts::CTR_WORDS;
    static_assert(sizeof(uint32_t) * pts::CTR_WORDS == GEMM_SCHED_COUNTER_BYTES, "counter block size");
    const size_t gbytes = sizeof(pts::GroupDesc) * plan->core.group_count;
    hipError_t e = hipMalloc(&plan->d_mem, cbytes + gbytes);
    if (e != hipSuccess) {
        plan->d_mem = nullptr;
        delete plan;
        (void)hipGetLastError();
        return fail(GEMM_ERR_OUT_OF_MEMORY, "hipMalloc of %zu bytes failed", cbytes + gbytes);
    }
    plan->d_counters = (uint32_t *)plan->d_mem;
    plan->d_groups = (pts::GroupDesc *)((uint8_t *)plan->d_mem + cbytes);
    e = hipMemcpy(plan->d_groups, plan->core.groups, gbytes, hipMemcpyHostToDevice);
    if (e == hipSuccess)
        e = hipMemset(plan->d_counters, 0, cbytes);
    if (e == hipSuccess)
        e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        (void)hipFree(plan->d_mem);
        delete plan;
        return hip_fail(e, "plan upload");
    }
    *out_plan = plan;
    return GEMM_OK;
}

gemm_status gemm_plan_destroy(gemm_plan *plan)
{
    if (plan == nullptr)
        return GEMM_OK;
    hipError_t e = hipSuccess;
    if (plan->d_mem != nullptr)
        e = hipFree(plan->d_mem); // the allocation's base address
    delete plan;
    return e == hipSuccess ? GEMM_OK : hip_fail(e, "hipFree");
}

gemm_status gemm_plan_query(const gemm_plan *plan, int64_t *num_tiles, int32_t *num_workers, int32_t *lds_bytes)
{
    if (plan == nullptr)
        return fail(GEMM_ERR_INVALID_VALUE, "plan is NULL");
    if (num_tiles) *num_tiles = plan->core.total_tiles;
    if (num_workers) *num_workers = plan->core.workers;
    if (lds_bytes) *lds_bytes = plan->core.kernel.lds_bytes + 8;
    return GEMM_OK;
}

gemm_status gemm_plan_query_kernel(const gemm_plan *plan, int32_t *tile_m, int32_t *tile_n, int32_t *tile_k,
                                   int32_t *stages, int32_t *waves, int32_t *mfma)
{
    if (plan == nullptr)
        return fail(GEMM_ERR_INVALID_VALUE, "plan is NULL");
    if (tile_m) *tile_m = plan->core.kernel.bm;
    if (tile_n) *tile_n = plan->core.kernel.bn;
    if (tile_k) *tile_k = plan->core.kernel.bk;
    if (stages) *stages = plan->core.kernel.stages;
    if (waves) *waves = plan->core.kernel.waves;
    if (mfma) *mfma = plan->core.kernel.mfma;
    return GEMM_OK;
}

gemm_status gemm_plan_set_trace(gemm_plan *plan, void *device_buf, size_t bytes)
{
    if (plan == nullptr)
        return fail(GEMM_ERR_INVALID_VALUE, "plan is NULL");
    if (device_buf == nullptr) {
        plan->trace = nullptr;
        plan->trace_bytes = 0;
        return GEMM_OK;
    }
    const size_t need =
        sizeof(pts::TileTrace) * (size_t)plan->core.total_tiles + sizeof(pts::WorkerTrace) * plan->core.workers;
    if (bytes < need)
        return fail(GEMM_ERR_INVALID_VALUE, "trace buffer of %zu bytes; %zu needed", bytes, need);
    if (((uintptr_t)device_buf % 16) != 0)
        return fail(GEMM_ERR_INVALID_VALUE, "trace buffer must be 16-byte aligned");
    plan->trace = device_buf;
    plan->trace_bytes = bytes;
    return GEMM_OK;
}

gemm_status gemm_plan_read_counters(const gemm_plan *plan, uint32_t out[5])
{
    if (plan == nullptr || out == nullptr)
        return fail(GEMM_ERR_INVALID_VALUE, "plan or out is NULL");
    hipError_t e = hipDeviceSynchronize();
    uint32_t words[pts::CTR_SYNC_STALLS + 1];
    if (e == hipSuccess)
        e = hipMemcpy(words, plan->d_counters, sizeof(words), hipMemcpyDeviceToHost);
    if (e != hipSuccess)
        return hip_fail(e, "reading counters");
    uint32_t live_xcd = 0;
    for (int x = 0; x < pts::NUM_XCD && e == hipSuccess; ++x) {
        uint32_t v = 0;
        e = hipMemcpy(&v, plan->d_counters + pts::ctr_xcd(x), sizeof(v), hipMemcpyDeviceToHost);
        live_xcd += v;
    }
    if (e != hipSuccess)
        return hip_fail(e, "reading counters");
    out[0] = words[pts::CTR_CLAIM] + live_xcd;
    out[1] = words[pts::CTR_EXIT];
    out[2] = words[pts::CTR_FINAL];
    out[3] = words[pts::CTR_RUNS];
    out[4] = words[pts::CTR_SYNC_STALLS];
    return GEMM_OK;
}

gemm_status gemm_plan_preset_claims(gemm_plan *plan, uint32_t value)
{
    if (plan == nullptr)
        return fail(GEMM_ERR_INVALID_VALUE, "plan is NULL");
    if (plan->core.schedule != GEMM_SCHEDULE_DYNAMIC && plan->core.schedule != GEMM_SCHEDULE_DYNAMIC_XCD)
        return fail(GEMM_ERR_INVALID_VALUE, "only the dynamic schedules claim tiles");
    if (value > 0x00FFFFFFu)
        return fail(GEMM_ERR_INVALID_VALUE, "preset value must be below 2^24");
    hipError_t e = hipDeviceSynchronize();
    if (plan->core.schedule == GEMM_SCHEDULE_DYNAMIC) {
        if (e == hipSuccess)
            e = hipMemcpy(plan->d_counters + pts::CTR_CLAIM, &value, sizeof value, hipMemcpyHostToDevice);
    } else {
        for (int x = 0; x < pts::NUM_XCD && e == hipSuccess; ++x)
            e = hipMemcpy(plan->d_counters + pts::ctr_xcd(x), &value, sizeof value, hipMemcpyHostToDevice);
    }
    return e == hipSuccess ? GEMM_OK : hip_fail(e, "presetting the claim counters");
}

gemm_status gemm_run(gemm_plan *plan, const gemm_operands *ops, void *stream)
{
    if (plan == nullptr)
        return fail(GEMM_ERR_INVALID_VALUE, "plan is NULL");
    pts::GemmArgs args;
    gemm_status st = fill_args(plan->core, ops, args);
    if (st != GEMM_OK)
        return st;
    if (plan->core.workers == 0)
        return GEMM_OK;
    args.groups = plan->d_groups;
    args.counters = plan->d_counters;
    args.trace = (uint8_t *)plan->trace;
    return launch_gemm(plan->core, args, stream);
}

gemm_status gemm_run_noalloc(const gemm_desc *desc, const gemm_operands *ops, void *stream)
{
    if (desc != nullptr && desc->group_count > GEMM_MAX_GROUPS)
        return fail(GEMM_ERR_UNSUPPORTED,
                    "group_count %d: the scratch of gemm_run_noalloc holds a table of at most %d problems",
                    desc->group_count, GEMM_MAX_GROUPS);
    PlanCore core;
    gemm_status st = build_core(desc, core);
    if (st != GEMM_OK)
        return st;
    pts::GemmArgs args;
    st = fill_args(core, ops, args);
    if (st != GEMM_OK)
        return st;
    if (core.workers == 0)
        return GEMM_OK;
    uint8_t *base = nullptr;
    st = scratch_address(core.device, &base);
    if (st != GEMM_OK)
        return st;
    NoallocSetup setup;
    memset(&setup, 0, sizeof setup);
    memcpy(setup.groups, core.groups, sizeof(pts::GroupDesc) * core.group_count);
    setup.scratch = base;
    setup.group_count = core.group_count;
    void *sargs[] = {&setup};
    hipError_t e = hipLaunchKernel((const void *)&noalloc_setup_kernel, dim3(1), dim3(64), sargs, 0,
                                   (hipStream_t)stream);
    if (e != hipSuccess)
        return hip_fail(e, "setup kernel launch");
    args.counters = (uint32_t *)base;
    args.groups = (const pts::GroupDesc *)(base + NOALLOC_TABLE_OFFSET);
    args.trace = nullptr;
    return launch_gemm(core, args, stream);
}

gemm_status pts_copy_int16(const void *src, void *dst, int64_t n, int32_t num_blocks, void *stream)
{
    if (n < 0)
        return fail(GEMM_ERR_INVALID_VALUE, "n must be >= 0");
    if (n == 0)
        return GEMM_OK;
    if (src == nullptr || dst == nullptr)
        return fail(GEMM_ERR_INVALID_VALUE, "NULL pointer");
    if (((uintptr_t)src % 16) != 0 || ((uintptr_t)dst % 16) != 0)
        return fail(GEMM_ERR_INVALID_VALUE, "src and dst must be 16-byte aligned");
    const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst, bytes = (uintptr_t)n * 2;
    if (s0 < d0 + bytes && d0 < s0 + bytes)
        return fail(GEMM_ERR_INVALID_VALUE, "src and dst overlap");
    int blocks = num_blocks;
    if (blocks <= 0) {
        int dev = 0, cus = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess)
            e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess)
            return hip_fail(e, "device query");
        blocks = cus * 4;
    }
    const int64_t nvec = n / 8;
    hipLaunchKernelGGL(pts::copy_int16_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       (const int4 *)src, (int4 *)dst, nvec, (const int16_t *)src, (int16_t *)dst, n);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? GEMM_OK : hip_fail(e, "copy launch");
}

gemm_status pts_stream_create_cu_masked(int32_t cu_count, void **out_stream)
{
    if (out_stream == nullptr)
        return fail(GEMM_ERR_INVALID_VALUE, "NULL out_stream");
    *out_stream = nullptr;
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess)
        return hip_fail(e, "device query");
    if (cu_count < 1 || cu_count > cus)
        return fail(GEMM_ERR_INVALID_VALUE, "cu_count must be in [1, compute units]");
    std::vector<uint32_t> mask((cus + 31) / 32, 0u);
    for (int c = 0; c < cu_count; ++c)
        mask[c / 32] |= 1u << (c % 32);
    hipStream_t st = nullptr;
    e = hipExtStreamCreateWithCUMask(&st, (uint32_t)mask.size(), mask.data());
    if (e != hipSuccess)
        return hip_fail(e, "hipExtStreamCreateWithCUMask");
    *out_stream = st;
    return GEMM_OK;
}

gemm_status pts_stream_destroy(void *stream)
{
    if (stream == nullptr)
        return GEMM_OK;
    hipError_t e = hipStreamDestroy((hipStream_t)stream);
    return e == hipSuccess ? GEMM_OK : hip_fail(e, "hipStreamDestroy");
}

gemm_status pts_sched_probe(int32_t num_tiles, int32_t num_workers, int32_t schedule, int32_t gate_worker,
                            int64_t work_ns, int64_t spin_limit, int32_t *out_tiles, int32_t *out_counts,
                            int32_t max_per_worker, uint32_t *counters, uint32_t *out_status, void *stream)
{
    if (num_tiles < 0 || num_workers < 1 || num_workers > 4096 || max_per_worker < 1)
        return fail(GEMM_ERR_INVALID_VALUE, "bad probe sizes");
    if (schedule != GEMM_SCHEDULE_STATIC && schedule != GEMM_SCHEDULE_DYNAMIC &&
        schedule != GEMM_SCHEDULE_DYNAMIC_XCD)
        return fail(GEMM_ERR_INVALID_VALUE, "bad schedule");
    if (gate_worker >= num_workers || work_ns < 0 || spin_limit < 0 || work_ns > 1000000000LL)
        return fail(GEMM_ERR_INVALID_VALUE, "bad probe parameters");
    if (out_tiles == nullptr || out_counts == nullptr || counters == nullptr || out_status == nullptr)
        return fail(GEMM_ERR_INVALID_VALUE, "NULL pointer");
    hipLaunchKernelGGL(pts::sched_probe_kernel, dim3(num_workers), dim3(64), 0, (hipStream_t)stream, num_tiles,
                       num_workers, schedule, gate_worker, work_ns / 10, spin_limit, out_tiles, out_counts,
                       max_per_worker, counters, out_status);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? GEMM_OK : hip_fail(e, "probe launch");
}

gemm_status pts_mfma_ceiling(const void *frags, float *out, uint64_t *stamps, int32_t num_blocks, int32_t steps,
                             void *stream)
{
    if (steps < 2 || (steps & 1) != 0)
        return fail(GEMM_ERR_INVALID_VALUE, "steps must be even and >= 2");
    if (num_blocks < 0 || num_blocks > 65536)
        return fail(GEMM_ERR_INVALID_VALUE, "num_blocks must be in [0, 65536]");
    if (frags == nullptr || out == nullptr || stamps == nullptr)
        return fail(GEMM_ERR_INVALID_VALUE, "NULL pointer");
    if (((uintptr_t)frags % 16) != 0 || ((uintptr_t)out % 4) != 0 || ((uintptr_t)stamps % 8) != 0)
        return fail(GEMM_ERR_INVALID_VALUE, "frags must be 16-byte, out 4-byte, stamps 8-byte aligned");
    int blocks = num_blocks;
    if (blocks == 0) {
        int dev = 0, cus = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess)
            e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess)
            return hip_fail(e, "device query");
        blocks = cus;
    }
    hipLaunchKernelGGL(pts::mfma_ceiling_kernel, dim3(blocks), dim3(512), 0, (hipStream_t)stream,
                       (const pts::bf16x8 *)frags, out, stamps, steps);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? GEMM_OK : hip_fail(e, "ceiling probe launch");
}

} // extern "C"
