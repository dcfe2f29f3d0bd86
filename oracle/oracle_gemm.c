/*
 * oracle_gemm.c -- plain, slow, obviously correct CPU oracle for D = A * B.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. The HIP library never
 * includes, links or calls anything here, and nothing here comes from it.
 *
 * What is computed. The CUTLASS Task Scheduling page "Pipeline Groups"
 * (section "Overview") gives the canonical Merge case as a GEMM mainloop:
 * LoadA fills smem_a, LoadB fills smem_b, the MMA task consumes both into the
 * accumulator tmem_c, and gmem_d is produced from tmem_c. Whatever the
 * pipelining and scheduling, the result is the matrix product
 *
 *     D[i][j] = sum over k = 0 .. K-1 of A[i][k] * B[k][j],
 *
 * and that plain definition is what this file writes out:
 *   - A and B arrive as bf16 bit patterns and are decoded exactly to double
 *     (a bf16 pattern is the high half of a float32 pattern);
 *   - each output element has one double accumulator, starting at zero, that
 *     adds the products for k = 0, 1, ..., K-1 in that order;
 *   - the result stays in double for the comparison.
 * A product of two bf16 values has at most 16 significant bits and is exact in
 * double, so fused or unfused multiply-add give the same bits here.
 *
 * Layouts (the reading the tests and the HIP path share):
 *   A is M x K row-major:    A[i][k] = a[i * lda + k]
 *   B is K x N column-major: B[k][j] = b[j * ldb + k]
 *   D is M x N row-major:    D[i][j] = d[i * ldd + j]
 *
 * bf16 output rounding is round-to-nearest, ties to even, written here from
 * the IEEE-754 definition (scale to the target grid, round, scale back); the
 * pages do not name a rounding, and this is the IEEE default.
 *
 * Parallelism: OpenMP over output rows only (and over k for the copy of B).
 * Every element's summation order is fixed, so the result does not depend on
 * the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

/* bf16 bits -> double, exact. */
static inline double decode(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double oracle_bf16_decode(uint16_t bits) { return decode(bits); }

void oracle_bf16_decode_array(const uint16_t *bits, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = decode(bits[i]);
}

/*
 * double -> bf16 bits, round to nearest with ties to even.
 *
 * bf16 keeps 8 significant bits and float32's exponent range. For a finite
 * non-zero x with 2^e <= |x| < 2^(e+1), the representable neighbours are
 * spaced 2^(e-7); below the normal range (e < -126) the spacing stays 2^-133.
 * x / spacing is exact (a power-of-two scaling), rint() rounds it to the
 * nearest integer with ties to even (the default rounding mode), and scaling
 * back is exact again. A result of 2^128 or more is an overflow to infinity.
 */
uint16_t oracle_bf16_round_rne(double x)
{
    if (isnan(x))
        return (uint16_t)0x7FC0;
    if (isinf(x))
        return (uint16_t)(x > 0 ? 0x7F80 : 0xFF80);
    if (x == 0.0)
        return (uint16_t)(signbit(x) ? 0x8000 : 0x0000);
    int e2;
    (void)frexp(x, &e2);            /* |x| = m * 2^e2, 0.5 <= m < 1 */
    int e = e2 - 1;                 /* 2^e <= |x| < 2^(e+1) */
    int q = e - 7;                  /* exponent of the spacing */
    if (q < -133)
        q = -133;
    double r = ldexp(rint(ldexp(x, -q)), q);
    if (fabs(r) >= ldexp(1.0, 128))
        return (uint16_t)(r > 0 ? 0x7F80 : 0xFF80);
    float f = (float)r;             /* exact: r has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

void oracle_bf16_round_array(const double *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_round_rne(x[i]);
}

static void set_threads(int nthreads)
{
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
}

int oracle_max_threads(void)
{
    return omp_get_max_threads();
}

/*
 * Full product: D (m x n, row-major, ldd) = A (m x k, row-major, lda)
 *                                          * B (k x n, column-major, ldb).
 *
 * Loop order i, k, j: for one output row i, every element D[i][j] holds its
 * own double accumulator, which starts at zero and receives the products
 * A[i][k] * B[k][j] for k = 0, 1, ..., K-1 in that order -- the same additions,
 * in the same order, with the same roundings as a per-element k loop. Only
 * which element is advanced next changes, so the result is bit-identical to
 * the i, j, k triple loop (oracle_gemm_entries computes single elements that
 * way). With j innermost, B is read along its rows, so a copy of B with its
 * rows contiguous (bt[kk * n + j] = B[kk][j], the bf16 bit patterns moved, not
 * changed) is made first. Returns 0, or -1 if that copy cannot be allocated.
 */
int oracle_gemm(int64_t m, int64_t n, int64_t k,
                const uint16_t *a, int64_t lda,
                const uint16_t *b, int64_t ldb,
                double *d, int64_t ldd, int nthreads)
{
    set_threads(nthreads);
    uint16_t *bt = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(k * n > 0 ? k * n : 1));
    if (bt == NULL)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t kk = 0; kk < k; ++kk)
        for (int64_t j = 0; j < n; ++j)
            bt[kk * n + j] = b[j * ldb + kk];
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i) {
        double *drow = d + i * ldd;
        for (int64_t j = 0; j < n; ++j)
            drow[j] = 0.0;
        for (int64_t kk = 0; kk < k; ++kk) {
            const double aik = decode(a[i * lda + kk]);
            const uint16_t *brow = bt + kk * n;
            for (int64_t j = 0; j < n; ++j)
                drow[j] += aik * decode(brow[j]);
        }
    }
    free(bt);
    return 0;
}

/*
 * The same definition evaluated only at the listed (row, col) entries:
 * out[e] = D[rows[e]][cols[e]]. Used where D is too large for the full loop.
 */
void oracle_gemm_entries(int64_t k,
                         const uint16_t *a, int64_t lda,
                         const uint16_t *b, int64_t ldb,
                         int64_t count, const int64_t *rows, const int64_t *cols,
                         double *out, int nthreads)
{
    set_threads(nthreads);
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < count; ++e) {
        const int64_t i = rows[e], j = cols[e];
        double acc = 0.0;
        for (int64_t kk = 0; kk < k; ++kk)
            acc += decode(a[i * lda + kk]) * decode(b[j * ldb + kk]);
        out[e] = acc;
    }
}
