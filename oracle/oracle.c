/*
 * CPU oracle for the fp16-operand / fp32-accumulate / fp16-result GEMM and for the
 * grouped program-id -> output-tile map.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load this library.  The GPU library shares no code, header, table
 * or helper with it, and neither side includes or links the other.
 *
 * What it computes, and where that is defined:
 *
 *   GEMM.  phobos "03: Matrix multiplication" (module docstring, the `matmul` kernel and
 *   the paragraph after it): C = A B with fp16 operands, products accumulated in an fp32
 *   accumulator, and the accumulator narrowed to fp16 once, on the store.  The accumulation
 *   order inside fp32 is left open by the page, so the oracle computes the plain
 *   definition more exactly than the method does: every fp16 x fp16 product is exact in
 *   double, the products are summed in double in ascending k, and the double sum is
 *   rounded once, to nearest with ties to even (the page's `.to(float16)`), to fp16.
 *   A GPU result is accepted when |gpu - oracle| <= 1e-2 + 2^-10 |oracle| element-wise.
 *   Elements of C outside the M x N block are never written; K = 0 gives +0.
 *
 *   Tile map.  kernl notebook "Computing coordinates on Triton GEMM example" (the quoted
 *   tutorial excerpt in the introduction and cells In[1]-In[7]): the number of programs
 *   per axis is a ceiling division, programs are grouped GROUP_SIZE_M tile-rows at a
 *   time, the last group may be smaller, and inside a group programs run column-major.
 *   The oracle builds the order by walking the bands and columns (not by evaluating the
 *   notebook's closed form); the row inside a column is the absolute program id modulo the
 *   band's height, as the notebook's formula has it, which matters only in a smaller last
 *   band.
 *
 *   XCD pre-permutation.  Not from the pages: a bijection applied to the hardware
 *   workgroup id before the grouped map, so that consecutive logical program ids land on
 *   the same L2 when workgroups are dealt round-robin over X dies.  With P programs,
 *   q = P / X, r = P % X and x = h % X, logical pid = x*q + min(x, r) + h / X.
 *
 * Build: gcc -O3 -std=c11 -fopenmp -ffp-contract=off -shared -fPIC.  No -ffast-math: the
 * ascending-k double sum must not be reassociated.
 */
#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

/* ---------------------------------------------------------------------------------------
 * fp16 codec (IEEE 754 binary16: 1 sign bit, 5 exponent bits with bias 15, 10 fraction
 * bits).  Decoding follows the format's definition; encoding rounds to nearest, ties to
 * even, with overflow to infinity.
 * ------------------------------------------------------------------------------------- */

static double f16_table[65536];
static int f16_table_ready = 0;

static double f16_decode_def(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);               /* zero or subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;                  /* infinity or NaN */
    else
        v = ldexp((double)(1024 + f), e - 25);   /* normal: (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

void oracle_init(void)
{
    if (f16_table_ready)
        return;
    for (int h = 0; h < 65536; ++h)
        f16_table[h] = f16_decode_def((uint16_t)h);
    f16_table_ready = 1;
}

double oracle_f16_to_f64(uint16_t h)
{
    return f16_decode_def(h);
}

/* Round a non-negative double q (0 <= q < 2^53) to the nearest integer, ties to even. */
static double round_half_even(double q)
{
    double f = floor(q);
    double r = q - f;     /* exact: f and q share the exponent range here */
    if (r > 0.5)
        return f + 1.0;
    if (r < 0.5)
        return f;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

uint16_t oracle_f64_to_f16(double x)
{
    if (isnan(x))
        return (uint16_t)(signbit(x) ? 0xfe00 : 0x7e00);
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isinf(a))
        return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: a = m * 2^-24 with m in [0, 1024]; m = 1024 is the smallest
         * normal, whose bit pattern is exactly 1024 (exponent field 1, fraction 0) */
        double m = round_half_even(ldexp(a, 24));
        return sign | (uint16_t)m;
    }
    int e;
    frexp(a, &e);          /* a = g * 2^e with g in [0.5, 1): unbiased exponent is e - 1 */
    int ub = e - 1;
    double q = round_half_even(ldexp(a, 10 - ub));   /* 11-bit significand in [1024, 2048] */
    if (q == 2048.0) {
        q = 1024.0;
        ub += 1;
    }
    if (ub + 15 >= 31)
        return sign | 0x7c00;                          /* overflow: |x| >= 65520 */
    return sign | (uint16_t)(((ub + 15) << 10) | ((int)q - 1024));
}

/* ---------------------------------------------------------------------------------------
 * GEMM.  Row-major A (M x K, leading dimension lda), B (K x N, ldb), C (M x N, ldc), all
 * fp16 bit patterns.  One output element: decode, multiply exactly, sum in ascending k in
 * double, round once.
 * ------------------------------------------------------------------------------------- */

static double dot_ascending_k(int64_t K, const uint16_t *A, int64_t lda, const uint16_t *B,
                              int64_t ldb, int64_t i, int64_t j)
{
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k)
        s += f16_table[A[i * lda + k]] * f16_table[B[k * ldb + j]];
    return s;
}

/* Full product.  The elements of C are visited in blocks of ORACLE_IB rows x ORACLE_JB
 * columns; inside a block every element has its own double accumulator, starting at +0, and
 * k runs from 0 to K-1 in the outermost loop, so each accumulator receives exactly the
 * additions of dot_ascending_k, in the same order.  Which elements are worked on together
 * is the only thing the blocks change (each element's k order is the definition; the order
 * in which elements are visited is not part of it).  Blocks are spread over OpenMP threads. */
#define ORACLE_IB 64
#define ORACLE_JB 256

/* acc[ii][jj] = sum over k ascending of A[i0+ii][k] B[k][j0+jj], ii < ni, jj < nj.  The
 * clones only let the compiler use wider vector registers for the jj loop (independent
 * accumulators, so nothing is reassociated). */
__attribute__((target_clones("avx512f", "avx2", "default")))
static void block_ascending_k(int64_t K, const uint16_t *A, int64_t lda, const uint16_t *B,
                              int64_t ldb, int64_t i0, int64_t ni, int64_t j0, int64_t nj,
                              double *acc, double *brow)
{
    for (int64_t x = 0; x < (int64_t)ORACLE_IB * ORACLE_JB; ++x)
        acc[x] = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        const uint16_t *b = B + k * ldb + j0;
        for (int64_t jj = 0; jj < nj; ++jj)
            brow[jj] = f16_table[b[jj]];
        for (int64_t ii = 0; ii < ni; ++ii) {
            const double a = f16_table[A[(i0 + ii) * lda + k]];
            double *row = acc + ii * ORACLE_JB;
            for (int64_t jj = 0; jj < nj; ++jj)
                row[jj] += a * brow[jj];
        }
    }
}

void oracle_gemm(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                 const uint16_t *B, int64_t ldb, uint16_t *C, int64_t ldc)
{
    oracle_init();
    if (M <= 0 || N <= 0)
        return;
    const int64_t nbi = (M + ORACLE_IB - 1) / ORACLE_IB, nbj = (N + ORACLE_JB - 1) / ORACLE_JB;
#pragma omp parallel
    {
        double *acc = malloc(sizeof(double) * ORACLE_IB * ORACLE_JB);
        double *brow = malloc(sizeof(double) * ORACLE_JB);
#pragma omp for schedule(dynamic, 1)
        for (int64_t blk = 0; blk < nbi * nbj; ++blk) {
            const int64_t i0 = (blk % nbi) * ORACLE_IB, j0 = (blk / nbi) * ORACLE_JB;
            const int64_t ni = M - i0 < ORACLE_IB ? M - i0 : ORACLE_IB;
            const int64_t nj = N - j0 < ORACLE_JB ? N - j0 : ORACLE_JB;
            block_ascending_k(K, A, lda, B, ldb, i0, ni, j0, nj, acc, brow);
            for (int64_t ii = 0; ii < ni; ++ii)
                for (int64_t jj = 0; jj < nj; ++jj)
                    C[(i0 + ii) * ldc + j0 + jj] = oracle_f64_to_f16(acc[ii * ORACLE_JB + jj]);
        }
        free(acc);
        free(brow);
    }
}

/* The plain form of the same product: one dot_ascending_k per element, rows spread over
 * OpenMP threads.  Kept beside the blocked form so that tests can compare the two. */
void oracle_gemm_plain(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                       const uint16_t *B, int64_t ldb, uint16_t *C, int64_t ldc)
{
    oracle_init();
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            C[i * ldc + j] = oracle_f64_to_f16(dot_ascending_k(K, A, lda, B, ldb, i, j));
}

/* Selected elements (rows[t], cols[t]) only, for shapes too large for the full product.
 * out_f16[t] is the rounded result; out_f64[t] (if not NULL) the double sum before it. */
void oracle_gemm_sampled(int64_t K, const uint16_t *A, int64_t lda, const uint16_t *B,
                         int64_t ldb, int64_t count, const int64_t *rows, const int64_t *cols,
                         uint16_t *out_f16, double *out_f64)
{
    oracle_init();
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < count; ++t) {
        double s = dot_ascending_k(K, A, lda, B, ldb, rows[t], cols[t]);
        out_f16[t] = oracle_f64_to_f16(s);
        if (out_f64)
            out_f64[t] = s;
    }
}

/* Number of OpenMP threads a parallel region of this library uses. */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}

/* ---------------------------------------------------------------------------------------
 * Tile map (kernl notebook, introduction excerpt and cells In[1], In[2], In[4]-In[7]).
 * ------------------------------------------------------------------------------------- */

int64_t oracle_cdiv(int64_t x, int64_t y)
{
    return (x + y - 1) / y;
}

/* Grouped order, built by walking it.  Program ids are handed out band by band: a band is
 * up to G consecutive tile rows (the last band holds the rows that are left), and it takes
 * as many consecutive ids as it has tiles.  Inside a band the ids go down the columns, left
 * to right: each column takes the next h ids, h being the band's height.  Within a column an
 * id lands on the row (id mod h) counted from the band's top row.  In a full band, and in any
 * band that follows only full ones when h divides their id count, that is the id's position
 * down the column; in a shorter last band the positions are rotated by (ids before the band)
 * mod h -- the notebook computes the row from the absolute id, not from the id's position in
 * its group.
 *
 * walk_grouped visits every program in id order and reports each to `visit`, with its band's
 * index, top row and height; it stops early when `visit` returns non-zero. */
typedef int (*grouped_visit)(void *ctx, int64_t id, int64_t row, int64_t col, int64_t band,
                             int64_t top, int64_t h);

static void walk_grouped(int64_t num_pid_m, int64_t num_pid_n, int64_t G, grouped_visit visit,
                         void *ctx)
{
    int64_t id = 0, band = 0;
    for (int64_t top = 0; top < num_pid_m; top += G, ++band) {
        const int64_t h = num_pid_m - top < G ? num_pid_m - top : G;
        for (int64_t col = 0; col < num_pid_n; ++col)
            for (int64_t t = 0; t < h; ++t, ++id)
                if (visit(ctx, id, top + id % h, col, band, top, h))
                    return;
    }
}

struct one_program {
    int64_t want, row, col, band, top, h;
};

static int find_program(void *ctx, int64_t id, int64_t row, int64_t col, int64_t band,
                        int64_t top, int64_t h)
{
    struct one_program *p = ctx;
    if (id != p->want)
        return 0;
    p->row = row, p->col = col, p->band = band, p->top = top, p->h = h;
    return 1;
}

static int grouped_args_ok(int64_t num_pid_m, int64_t num_pid_n, int64_t G)
{
    return num_pid_m > 0 && num_pid_n > 0 && G > 0;
}

/* Tile (pid_m, pid_n) of program `pid`.  Returns 0, or -1 if the arguments are out of range
 * (pid outside [0, num_pid_m*num_pid_n), or a non-positive size). */
int oracle_tile_map(int64_t num_pid_m, int64_t num_pid_n, int64_t group_size_m, int64_t pid,
                    int64_t *pid_m, int64_t *pid_n)
{
    if (!grouped_args_ok(num_pid_m, num_pid_n, group_size_m) || pid < 0 ||
        pid >= num_pid_m * num_pid_n)
        return -1;
    struct one_program p = {pid, -1, -1, -1, -1, -1};
    walk_grouped(num_pid_m, num_pid_n, group_size_m, find_program, &p);
    *pid_m = p.row;
    *pid_n = p.col;
    return 0;
}

/* The quantities the notebook prints for one program (cells In[4]-In[7]), from the walk:
 * out[0] = ids per full band (G * num_pid_n), out[1] = the band's index, out[2] = its top
 * row, out[3] = its height, out[4] = pid_m, out[5] = pid_n.  Returns 0, or -1 on
 * out-of-range arguments. */
int oracle_tile_map_detail(int64_t num_pid_m, int64_t num_pid_n, int64_t group_size_m,
                           int64_t pid, int64_t *out)
{
    if (!grouped_args_ok(num_pid_m, num_pid_n, group_size_m) || pid < 0 ||
        pid >= num_pid_m * num_pid_n)
        return -1;
    struct one_program p = {pid, -1, -1, -1, -1, -1};
    walk_grouped(num_pid_m, num_pid_n, group_size_m, find_program, &p);
    out[0] = group_size_m * num_pid_n;
    out[1] = p.band;
    out[2] = p.top;
    out[3] = p.h;
    out[4] = p.row;
    out[5] = p.col;
    return 0;
}

struct all_programs {
    int64_t *pid_m, *pid_n;
};

static int record_program(void *ctx, int64_t id, int64_t row, int64_t col, int64_t band,
                          int64_t top, int64_t h)
{
    struct all_programs *p = ctx;
    (void)band, (void)top, (void)h;
    p->pid_m[id] = row;
    p->pid_n[id] = col;
    return 0;
}

/* (pid_m, pid_n) of every program 0 .. P-1, P = num_pid_m * num_pid_n, in one walk. */
int oracle_tile_map_fill(int64_t num_pid_m, int64_t num_pid_n, int64_t group_size_m,
                         int64_t *pid_m, int64_t *pid_n)
{
    if (!grouped_args_ok(num_pid_m, num_pid_n, group_size_m))
        return -1;
    struct all_programs p = {pid_m, pid_n};
    walk_grouped(num_pid_m, num_pid_n, group_size_m, record_program, &p);
    return 0;
}

/* Element offsets of one program's panels (notebook cell In[8], with unit inner strides):
 * A[pid_m*BM + r][k] sits at (pid_m*BM + r)*lda + k and B[k][pid_n*BN + c] at
 * k*ldb + pid_n*BN + c, counted in elements from each matrix's first element. */
int64_t oracle_offset_a(int64_t pid_m, int64_t BM, int64_t lda, int64_t r, int64_t k)
{
    return (pid_m * BM + r) * lda + k;
}

int64_t oracle_offset_b(int64_t pid_n, int64_t BN, int64_t ldb, int64_t k, int64_t c)
{
    return k * ldb + pid_n * BN + c;
}

/* XCD pre-permutation: hardware id h in [0, P) -> logical pid, X dies dealt round-robin. */
int64_t oracle_xcd_remap(int64_t P, int64_t X, int64_t h)
{
    int64_t q = P / X, r = P % X, x = h % X;
    return x * q + (x < r ? x : r) + h / X;
}
