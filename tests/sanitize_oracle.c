/*
 * Drives every function of oracle/oracle.c on edge inputs, for a build under AddressSanitizer
 * and UndefinedBehaviorSanitizer (tests/test_sanitizers.py).  Every buffer is heap-allocated
 * at its exact size, so a read or write past one is reported.  Prints "ok" and exits 0 when
 * no sanitizer fires (they abort the process otherwise).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_init(void);
double oracle_f16_to_f64(uint16_t h);
uint16_t oracle_f64_to_f16(double x);
void oracle_gemm(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                 const uint16_t *B, int64_t ldb, uint16_t *C, int64_t ldc);
void oracle_gemm_sampled(int64_t K, const uint16_t *A, int64_t lda, const uint16_t *B,
                         int64_t ldb, int64_t count, const int64_t *rows, const int64_t *cols,
                         uint16_t *out_f16, double *out_f64);
int oracle_num_threads(void);
int64_t oracle_cdiv(int64_t x, int64_t y);
int oracle_tile_map(int64_t num_pid_m, int64_t num_pid_n, int64_t group_size_m, int64_t pid,
                    int64_t *pid_m, int64_t *pid_n);
int oracle_tile_map_detail(int64_t num_pid_m, int64_t num_pid_n, int64_t group_size_m,
                           int64_t pid, int64_t *out);
int oracle_tile_map_fill(int64_t num_pid_m, int64_t num_pid_n, int64_t group_size_m,
                         int64_t *pid_m, int64_t *pid_n);
int64_t oracle_offset_a(int64_t pid_m, int64_t BM, int64_t lda, int64_t r, int64_t k);
int64_t oracle_offset_b(int64_t pid_n, int64_t BN, int64_t ldb, int64_t k, int64_t c);
int64_t oracle_xcd_remap(int64_t P, int64_t X, int64_t h);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint16_t next_bits(void)
{
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint16_t)(state >> 48);
}

/* exact-size buffer of rows x ld elements (ld >= cols), random fp16 patterns */
static uint16_t *matrix(int64_t rows, int64_t cols, int64_t ld)
{
    size_t n = rows > 0 && cols > 0 ? (size_t)((rows - 1) * ld + cols) : 1;
    uint16_t *p = (uint16_t *)malloc(n * sizeof(uint16_t));
    for (size_t i = 0; i < n; ++i) p[i] = next_bits();
    return p;
}

int main(void)
{
    oracle_init();
    /* codec: every pattern, and doubles around every edge */
    for (uint32_t h = 0; h < 65536; ++h) {
        const double v = oracle_f16_to_f64((uint16_t)h);
        const uint16_t back = oracle_f64_to_f16(v);
        if (!isnan(v) && back != h) {
            printf("round trip failed at %u\n", h);
            return 1;
        }
    }
    const double edges[] = {0.0, -0.0, INFINITY, -INFINITY, NAN, 65504.0, 65519.99, 65520.0,
                            -65520.0, 1e300, -1e300, 5.960464477539063e-08, 2.98e-08, 1e-300,
                            6.103515625e-05, 0.5, 1.0 + 1.0 / 2048, 2049.0, 4095.0};
    for (size_t i = 0; i < sizeof edges / sizeof edges[0]; ++i) (void)oracle_f64_to_f16(edges[i]);

    /* GEMM and sampled GEMM on ragged shapes with padded leading dimensions */
    const int64_t shapes[][3] = {{1, 1, 0}, {1, 1, 1}, {3, 5, 7}, {17, 1, 33}, {1, 64, 130},
                                 {40, 30, 65}, {2, 3, 1000}};
    for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s) {
        const int64_t M = shapes[s][0], N = shapes[s][1], K = shapes[s][2];
        const int64_t lda = K + 3, ldb = N + 1, ldc = N + 2;
        uint16_t *A = matrix(M, K, lda > 0 ? lda : 1), *B = matrix(K, N, ldb);
        uint16_t *C = matrix(M, N, ldc);
        oracle_gemm(M, N, K, A, lda, B, ldb, C, ldc);
        int64_t rows[4] = {0, M - 1, M / 2, 0}, cols[4] = {0, N - 1, N / 2, N - 1};
        uint16_t *o16 = (uint16_t *)malloc(4 * sizeof(uint16_t));
        double *o64 = (double *)malloc(4 * sizeof(double));
        oracle_gemm_sampled(K, A, lda, B, ldb, 4, rows, cols, o16, o64);
        oracle_gemm_sampled(K, A, lda, B, ldb, 4, rows, cols, o16, NULL);
        for (int t = 0; t < 4; ++t)
            if (o16[t] != C[rows[t] * ldc + cols[t]]) {
                printf("sampled and full differ\n");
                return 1;
            }
        free(A), free(B), free(C), free(o16), free(o64);
    }
    if (oracle_num_threads() < 1) return 1;

    /* tile map: every pid of small grids, its intermediates, the fill, and the rejections */
    for (int64_t m = 1; m <= 12; ++m)
        for (int64_t n = 1; n <= 12; ++n)
            for (int64_t G = 1; G <= 14; ++G) {
                const int64_t P = m * n;
                int64_t *pm = (int64_t *)malloc((size_t)P * sizeof(int64_t));
                int64_t *pn = (int64_t *)malloc((size_t)P * sizeof(int64_t));
                if (oracle_tile_map_fill(m, n, G, pm, pn) != 0) return 1;
                int64_t out[6];
                for (int64_t p = 0; p < P; ++p)
                    if (oracle_tile_map_detail(m, n, G, p, out) != 0 || out[4] != pm[p] ||
                        out[5] != pn[p])
                        return 1;
                free(pm), free(pn);
            }
    int64_t a, b, out[6];
    if (oracle_tile_map(0, 3, 1, 0, &a, &b) != -1 || oracle_tile_map(3, 3, 0, 0, &a, &b) != -1 ||
        oracle_tile_map(3, 3, 1, 9, &a, &b) != -1 || oracle_tile_map(3, 3, 1, -1, &a, &b) != -1 ||
        oracle_tile_map_detail(2, 2, 1, 4, out) != -1)
        return 1;
    (void)oracle_cdiv(8191, 256);
    (void)oracle_offset_a(31, 256, 8192, 255, 8191);
    (void)oracle_offset_b(31, 256, 8192, 8191, 255);
    for (int64_t P = 1; P <= 300; ++P)
        for (int64_t h = 0; h < P; ++h) (void)oracle_xcd_remap(P, 8, h);
    printf("ok\n");
    return 0;
}
