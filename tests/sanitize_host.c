/*
 * Drives the host side of libgemm_f16f32 (argument checks, storage-order normalisation, tile
 * choice, edge split, split K, error strings) over a large seeded sample of valid and invalid
 * arguments, for a host-only build under AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_sanitizers.py).  Nothing is launched: the plan entry points touch no GPU, and
 * the launching entry points are called only with arguments their plan rejects or an empty
 * C.  Pointers are fake, never dereferenced.  Prints counts and "ok"; sanitizers abort the
 * process on the first finding.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gemm_f16f32.h"

/* The library's host side imports a few HIP runtime entry points (kernel registration and
 * launch).  This program runs without a GPU and without the HIP runtime: these inert
 * definitions satisfy them.  Registration does nothing; a launch is counted and fails, and
 * the program requires that none was attempted.  FATBIN_SYM names the device-code blob the
 * host-only build refers to (taken from the built library's undefined symbols). */
typedef struct { unsigned x, y, z; } dim3_t;
char FATBIN_SYM[64];
static long launch_attempts = 0;
void **__hipRegisterFatBinary(const void *data) { static void *h; (void)data; return &h; }
void __hipRegisterFunction(void **m, const void *f, char *d, const char *n, unsigned t, void *a,
                           void *b, void *c, void *e, int *w)
{
    (void)m, (void)f, (void)d, (void)n, (void)t, (void)a, (void)b, (void)c, (void)e, (void)w;
}
void __hipUnregisterFatBinary(void **m) { (void)m; }
int __hipPushCallConfiguration(dim3_t g, dim3_t b, size_t s, void *q)
{
    (void)g, (void)b, (void)s, (void)q;
    return 0;
}
int __hipPopCallConfiguration(dim3_t *g, dim3_t *b, size_t *s, void **q)
{
    (void)g, (void)b, (void)s, (void)q;
    return 0;
}
int hipLaunchKernel(const void *f, dim3_t g, dim3_t b, void **a, size_t s, void *q)
{
    (void)f, (void)g, (void)b, (void)a, (void)s, (void)q;
    ++launch_attempts;
    return 1; /* an error code: the library reports GEMM_F16F32_ERR_HIP */
}
int hipGetLastError(void) { return 0; }
void __hipRegisterVar(void **m, void *var, char *hv, const char *dv, int ext, size_t size,
                      int constant, int global)
{
    (void)m, (void)var, (void)hv, (void)dv, (void)ext, (void)size, (void)constant, (void)global;
}
/* One fake device, no streams of other devices; the static scratch's "address" is a fake
 * pointer that is never dereferenced (nothing is launched). */
int hipGetDevice(int *d) { *d = 0; return 0; }
int hipStreamGetDevice(void *s, int *d) { (void)s; *d = 0; return 0; }
int hipGetSymbolAddress(void **p, const void *sym) { (void)sym; *p = (void *)(uintptr_t)0x4000000000ull; return 0; }

static uint64_t state = 0x2545F4914F6CDD1Dull;
static uint64_t next(void)
{
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return state;
}
static int64_t pick(const int64_t *v, int n) { return v[next() % (uint64_t)n]; }
/* the first n_valid entries of v are valid values: drawn 7 times in 8 */
static int64_t pick_mostly(const int64_t *v, int n_valid, int n)
{
    return (next() & 7) ? pick(v, n_valid) : pick(v, n);
}

int main(void)
{
    const int64_t dims[] = {0, 1, 2, 31, 32, 33, 63, 255, 256, 257, 1000, 4093, 4095, 4096,
                            4097, 8192, 65536, 1 << 20, ((int64_t)1 << 31) - 1,
                            (int64_t)1 << 31, -1, -((int64_t)1 << 40), (int64_t)1 << 62};
    const int64_t pads[] = {0, 0, 0, 1, 3, 8, 64, -1, -5, (int64_t)1 << 40, INT64_MAX / 4};
    const int64_t ptrs[] = {0x10000000, 0x10000002, 0x10000010, 0x7000000000, (int64_t)1 << 46,
                            0, 0x10000001};
    const int64_t opt_vals[] = {-3, -2, -1, 0, 0, 0, 1, 1, 2, 3, 4, 8, 16, 17, 33, 1 << 20};
    long plans = 0, ok = 0, runs = 0;
    for (int it = 0; it < 1000000; ++it) {
        const int64_t M = pick_mostly(dims, 18, 23), N = pick_mostly(dims, 18, 23),
                      K = pick_mostly(dims, 18, 23);
        const uint16_t *A = (const uint16_t *)(uintptr_t)pick_mostly(ptrs, 5, 7);
        const uint16_t *B =
            (const uint16_t *)(uintptr_t)(pick_mostly(ptrs, 5, 7) + ((int64_t)1 << 36));
        uint16_t *C = (uint16_t *)(uintptr_t)(pick_mostly(ptrs, 5, 7) + ((int64_t)1 << 37));
        gemm_f16f32_opts o;
        memset(&o, 0, sizeof o);
        const int use_opts = (int)(next() % 3);
        if (use_opts) {
            o.tile = (int32_t)pick(opt_vals, 16);
            o.group_m = (int32_t)pick(opt_vals, 16);
            o.xcd_remap = (int32_t)pick(opt_vals, 16) & 3;
            o.force_generic = (int32_t)(next() % 3);
            o.split_edges = (int32_t)(next() % 4);
            o.persistent = (int32_t)(next() % 4);
            o.split_k = (int32_t)pick(opt_vals, 16);
        }
        const gemm_f16f32_opts *op = use_opts ? &o : NULL;
        gemm_f16f32_plan_info info;
        int rc;
        if (next() & 1) {
            const int64_t lda = K + pick_mostly(pads, 7, 11), ldb = N + pick_mostly(pads, 7, 11),
                          ldc = N + pick_mostly(pads, 7, 11);
            rc = gemm_f16f32_plan(M, N, K, A, B, C, lda, ldb, ldc, op, &info);
            if (rc != GEMM_F16F32_OK || info.num_programs == 0) {
                (void)gemm_f16f32_ex(M, N, K, A, B, C, lda, ldb, ldc, NULL, op);
                ++runs;
            }
        } else {
            /* strides: row- or column-major per matrix, or something else */
            const int64_t la = pick_mostly(pads, 7, 11), lb = pick_mostly(pads, 7, 11),
                          lc = pick_mostly(pads, 7, 11);
            int64_t sam = K + la, sak = 1, sbk = N + lb, sbn = 1, scm = N + lc, scn = 1;
            if (next() & 1) sam = 1, sak = M + la;
            if (next() & 1) sbk = 1, sbn = K + lb;
            if (next() & 1) scm = 1, scn = M + lc;
            if ((next() & 31) == 0) sak = pick(pads, 11);
            rc = gemm_f16f32_strided_plan(M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, op,
                                          &info);
            const int64_t wsb = pick(dims, 23);
            void *ws = (void *)(uintptr_t)(pick(ptrs, 7) + ((int64_t)1 << 38));
            if (rc != GEMM_F16F32_OK || info.num_programs == 0) {
                (void)gemm_f16f32_strided(M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, NULL,
                                          op);
                (void)gemm_f16f32_strided_ws(M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, ws,
                                             wsb, NULL, op);
                (void)gemm_f16f32_strided_scratch(M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn,
                                                  NULL, op);
                runs += 3;
            } else if (use_opts && o.split_k >= 2 && info.splits > 1) {
                /* an explicit split with too small a workspace is refused before any launch
                   (the automatic choice would run unsplit instead) */
                if (wsb < info.workspace_bytes) {
                    if (gemm_f16f32_strided_ws(M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, ws,
                                               wsb, NULL, op) != GEMM_F16F32_ERR_WORKSPACE)
                        return 1;
                    ++runs;
                }
                /* likewise one that needs more than the static scratch */
                if (info.workspace_bytes > GEMM_F16F32_SCRATCH_BYTES) {
                    if (gemm_f16f32_strided_scratch(M, N, K, A, sam, sak, B, sbk, sbn, C, scm,
                                                    scn, NULL, op) != GEMM_F16F32_ERR_SCRATCH)
                        return 1;
                    ++runs;
                }
            }
        }
        ++plans;
        ok += rc == GEMM_F16F32_OK;
    }
    for (int code = -20; code <= 5; ++code)
        if (gemm_f16f32_strerror(code) == NULL) return 1;
    if (gemm_f16f32_tile_map(0, 1, 1, 1, NULL, NULL) != GEMM_F16F32_ERR_DIM ||
        gemm_f16f32_tile_map(1, 1, 0, 1, NULL, NULL) != GEMM_F16F32_ERR_OPTS ||
        gemm_f16f32_tile_map(1, 1, 1, 1, NULL, NULL) != GEMM_F16F32_ERR_NULL ||
        gemm_f16f32_tile_map(1 << 20, 1 << 20, 1, 1, NULL, NULL) != GEMM_F16F32_ERR_DIM)
        return 1;
    if (launch_attempts != 0) {
        printf("%ld launches attempted\n", launch_attempts);
        return 1;
    }
    printf("plans %ld (valid %ld), refused or empty calls %ld, version %d\nok\n", plans, ok,
           runs, gemm_f16f32_version());
    return 0;
}
