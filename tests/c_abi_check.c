/*
 * The C-ABI of libgemm_f16f32.so used from plain C, with no Python and no torch: device
 * memory from the HIP runtime, one default call, one strided call with a column-major C, one
 * split-K call with a workspace, and the host-side error codes.  Built by
 * dense_gemm_f16f32_amd/build.py (gcc, C99) next to this file; run by tests/test_gpu_boundary.py.
 *
 * Usage: c_abi_check M N K in.bin out.bin
 *   in.bin:  A (M x K, row-major) then B (K x N, row-major), IEEE binary16 bit patterns.
 *   out.bin: C three times (M x N, row-major each): from gemm_f16f32, from gemm_f16f32_strided
 *            into a column-major C (transposed back here), and from gemm_f16f32_strided_ws
 *            with split_k = 4.
 * Prints one line per check; exits non-zero on the first failure.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "gemm_f16f32.h"

#define HIP_OK(x)                                                         \
    do {                                                                  \
        hipError_t e_ = (x);                                              \
        if (e_ != hipSuccess) {                                           \
            fprintf(stderr, "HIP error %s: %s\n", #x, hipGetErrorString(e_)); \
            return 2;                                                     \
        }                                                                 \
    } while (0)

#define EXPECT(what, got, want)                                                        \
    do {                                                                               \
        long long g_ = (long long)(got), w_ = (long long)(want);                       \
        printf("%s: %lld (want %lld)\n", what, g_, w_);                                \
        if (g_ != w_) return 1;                                                        \
    } while (0)

int main(int argc, char **argv) {
    if (argc != 6) {
        fprintf(stderr, "usage: %s M N K in.bin out.bin\n", argv[0]);
        return 2;
    }
    const int64_t M = atoll(argv[1]), N = atoll(argv[2]), K = atoll(argv[3]);
    const size_t na = (size_t)(M * K), nb = (size_t)(K * N), nc = (size_t)(M * N);
    uint16_t *h = (uint16_t *)malloc((na + nb + 3 * nc) * sizeof(uint16_t));
    if (!h) return 2;
    FILE *f = fopen(argv[4], "rb");
    if (!f || fread(h, sizeof(uint16_t), na + nb, f) != na + nb) return 2;
    fclose(f);

    uint16_t *A, *B, *C, *Ct;
    void *ws;
    HIP_OK(hipMalloc((void **)&A, na * 2 + 16));
    HIP_OK(hipMalloc((void **)&B, nb * 2 + 16));
    HIP_OK(hipMalloc((void **)&C, nc * 2 + 16));
    HIP_OK(hipMalloc((void **)&Ct, nc * 2 + 16));
    HIP_OK(hipMemcpy(A, h, na * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(B, h + na, nb * 2, hipMemcpyHostToDevice));
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));

    /* host-side checks: nothing is launched for these */
    EXPECT("negative M", gemm_f16f32(-1, N, K, A, B, C, K, N, N, s), GEMM_F16F32_ERR_DIM);
    EXPECT("lda < K", gemm_f16f32(M, N, K, A, B, C, K - 1, N, N, s), GEMM_F16F32_ERR_LD);
    EXPECT("C overlaps A", gemm_f16f32(M, N, K, A, B, A, K, N, N, s), GEMM_F16F32_ERR_OVERLAP);
    EXPECT("strerror is static text", gemm_f16f32_strerror(GEMM_F16F32_ERR_DIM) != NULL, 1);
    EXPECT("version", gemm_f16f32_version() >= 400, 1);

    gemm_f16f32_plan_info info;
    EXPECT("plan", gemm_f16f32_plan(M, N, K, A, B, C, K, N, N, NULL, &info), GEMM_F16F32_OK);
    printf("plan tile %d bm %d bn %d programs %d launches %d\n", info.tile, info.bm, info.bn,
           info.num_programs, info.launches);

    /* 1: the default call */
    EXPECT("gemm_f16f32", gemm_f16f32(M, N, K, A, B, C, K, N, N, s), GEMM_F16F32_OK);
    /* 2: column-major C (C[i][j] at Ct + j*M + i) */
    EXPECT("gemm_f16f32_strided", gemm_f16f32_strided(M, N, K, A, K, 1, B, N, 1, Ct, 1, M, s,
                                                      NULL),
           GEMM_F16F32_OK);
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(h + na + nb, C, nc * 2, hipMemcpyDeviceToHost));
    uint16_t *tmp = (uint16_t *)malloc(nc * 2);
    if (!tmp) return 2;
    HIP_OK(hipMemcpy(tmp, Ct, nc * 2, hipMemcpyDeviceToHost));
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) h[na + nb + nc + i * N + j] = tmp[j * M + i];

    /* 3: split K through the workspace entry point */
    gemm_f16f32_opts o = {0};
    o.split_k = 4;
    gemm_f16f32_plan_info sp;
    EXPECT("split plan", gemm_f16f32_strided_plan(M, N, K, A, K, 1, B, N, 1, C, N, 1, &o, &sp),
           GEMM_F16F32_OK);
    printf("split slices %d depth %d workspace %lld\n", sp.splits, sp.split_depth,
           (long long)sp.workspace_bytes);
    EXPECT("split without workspace",
           gemm_f16f32_strided(M, N, K, A, K, 1, B, N, 1, C, N, 1, s, &o),
           sp.splits > 1 ? GEMM_F16F32_ERR_WORKSPACE : GEMM_F16F32_OK);
    const int64_t wsb = sp.workspace_bytes > 0 ? sp.workspace_bytes : 16;
    HIP_OK(hipMalloc(&ws, (size_t)wsb));
    EXPECT("gemm_f16f32_strided_ws",
           gemm_f16f32_strided_ws(M, N, K, A, K, 1, B, N, 1, C, N, 1, ws, wsb, s, &o),
           GEMM_F16F32_OK);
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(h + na + nb + 2 * nc, C, nc * 2, hipMemcpyDeviceToHost));

    f = fopen(argv[5], "wb");
    if (!f || fwrite(h + na + nb, sizeof(uint16_t), 3 * nc, f) != 3 * nc) return 2;
    fclose(f);
    HIP_OK(hipStreamDestroy(s));
    HIP_OK(hipFree(A));
    HIP_OK(hipFree(B));
    HIP_OK(hipFree(C));
    HIP_OK(hipFree(Ct));
    HIP_OK(hipFree(ws));
    free(tmp);
    free(h);
    printf("done\n");
    return 0;
}
