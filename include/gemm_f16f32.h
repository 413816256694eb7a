/*
 * gemm_f16f32: C = A B on one MI355X (gfx950), fp16 operands, fp32 accumulation, one
 * narrowing to fp16 on the store, output tiles visited in grouped GROUP_SIZE_M order.
 *
 * The operation is the matmul of phobos "03: Matrix multiplication" (the `matmul` kernel,
 * its docstring and the paragraph after it): A is M x K, B is K x N, C is M x N, every
 * element C[i][j] is the fp32 sum over k of A[i][k] * B[k][j], rounded once to fp16 (round
 * to nearest, ties to even, as a `.to(float16)` narrowing does).  Inside fp32 the order of
 * the k-sum is the kernel's own; results agree with the exactly rounded sum within
 * 1e-2 + 2^-10 |C| element-wise.  There is no alpha/beta: C is overwritten, never read.
 *
 * The launch order of output tiles is the grouped order of the kernl notebook "Computing
 * coordinates on Triton GEMM example" (introduction excerpt, cells In[1]-In[7]): with
 * num_pid_m = cdiv(M, BM) and num_pid_n = cdiv(N, BN) tiles per axis, program pid belongs to
 * group pid / (G * num_pid_n), groups cover G tile-rows (the last one may be smaller) and
 * programs inside a group run column-major.  Before that map the hardware workgroup id may
 * be permuted so that consecutive program ids share one XCD's L2 (gemm_f16f32_tile_map
 * documents the permutation).
 *
 * Layout: gemm_f16f32, gemm_f16f32_ex and gemm_f16f32_plan take row-major matrices with unit
 * stride along a row and a leading dimension (elements between the starts of consecutive
 * rows): A[i][k] is at A + i*lda + k, B[k][j] at B + k*ldb + j, C[i][j] at C + i*ldc + j.
 * gemm_f16f32_strided takes the notebook's general form (cell In[8] derives every pointer
 * from stride_am, stride_ak, stride_bk, stride_bn): A[i][k] at A + i*stride_am +
 * k*stride_ak, and likewise for B and C, with one unit stride per matrix (row- or
 * column-major storage, any leading dimension).  Values are IEEE binary16 bit patterns passed
 * as uint16_t.
 *
 * Ownership and execution: A, B, C (and the split-K workspace of gemm_f16f32_strided_ws) are
 * device pointers owned by the caller.  The library allocates nothing and keeps no state
 * between calls, so calls from several host threads are safe -- except for
 * gemm_f16f32_strided_scratch, whose split-K workspace is one static device array per GPU
 * (see there).  A call checks its arguments,
 * launches on `stream` (a hipStream_t; NULL is the null stream) and returns without waiting;
 * faults inside a kernel surface at the caller's next synchronisation.  Only C[i][j] with i < M, j < N is written (padding between N and ldc is
 * left as it was).  M == 0 or N == 0 is a successful no-op; K == 0 writes +0 to the M x N
 * block.
 *
 * Errors: every entry point returns GEMM_F16F32_OK (0) or a negative code; argument errors
 * are found on the host before anything is launched.
 */
#ifndef GEMM_F16F32_H
#define GEMM_F16F32_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    GEMM_F16F32_OK = 0,
    GEMM_F16F32_ERR_DIM = -1,       /* M, N or K negative, or >= 2^31 */
    GEMM_F16F32_ERR_NULL = -2,      /* a NULL pointer for a non-empty operand */
    GEMM_F16F32_ERR_LD = -3,        /* lda < max(K,1), ldb < max(N,1) or ldc < max(N,1);
                                       strided: a matrix with no unit stride, or a leading
                                       stride below its row (column) length */
    GEMM_F16F32_ERR_OVERLAP = -4,   /* C's footprint overlaps A's or B's */
    GEMM_F16F32_ERR_OPTS = -5,      /* an option outside its range, or an odd pointer address */
    GEMM_F16F32_ERR_TOO_LARGE = -6, /* a leading dimension beyond the kernels' 32-bit offsets:
                                       BM * ldc, and for each operand (rows of one stored
                                       panel) * ld must stay below 2^31, where a panel has BM
                                       (BN) rows when k is the unit-stride axis, else one row
                                       per k value of the panel (the tile's BK, 32-128; 64 on
                                       the generic path); with split K also BM * ldw * 4
                                       bytes, M * ldw / 4 and the grid splits * programs
                                       (ldw = N rounded up to 4).  A tile the library chose
                                       that fails this gives way to the 32 x 32 x 64 tile
                                       first; a forced tile does not. */
    GEMM_F16F32_ERR_HIP = -7,       /* the HIP runtime rejected the launch */
    GEMM_F16F32_ERR_WORKSPACE = -8, /* split K planned but no workspace (an entry point without
                                       one), or the workspace is smaller than
                                       plan_info.workspace_bytes or not 16-byte aligned */
    GEMM_F16F32_ERR_SCRATCH = -9    /* gemm_f16f32_strided_scratch: the split asked for needs
                                       more than GEMM_F16F32_SCRATCH_BYTES of workspace, or
                                       `stream` belongs to a device other than the current
                                       one */
};

/* Tile configurations: BM x BN x BK, computed by a workgroup of wavefronts (64 lanes each)
 * that each accumulate a block of C with 32x32x16 fp16 MFMAs (tile 1: 16x16x32).  Unless
 * noted, 4 wavefronts in a 2 x 2 arrangement (256 threads).  BK is the k depth of one
 * LDS-staged panel of the DMA path; the generic path stages 64-deep panels for every tile.
 * Every tile gives the same result bit for bit (each element's k-sum is the same sequence of
 * 16-deep MFMA steps; a 32-deep 16x16x32 step sums exactly as two of them). */
enum {
    GEMM_F16F32_TILE_AUTO = 0,
    GEMM_F16F32_TILE_256x256x64 = 1,     /* 16x16x32 MFMAs; panels in five 32 KiB LDS slots */
    GEMM_F16F32_TILE_128x128x64 = 2,     /* 2 stages, operands read 3 k steps ahead */
    GEMM_F16F32_TILE_128x64x64 = 3,      /* 2 stages */
    GEMM_F16F32_TILE_256x128x64 = 4,     /* 2 stages, operands read 3 k steps ahead */
    GEMM_F16F32_TILE_256x256x32 = 5,     /* 4 stages */
    GEMM_F16F32_TILE_64x64x32 = 6,       /* 5 stages */
    GEMM_F16F32_TILE_128x64x32 = 7,      /* 5 stages */
    GEMM_F16F32_TILE_256x256x64_W8 = 8,  /* 8 wavefronts (2 x 4, 512 threads, two per SIMD) */
    GEMM_F16F32_TILE_64x64x64 = 9,       /* 4 stages, read 3 ahead */
    GEMM_F16F32_TILE_32x32x64 = 10,      /* 1 wavefront, 4 stages, read 3 ahead */
    GEMM_F16F32_TILE_32x64x64 = 11,      /* 2 wavefronts (1 x 2), 4 stages, read 3 ahead */
    GEMM_F16F32_TILE_64x32x64 = 12,      /* 2 wavefronts (2 x 1), 4 stages, read 3 ahead */
    GEMM_F16F32_TILE_32x64x128 = 13,     /* 2 wavefronts (1 x 2), 4 stages, read 3 ahead */
    GEMM_F16F32_TILE_64x64x128 = 14,     /* 3 stages, read 3 ahead */
    GEMM_F16F32_TILE_32x32x128 = 15,     /* 1 wavefront, 4 stages, read 3 ahead */
    GEMM_F16F32_TILE_64x32x128 = 16,     /* 2 wavefronts (2 x 1), 4 stages, read 3 ahead */
    GEMM_F16F32_TILE_256x256x32_PP = 17  /* 8 wavefronts (2 x 4), 16x16x32 MFMAs, ping-pong:
                                            the two waves of a SIMD take turns multiplying */
};

/* opts.split_k: the library chooses the number of k slices (see gemm_f16f32_opts). */
#define GEMM_F16F32_SPLIT_K_AUTO (-1)

/* Kernel families.  Both accept any shape, leading dimension and 2-byte alignment. */
enum {
    GEMM_F16F32_PATH_DMA = 0,     /* default: 16-byte buffer->LDS loads of full BK-deep
                                     panels; when BK does not divide K the first panel holds
                                     the K mod BK leading k values, zero-padded in front */
    GEMM_F16F32_PATH_GENERIC = 1  /* only when forced: panels staged through registers,
                                     zero fill past K in the last panel */
};

/* Options for gemm_f16f32_ex.  Zero-initialised options mean "library default" throughout. */
typedef struct gemm_f16f32_opts {
    int32_t tile;          /* GEMM_F16F32_TILE_*; 0 = chosen from the shape */
    int32_t group_m;       /* GROUP_SIZE_M >= 1; 0 = library default for the tile */
    int32_t xcd_remap;     /* 0 = default (on), 1 = on, 2 = off (hardware id = program id) */
    int32_t force_generic; /* 1 = use the generic (register-staged) path */
    int32_t split_edges;   /* 0 = default (on when the tile is chosen by the library), 1 = on,
                              2 = off.  When the last tile column holds <= 1/4 of a tile's
                              columns (or the last tile row <= 1/4 of its rows) and the rest
                              spans >= 128 tiles, that sliver is computed by separate launches
                              with tiles sized for it; results are unchanged. */
    int32_t persistent;    /* 0 = default (off), 1 = persistent grouped schedule: the DMA path
                              launches one round of workgroups (256 CUs x as many per CU as fit
                              in LDS, a multiple of 8) and workgroup h computes programs h,
                              h + grid, ... through the same map; results are unchanged. 2 = off */
    int32_t split_k;       /* 0 or 1 = no split (default).  S >= 2: split K into at most S slices
                              of L = roundup(cdiv(K, S), 128) k values, cut from the end of k
                              (the first slice holds the rest), when K > L.  Each slice's fp32
                              tile sums go to a caller workspace (gemm_f16f32_strided_ws), a
                              second kernel adds the slices in order in fp32 and narrows once.
                              Results then depend on L (not on the tile) and stay within the
                              tolerance of the unsplit sum.  The tile is chosen for M x N x L;
                              no edge split; not with force_generic or persistent = 1 (ERR_OPTS).
                              Helps when M x N has too few tiles to fill the chip and K is deep.
                              GEMM_F16F32_SPLIT_K_AUTO (-1): the library picks S from the shape
                              (S = 1 when a split would not pay); only gemm_f16f32_strided_ws
                              acts on it, and only when its workspace holds the plan's
                              workspace_bytes (otherwise, and for the other entry points, the
                              call runs unsplit).  Plans report the automatic choice. */
} gemm_f16f32_opts;

/* What a call with these arguments would launch (filled by gemm_f16f32_plan).  The fields
 * describe the main launch, over C[0:main_m, 0:main_n]; edge strips, if any, follow it. */
typedef struct gemm_f16f32_plan_info {
    int32_t path;          /* GEMM_F16F32_PATH_* */
    int32_t tile;          /* GEMM_F16F32_TILE_* actually used */
    int32_t bm, bn, bk;    /* tile sizes (bk: panel depth of the kernel chosen) */
    int32_t group_m;       /* GROUP_SIZE_M actually used */
    int32_t xcd_remap;     /* 1 if the XCD permutation is applied */
    int32_t num_pid_m;     /* cdiv(M, bm) */
    int32_t num_pid_n;     /* cdiv(N, bn) */
    int32_t num_programs;  /* num_pid_m * num_pid_n = workgroups launched (0 if none) */
    int32_t launches;      /* kernel launches the call makes (1 + edge strips; 0 if empty) */
    int32_t main_m;        /* rows of C covered by the launch described above */
    int32_t main_n;        /* columns of C covered by the launch described above */
    int32_t a_kmajor;      /* 1: the launch's first operand has consecutive k adjacent in
                              memory (A row-major); 0: consecutive rows adjacent */
    int32_t b_kmajor;      /* 1: the launch's second operand has consecutive k adjacent (B
                              column-major); 0: consecutive columns adjacent (B row-major) */
    int32_t swapped;       /* 1: C is column-major and the launch computes C^T = B^T A^T; its
                              first operand is then B^T, and bm, num_pid_m, main_m run along
                              N, bn, num_pid_n, main_n along M */
    int32_t threads;       /* workgroup size of the main launch */
    int32_t persistent;    /* 1 if the main launch uses the persistent schedule */
    int32_t grid;          /* workgroups of the main launch (num_programs unless persistent;
                              splits * num_programs when split) */
    int32_t splits;        /* k slices (1 = no split K) */
    int32_t split_depth;   /* k values per slice L (0 = no split K) */
    int32_t strip_n;       /* columns of C right of main_n (rows, when swapped, below it)
                              that the main launch computes itself: the ping-pong tile takes a
                              last tile column of 1-16 columns into the tile rows' workgroups
                              (0 = none; otherwise such a sliver is a launch of its own) */
    int64_t workspace_bytes; /* workspace the call needs, splits * M' * roundup(N', 4) * 4 bytes
                              where M' x N' is the launch's C (M x N, or N x M when swapped):
                              slice z's fp32 sums at workspace + 4 (z M' + i) roundup(N', 4) + 4 j;
                              0 without split K */
} gemm_f16f32_plan_info;

/*
 * C[0:M, 0:N] = fp16( A[0:M, 0:K] . B[0:K, 0:N] ), fp32 accumulation, default options.
 * M, N, K: problem sizes (>= 0).  A, B, C: device pointers (see Layout).  lda >= max(K,1),
 * ldb >= max(N,1), ldc >= max(N,1).  stream: hipStream_t or NULL.
 */
int gemm_f16f32(int64_t M, int64_t N, int64_t K, const uint16_t *A, const uint16_t *B,
                uint16_t *C, int64_t lda, int64_t ldb, int64_t ldc, void *stream);

/* Same as gemm_f16f32 with explicit options (opts may be NULL = defaults). */
int gemm_f16f32_ex(int64_t M, int64_t N, int64_t K, const uint16_t *A, const uint16_t *B,
                   uint16_t *C, int64_t lda, int64_t ldb, int64_t ldc, void *stream,
                   const gemm_f16f32_opts *opts);

/* Host only, no GPU work: validates like gemm_f16f32_ex and reports in *info which kernel,
 * tile, GROUP_SIZE_M and grid that call would use.  Pointers are inspected for alignment and
 * overlap only, never dereferenced. */
int gemm_f16f32_plan(int64_t M, int64_t N, int64_t K, const uint16_t *A, const uint16_t *B,
                     const uint16_t *C, int64_t lda, int64_t ldb, int64_t ldc,
                     const gemm_f16f32_opts *opts, gemm_f16f32_plan_info *info);

/*
 * C[0:M, 0:N] = fp16( A[0:M, 0:K] . B[0:K, 0:N] ) for matrices given by element strides, the
 * general form of the notebook's cell In[8]: A[i][k] at A + i*stride_am + k*stride_ak,
 * B[k][j] at B + k*stride_bk + j*stride_bn, C[i][j] at C + i*stride_cm + j*stride_cn.
 * Each matrix must be row-major (column stride 1, row stride >= its column count) or
 * column-major (row stride 1, column stride >= its row count); a stride along an axis of
 * extent 1 is ignored, and an empty matrix may have any strides.  Anything else returns
 * GEMM_F16F32_ERR_LD.  All four storage orders of A and B run on the same kernels (an
 * operand stored with k contiguous is staged as rows of k, the other order as rows of i or
 * j), and every element gets the same fp32 k-sum as in the row-major call, bit for bit.  A
 * column-major C is computed as its transpose, C^T = B^T A^T.  Other arguments, ownership,
 * asynchrony and errors as for gemm_f16f32_ex.
 */
int gemm_f16f32_strided(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t stride_am,
                        int64_t stride_ak, const uint16_t *B, int64_t stride_bk,
                        int64_t stride_bn, uint16_t *C, int64_t stride_cm, int64_t stride_cn,
                        void *stream, const gemm_f16f32_opts *opts);

/*
 * gemm_f16f32_strided with a caller-owned device workspace for split K (opts->split_k >= 2):
 * workspace must be 16-byte aligned, hold at least the plan's workspace_bytes, and overlap
 * none of A, B, C (ERR_WORKSPACE, ERR_OVERLAP otherwise).  The call launches the slice
 * kernel and the reduction on `stream`, one after the other; the workspace is scratch that is
 * read and written by those two kernels only and may be reused once they are done (stream
 * order), so calls in flight at the same time need separate workspaces.  Without a split
 * (split_k 0 or 1, or K no deeper than one slice) the workspace is not touched and the call is
 * gemm_f16f32_strided.  The other entry points return ERR_WORKSPACE when split_k asks for a
 * split that would take place.
 */
int gemm_f16f32_strided_ws(int64_t M, int64_t N, int64_t K, const uint16_t *A,
                           int64_t stride_am, int64_t stride_ak, const uint16_t *B,
                           int64_t stride_bk, int64_t stride_bn, uint16_t *C, int64_t stride_cm,
                           int64_t stride_cn, void *workspace, int64_t workspace_bytes,
                           void *stream, const gemm_f16f32_opts *opts);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): gemm_f16f32_strided_ws without a workspace
 * argument.  A split (opts->split_k >= 2, or GEMM_F16F32_SPLIT_K_AUTO) keeps its fp32 slices
 * in a file-scope device array of GEMM_F16F32_SCRATCH_BYTES (16 MiB) that each GPU the
 * library runs on holds until the process ends; the call allocates nothing and calls no
 * allocating routine.  Its device address is looked up once per device, on the first call
 * made with that device current (hipGetSymbolAddress); `stream` must belong to the current
 * device (ERR_SCRATCH otherwise; NULL is the current device's null stream).  An explicit
 * split whose plan needs more than GEMM_F16F32_SCRATCH_BYTES returns ERR_SCRATCH before
 * anything is launched; the automatic split falls back to no split when it would not fit.
 * Nothing in the array needs to start at zero: the slice kernel writes every element the
 * reduction adds into C before the reduction reads it.  Every call on one GPU shares that
 * GPU's array, so calls that may overlap in time on one GPU (different streams, or different
 * host threads) race on it and give wrong results; calls ordered on one stream are safe.
 * Results are those of gemm_f16f32_strided_ws with the same arguments, bit for bit.
 */
#define GEMM_F16F32_SCRATCH_BYTES ((int64_t)16 << 20)
int gemm_f16f32_strided_scratch(int64_t M, int64_t N, int64_t K, const uint16_t *A,
                                int64_t stride_am, int64_t stride_ak, const uint16_t *B,
                                int64_t stride_bk, int64_t stride_bn, uint16_t *C,
                                int64_t stride_cm, int64_t stride_cn, void *stream,
                                const gemm_f16f32_opts *opts);

/* Host only, no GPU work: what gemm_f16f32_strided (or, with split_k, gemm_f16f32_strided_ws)
 * with these arguments would launch, including the workspace a split needs. */
int gemm_f16f32_strided_plan(int64_t M, int64_t N, int64_t K, const uint16_t *A,
                             int64_t stride_am, int64_t stride_ak, const uint16_t *B,
                             int64_t stride_bk, int64_t stride_bn, const uint16_t *C,
                             int64_t stride_cm, int64_t stride_cn, const gemm_f16f32_opts *opts,
                             gemm_f16f32_plan_info *info);

/*
 * Writes, for every hardware workgroup id h in [0, P), P = num_pid_m * num_pid_n, the
 * triple (logical program id, pid_m, pid_n) to out_dev[3h], out_dev[3h+1], out_dev[3h+2]
 * (device memory, 3P int32 owned by the caller), computed on the GPU by the same device
 * function the GEMM kernels use.  xcd_remap 1: logical id = x*q + min(x, r) + h/8 with
 * x = h % 8, q = P / 8, r = P % 8 (the 8 XCDs receive workgroups round-robin, so each XCD's
 * workgroups get one contiguous run of program ids); xcd_remap 0 (or 2): logical id = h.
 * The grouped map of the kernl notebook's introduction excerpt then gives (pid_m, pid_n).
 * Errors: GEMM_F16F32_ERR_DIM if a size is < 1 or P >= 2^31, ERR_OPTS for group_m < 1 or
 * xcd_remap outside 0..2, ERR_NULL for a NULL out_dev, ERR_HIP for a rejected launch.
 */
int gemm_f16f32_tile_map(int32_t num_pid_m, int32_t num_pid_n, int32_t group_m,
                         int32_t xcd_remap, int32_t *out_dev, void *stream);

/* Static description of an error code (never NULL). */
const char *gemm_f16f32_strerror(int code);

/* Library version as major*10000 + minor*100 + patch. */
int gemm_f16f32_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_F16F32_H */
