// C-ABI of the gfx950 fp16/fp32-accumulate GEMM: argument checks, kernel choice, launch.
// The declarations and their contracts are in include/gemm_f16f32.h.
#include "gemm_f16f32.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <mutex>

#include "gemm_kernels.hpp"
#include "gemm_tiles.hpp"

// Split-K workspace of gemm_f16f32_strided_scratch: one array per GPU, resident from the
// library's code-object load until the process ends.  In host code `scratch` only names the
// symbol; its device address comes from hipGetSymbolAddress, once per device, and only that
// address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[GEMM_F16F32_SCRATCH_BYTES];

namespace {

constexpr int kVersion = 500;  // 0.5.0
constexpr int kCUs = 256;       // compute units of an MI355X (persistent grid width, split-K grid budget)

struct TileDesc {
  int id, bm, bn, bk, stages, read_ahead, wm, wn, default_group;
};

#define GEMM_F16F32_TILE_DESC(id, bm, bn, bk, ns, rd, wm, wn, g) {id, bm, bn, bk, ns, rd, wm, wn, g},
constexpr TileDesc kTiles[] = {GEMM_F16F32_TILES(GEMM_F16F32_TILE_DESC)};
#undef GEMM_F16F32_TILE_DESC

const TileDesc* find_tile(int id) {
  for (const TileDesc& t : kTiles)
    if (t.id == id) return &t;
  return nullptr;
}

int64_t cdiv(int64_t x, int64_t y) { return (x + y - 1) / y; }

// LDS bytes of a tile's DMA kernels: its stages of A and B panels, or, for the 256 x 256 x 64
// tile on 2 x 2 wavefronts, the five 32 KiB panel slots its kernels keep instead.
int64_t dma_lds_bytes(const TileDesc* t) {
  if (t->bm == 256 && t->bn == 256 && t->bk == 64 && t->stages == 2 && t->wm == 2 && t->wn == 2)
    return 5 * 32768;
  return (int64_t)t->stages * (t->bm + t->bn) * t->bk * 2;
}

// Tile chosen from the shape when no table entry applies: the largest tile whose grid still
// covers the 256 CUs about once; smaller problems fall back to smaller tiles so that more CUs
// take part.  Thin shapes (a side of at most 64) are latency bound over their whole K and
// take the 64 x 64 tile with 32-deep panels and 5 LDS stages, which keeps 4 panels in flight.
int heuristic_tile(int64_t M, int64_t N) {
  if (cdiv(M, 256) * cdiv(N, 256) >= 240) return GEMM_F16F32_TILE_256x256x64;
  if (cdiv(M, 256) * cdiv(N, 128) >= 240) return GEMM_F16F32_TILE_256x128x64;
  if (cdiv(M, 128) * cdiv(N, 128) >= 120) return GEMM_F16F32_TILE_128x128x64;
  if (M <= 64 || N <= 64) return GEMM_F16F32_TILE_64x64x32;
  return GEMM_F16F32_TILE_128x64x64;
}

// The dispatch table measured offline by tune.py: for each shape class (rounded log2 of M,
// N and K) the fastest tile and, where it mattered, GROUP_SIZE_M (0 = the tile's default) and
// the XCD permutation (0 = on, the default; 2 = off).
struct TuneEntry {
  int8_t lm, ln, lk, tile, group, remap;
};
constexpr TuneEntry kTune[] = {
#include "tune_table.inc"
    {-1, -1, -1, 0, 0, 0}};  // end marker

int log2_class(int64_t x, int lo, int hi) {
  const int l = x < 1 ? lo : (int)std::lround(std::log2((double)x));
  return l < lo ? lo : (l > hi ? hi : l);
}

struct Choice {
  int tile, group, remap;   // remap as in gemm_f16f32_opts: 0 default (on), 1 on, 2 off
};

// Tile and group size for an M x N x K launch: the table's entry for its shape class, else
// the heuristic with the tile's default group size.
Choice choose_tile(int64_t M, int64_t N, int64_t K) {
  const int lm = log2_class(M, 5, 13), ln = log2_class(N, 5, 13), lk = log2_class(K, 6, 13);
  Choice c = {heuristic_tile(M, N), 0, 0};
  for (const TuneEntry& e : kTune)
    if (e.lm == lm && e.ln == ln && e.lk == lk && find_tile(e.tile) != nullptr) {
      c = {e.tile, e.group, e.remap};
      break;
    }
  return c;
}

// Bytes from a matrix's first element to one past its last, for rows x cols at leading
// dimension ld (0 if empty); saturates at UINT64_MAX (rows, cols < 2^31 here, ld any value
// the caller passed, so the product is taken in 128 bits).
uint64_t footprint(int64_t rows, int64_t cols, int64_t ld) {
  if (rows <= 0 || cols <= 0) return 0;
  const __int128 b = 2 * ((__int128)(rows - 1) * ld + cols);
  return b > (__int128)UINT64_MAX ? UINT64_MAX : (uint64_t)b;
}

// Whether [a, a + na) and [b, b + nb) intersect, without forming either end address.
bool overlaps(const void* a, uint64_t na, const void* b, uint64_t nb) {
  if (na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x >= y ? x - y < nb : y - x < na;
}

// rows * ld >= limit, for rows, limit > 0 and any ld >= 0, without overflow.
bool product_reaches(int64_t rows, int64_t ld, int64_t limit) {
  return (__int128)rows * ld >= limit;
}

// A problem as the kernels see it: C (M x N, row-major, ldc) = A (M x K) B (K x N), each
// operand either k-major (consecutive k adjacent: A[i][k] at A + i*lda + k, B[k][j] at
// B + j*ldb + k) or x-major (A[i][k] at A + k*lda + i, B[k][j] at B + k*ldb + j).
// `swapped`: the caller's C is column-major and this is its transpose, C^T = B^T A^T.
struct Problem {
  int64_t M, N, K;
  const uint16_t* A;
  const uint16_t* B;
  const uint16_t* C;
  int64_t lda, ldb, ldc;
  bool a_kmajor, b_kmajor, swapped;
};

// Storage order of an R x S matrix with element strides sr (between rows) and sc (between
// columns): 0 = row-major (sc == 1, ld = sr >= S), 1 = column-major (sr == 1, ld = sc >= R),
// -1 = neither.  The stride along an axis of extent 1 is never used and is ignored; an empty
// matrix is never addressed and counts as row-major.
int order_of(int64_t R, int64_t S, int64_t sr, int64_t sc, int64_t* ld) {
  if (R == 0 || S == 0 || (R == 1 && S == 1)) {
    *ld = S > 1 ? S : 1;
    return 0;
  }
  if (R == 1) {  // one row: only sc is used
    if (sc == 1) {
      *ld = S;
      return 0;
    }
    *ld = sc;
    return sc >= 1 ? 1 : -1;
  }
  if (S == 1) {  // one column: only sr is used
    *ld = sr;
    return sr >= 1 ? 0 : -1;
  }
  if (sc == 1 && sr >= S) {
    *ld = sr;
    return 0;
  }
  if (sr == 1 && sc >= R) {
    *ld = sc;
    return 1;
  }
  return -1;
}

// 16-byte aligned rows of both operands (the dispatch table's measurement condition).
bool aligned_rows(const Problem& pr) {
  return (((uintptr_t)pr.A | (uintptr_t)pr.B) & 15) == 0 && pr.lda % 8 == 0 && pr.ldb % 8 == 0;
}

// Slices of the automatic split K.  A slice computes M x N x L on its own workgroups, so a
// split pays when the unsplit grid leaves most CUs idle and K is deep: one workgroup streams
// its panels through one CU at that CU's fetch rate, S slices through S CUs.  Measured on
// MI355X (graph-timed, M, N in 32 .. 4096, K in 1024 .. 8192): the best S kept the split grid
// (S times the programs of the tile chosen for M x N x L) within the 256 CUs and every slice
// at least 512 deep; two slices paid off only from K = 4096 on (the reduction's launch and
// fp32 traffic cost about 1-2 us).  So: the largest power of two S <= 16 with that grid
// within 256 and K >= 512 S, and S = 2 only for K >= 4096.
int auto_splits(int64_t M, int64_t N, int64_t K, int tile) {
  int best = 1;
  for (int S = 2; S <= 16 && K >= 512 * (int64_t)S; S *= 2) {
    const int64_t L = cdiv(cdiv(K, S), 128) * 128;
    const TileDesc* t = find_tile(tile ? tile : choose_tile(M, N, L).tile);
    if (cdiv(M, t->bm) * cdiv(N, t->bn) * S <= kCUs) best = S;
  }
  return (best == 2 && K < 4096) ? 1 : best;
}

// One launch over an M x N block of C (all of it, or one part of an edge split).
struct Part {
  int64_t m_off, n_off, M, N;
  gemm_f16f32_plan_info r;
};

// Fills r for one launch of tile `tile` over M x N (no argument checks here).
int plan_launch(const Problem& pr, int64_t M, int64_t N, const TileDesc* t, int group,
                int remap, const gemm_f16f32_opts& o, gemm_f16f32_plan_info* r) {
  const int64_t kMax = (int64_t)1 << 31;
  const bool dma = !o.force_generic;
  // 32-bit in-kernel offsets: one panel's stored rows of A (bm rows if k-major, else one k row
  // per k value of the panel: the tile's BK on the DMA path, 64 on the generic one) and of B
  // (bn, or the same k rows), and one tile's bm rows of C.
  const int64_t depth = dma ? t->bk : gk::kBK;
  const int64_t rows_a = pr.a_kmajor ? t->bm : depth, rows_b = pr.b_kmajor ? t->bn : depth;
  if (product_reaches(rows_a, pr.lda, kMax) || product_reaches(rows_b, pr.ldb, kMax) ||
      product_reaches(t->bm, pr.ldc, kMax))
    return GEMM_F16F32_ERR_TOO_LARGE;
  r->path = dma ? GEMM_F16F32_PATH_DMA : GEMM_F16F32_PATH_GENERIC;
  r->tile = t->id;
  r->bm = t->bm;
  r->bn = t->bn;
  r->bk = dma ? t->bk : gk::kBK;
  r->threads = 64 * t->wm * t->wn;
  r->group_m = o.group_m ? o.group_m : (group ? group : t->default_group);
  r->xcd_remap = ((o.xcd_remap ? o.xcd_remap : remap) == 2) ? 0 : 1;
  const bool empty = (M == 0 || N == 0);
  r->num_pid_m = empty ? 0 : (int32_t)cdiv(M, t->bm);
  r->num_pid_n = empty ? 0 : (int32_t)cdiv(N, t->bn);
  const int64_t P = (int64_t)r->num_pid_m * r->num_pid_n;
  if (P >= kMax) return GEMM_F16F32_ERR_TOO_LARGE;
  r->num_programs = (int32_t)P;
  // Persistent schedule (DMA path only): one round of workgroups over all CUs, as many per CU
  // as fit in LDS, rounded down to a multiple of the 8 XCDs; never more than the programs.
  r->persistent = dma && o.persistent == 1 && P > 0;
  r->grid = (int32_t)P;
  if (r->persistent) {
    const int64_t lds = dma_lds_bytes(t);
    const int64_t per_cu = lds > 0 ? (160 * 1024) / lds : 1;
    int64_t g = (int64_t)kCUs * (per_cu > 1 ? per_cu : 1);
    g -= g % 8;
    r->grid = (int32_t)(P < g ? P : g);
  }
  r->launches = empty ? 0 : 1;
  r->main_m = (int32_t)M;
  r->main_n = (int32_t)N;
  r->a_kmajor = pr.a_kmajor;
  r->b_kmajor = pr.b_kmajor;
  r->swapped = pr.swapped;
  r->splits = 1;
  r->split_depth = 0;
  r->strip_n = 0;
  r->workspace_bytes = 0;
  return GEMM_F16F32_OK;
}

// Split K over the whole M x N launch: slices of L = roundup(cdiv(K, S), 128) k values cut
// from the end of k (the first slice holds the rest), S' = cdiv(K, L) <= S of them.  Writes
// splits, split_depth, workspace_bytes (S' slices of M x ldw fp32, ldw = N rounded up to a
// multiple of 4), grid = S' P and launches = 2 (the slices, then the reduction).
int plan_split(const Problem& pr, int64_t L, gemm_f16f32_plan_info* r) {
  const int64_t kMax = (int64_t)1 << 31;
  const int64_t S = cdiv(pr.K, L);
  const int64_t ldw = cdiv(pr.N, 4) * 4;
  // 32-bit workspace offsets within one tile's rows; the x extent of the slice grid; the
  // reduction's 32-bit thread index (one thread per 4 workspace elements of a slice)
  if ((int64_t)r->bm * ldw * 4 >= kMax || S * r->num_programs >= kMax ||
      pr.M * (ldw / 4) >= kMax)
    return GEMM_F16F32_ERR_TOO_LARGE;
  r->splits = (int32_t)S;
  r->split_depth = (int32_t)L;
  r->workspace_bytes = S * pr.M * ldw * 4;
  r->grid = (int32_t)(S * r->num_programs);
  r->launches = 2;
  return GEMM_F16F32_OK;
}

// Argument checks, tile choice and the edge split.  parts[0] is the main block; parts[1..]
// are the thin strips (right, bottom, corner) when the split applies.  Returns the number of
// parts through *nparts.
//
// Edge split: when the last tile column holds at most a quarter of a tile's columns (or the
// last tile row a quarter of its rows) and the problem is large, those tiles would each do a
// full tile's work for a sliver of C and often cost a whole extra wave of workgroups.  The
// sliver is then computed by separate launches with tiles chosen for its own shape.  Every
// element's k-sum is the same sequence of MFMA steps whatever the tile, so results do not
// change.
//
// ws_bytes: the caller's split-K workspace (-1: the entry point takes none).  The automatic
// split (split_k = -1) is planned only when a workspace is given and used only when it fits.
int plan_parts(const Problem& pr, const gemm_f16f32_opts* opts, int64_t ws_bytes, Part* parts,
               int* nparts) {
  const int64_t kMax = (int64_t)1 << 31;
  const int64_t M = pr.M, N = pr.N, K = pr.K;
  *nparts = 0;
  if (M < 0 || N < 0 || K < 0 || M >= kMax || N >= kMax || K >= kMax) return GEMM_F16F32_ERR_DIM;
  const int64_t min_lda = pr.a_kmajor ? K : M, min_ldb = pr.b_kmajor ? K : N;
  if (pr.lda < (min_lda > 1 ? min_lda : 1) || pr.ldb < (min_ldb > 1 ? min_ldb : 1) ||
      pr.ldc < (N > 1 ? N : 1))
    return GEMM_F16F32_ERR_LD;
  const bool emptyC = (M == 0 || N == 0);
  if (!emptyC && pr.C == nullptr) return GEMM_F16F32_ERR_NULL;
  if (!emptyC && K > 0 && (pr.A == nullptr || pr.B == nullptr)) return GEMM_F16F32_ERR_NULL;
  if (((uintptr_t)pr.A | (uintptr_t)pr.B | (uintptr_t)pr.C) & 1) return GEMM_F16F32_ERR_OPTS;

  gemm_f16f32_opts o = {0, 0, 0, 0, 0, 0, 0};
  if (opts) o = *opts;
  if (o.tile != 0 && find_tile(o.tile) == nullptr) return GEMM_F16F32_ERR_OPTS;
  if (o.group_m < 0 || o.xcd_remap < 0 || o.xcd_remap > 2 || o.force_generic < 0 ||
      o.force_generic > 1 || o.split_edges < 0 || o.split_edges > 2 || o.persistent < 0 ||
      o.persistent > 2 || o.split_k < GEMM_F16F32_SPLIT_K_AUTO)
    return GEMM_F16F32_ERR_OPTS;
  if (o.split_k == GEMM_F16F32_SPLIT_K_AUTO) {
    const bool may = ws_bytes > 0 && !emptyC && o.force_generic != 1 && o.persistent != 1;
    const int S = may ? auto_splits(M, N, K, o.tile) : 1;
    if (S > 1) {
      gemm_f16f32_opts os = o;
      os.split_k = S;
      const int rc = plan_parts(pr, &os, ws_bytes, parts, nparts);
      if (rc == GEMM_F16F32_OK && parts[0].r.workspace_bytes <= ws_bytes) return rc;
    }
    o.split_k = 1;   // no split: not worth it, no workspace, or it does not fit
  }
  // Split K: asked for with split_k >= 2; it takes effect when K spans more than one slice.
  if (o.split_k >= 2 && (o.force_generic == 1 || o.persistent == 1))
    return GEMM_F16F32_ERR_OPTS;
  const int64_t L = o.split_k >= 2 ? cdiv(cdiv(K, o.split_k), 128) * 128 : 0;
  const bool split_k = L > 0 && K > L && !emptyC;

  if (!emptyC) {
    const uint64_t fc = footprint(M, N, pr.ldc);
    const uint64_t fa = pr.a_kmajor ? footprint(M, K, pr.lda) : footprint(K, M, pr.lda);
    const uint64_t fb = pr.b_kmajor ? footprint(N, K, pr.ldb) : footprint(K, N, pr.ldb);
    if (overlaps(pr.C, fc, pr.A, fa) || overlaps(pr.C, fc, pr.B, fb))
      return GEMM_F16F32_ERR_OVERLAP;
  }

  // A split problem is chosen for as the slices' own shape, M x N x L.
  Choice ch = o.tile ? Choice{o.tile, 0, 0} : choose_tile(M, N, split_k ? L : K);
  const bool split =
      !split_k && (o.split_edges == 1 || (o.split_edges == 0 && o.tile == 0));
  // A right sliver of 1..16 columns with misaligned rows (an odd leading dimension or a 2-byte
  // aligned start, where a 16-byte load of a panel row straddles one more cache line): where
  // the table picks the 256 x 256 x 64 tile, the ping-pong tile of the same size computes the
  // sliver inside its own launch instead of a second launch (measured on 4095 x 4097 x 4093:
  // 144 against 152 us).  Without such a sliver misaligned rows keep the table's tile.
  if (o.tile == 0 && split && !emptyC && ch.tile == GEMM_F16F32_TILE_256x256x64 &&
      !aligned_rows(pr) && o.force_generic != 1 && o.persistent != 1) {
    const int64_t rn = N % 256, rm = M % 256, fm = M / 256, fn = N / 256;
    const bool bottom = fm * fn >= 128 && rm > 0 && 4 * rm <= 256;
    if (rn > 0 && rn <= 16 && fn >= 16 && !bottom)
      ch = Choice{GEMM_F16F32_TILE_256x256x32_PP, 0, 0};
  }
  const TileDesc* t = find_tile(ch.tile);
  int64_t Mm = M, Nm = N;
  int64_t strip_n = 0;
  if (split && !emptyC) {
    const int64_t rm = M % t->bm, rn = N % t->bn;
    const int64_t full_m = M / t->bm, full_n = N / t->bn;
    if (full_m * full_n >= 128) {
      if (rn > 0 && 4 * rn <= t->bn) Nm = N - rn;
      if (rm > 0 && 4 * rm <= t->bm) Mm = M - rm;
    }
    // A right strip of at most 16 columns, with no bottom strip, is computed inside the
    // ping-pong tile's own launch when each tile row has at least 16 workgroups (one 16-row
    // block of the strip each); it costs one MFMA per panel in one wave, so it is taken at
    // any size.
    if (t->read_ahead == 0 && o.force_generic != 1 && o.persistent != 1 && rn > 0 &&
        rn <= 16 && full_n >= 16 && Mm == M) {
      Nm = N - rn;
      strip_n = rn;
    }
  }
  // A tile chosen here (not forced by the caller) that cannot address the operands with
  // 32-bit offsets -- a leading dimension of about 2^24 elements or more -- gives way to the
  // 32 x 32 x 64 tile, whose panels store the fewest rows, before the call is refused.
  auto plan_or_fallback = [&](int64_t m, int64_t n, const TileDesc* tt, int group, int remap,
                              bool forced, const gemm_f16f32_opts& oo,
                              gemm_f16f32_plan_info* r) {
    int rc = plan_launch(pr, m, n, tt, group, remap, oo, r);
    if (rc == GEMM_F16F32_ERR_TOO_LARGE && !forced && tt->id != GEMM_F16F32_TILE_32x32x64)
      rc = plan_launch(pr, m, n, find_tile(GEMM_F16F32_TILE_32x32x64), 0, 0, oo, r);
    return rc;
  };
  Part* pp = parts;
  pp->m_off = 0, pp->n_off = 0, pp->M = Mm, pp->N = Nm;
  int rc = plan_or_fallback(Mm, Nm, t, ch.group, ch.remap, o.tile != 0, o, &pp->r);
  if (rc != GEMM_F16F32_OK) return rc;
  if (split_k) {
    *nparts = 1;
    return plan_split(pr, L, &parts[0].r);
  }
  if (strip_n > 0 && pp->r.tile == t->id) {
    pp->r.strip_n = (int32_t)strip_n;
    Nm = N;   // no separate launch for it
  }
  ++pp;
  const int64_t strips[3][4] = {{0, Nm, Mm, N - Nm}, {Mm, 0, M - Mm, Nm}, {Mm, Nm, M - Mm, N - Nm}};
  gemm_f16f32_opts os = o;
  os.tile = 0;
  os.group_m = 0;
  for (const auto& st : strips) {
    if (st[2] == 0 || st[3] == 0) continue;
    pp->m_off = st[0], pp->n_off = st[1], pp->M = st[2], pp->N = st[3];
    const Choice cs = choose_tile(st[2], st[3], K);
    rc = plan_or_fallback(st[2], st[3], find_tile(cs.tile), cs.group, cs.remap, false, os, &pp->r);
    if (rc != GEMM_F16F32_OK) return rc;
    ++pp;
  }
  *nparts = (int)(pp - parts);
  parts[0].r.launches = emptyC ? 0 : *nparts;
  return GEMM_F16F32_OK;
}

template <int BM, int BN, int BK, int NS, int RD, int WM, int WN, bool AKM, bool BKM>
hipError_t launch_layout(const gemm_f16f32_plan_info& r, const gk::Args& a, bool odd,
                         hipStream_t stream) {
  const dim3 grid(r.grid), block(64 * WM * WN);
  if constexpr (RD == 0) {
    // the ping-pong tile on the DMA path
    if (r.path == GEMM_F16F32_PATH_DMA) {
      if (r.splits > 1)
        hipLaunchKernelGGL((gk::gemm_pp_splitk<AKM, BKM>), grid, block, 0, stream, a);
      else if (r.persistent)
        hipLaunchKernelGGL((gk::gemm_pp_persistent<AKM, BKM>), grid, block, 0, stream, a);
      else if (a.strip_n > 0)
        hipLaunchKernelGGL((gk::gemm_pp<AKM, BKM, true>), grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL((gk::gemm_pp<AKM, BKM, false>), grid, block, 0, stream, a);
      return hipGetLastError();
    }
  } else if (r.splits > 1) {
    hipLaunchKernelGGL((gk::gemm_dma_splitk<BM, BN, BK, NS, RD, WM, WN, AKM, BKM>), grid, block,
                       0, stream, a);
    return hipGetLastError();
  } else if (r.path == GEMM_F16F32_PATH_DMA && r.persistent) {
    hipLaunchKernelGGL((gk::gemm_dma_persistent<BM, BN, BK, NS, RD, WM, WN, AKM, BKM>), grid,
                       block, 0, stream, a);
    return hipGetLastError();
  } else if (r.path == GEMM_F16F32_PATH_DMA) {
    hipLaunchKernelGGL((gk::gemm_dma<BM, BN, BK, NS, RD, WM, WN, AKM, BKM>), grid, block, 0,
                       stream, a);
    return hipGetLastError();
  }
  if (odd)
    hipLaunchKernelGGL((gk::gemm_generic<BM, BN, true, WM, WN, AKM, BKM>), grid, block, 0,
                       stream, a);
  else
    hipLaunchKernelGGL((gk::gemm_generic<BM, BN, false, WM, WN, AKM, BKM>), grid, block, 0,
                       stream, a);
  return hipGetLastError();
}

// One tile configuration: BM x BN x BK, NS LDS stages, operands read RD k steps ahead,
// WM x WN wavefronts.
template <int BM, int BN, int BK, int NS, int RD, int WM, int WN>
hipError_t launch(const gemm_f16f32_plan_info& r, const gk::Args& a, bool odd,
                  hipStream_t stream) {
  if (r.a_kmajor)
    return r.b_kmajor
               ? launch_layout<BM, BN, BK, NS, RD, WM, WN, true, true>(r, a, odd, stream)
               : launch_layout<BM, BN, BK, NS, RD, WM, WN, true, false>(r, a, odd, stream);
  return r.b_kmajor
             ? launch_layout<BM, BN, BK, NS, RD, WM, WN, false, true>(r, a, odd, stream)
             : launch_layout<BM, BN, BK, NS, RD, WM, WN, false, false>(r, a, odd, stream);
}

// Launches one part; `ws` is the split-K workspace (used only when r.splits > 1).
int launch_part(const Problem& pr, const Part& pt, float* ws, hipStream_t s) {
  const gemm_f16f32_plan_info& r = pt.r;
  if (r.num_programs == 0) return GEMM_F16F32_OK;
  gk::Args a;
  a.A = pr.A + (pr.a_kmajor ? pt.m_off * pr.lda : pt.m_off);
  a.B = pr.B + (pr.b_kmajor ? pt.n_off * pr.ldb : pt.n_off);
  a.C = const_cast<uint16_t*>(pr.C) + pt.m_off * pr.ldc + pt.n_off;
  a.lda = pr.lda;
  a.ldb = pr.ldb;
  a.ldc = pr.ldc;
  a.M = (int32_t)pt.M;
  a.N = (int32_t)pt.N;
  a.K = (int32_t)pr.K;
  a.num_pid_m = r.num_pid_m;
  a.num_pid_n = r.num_pid_n;
  // A group of G >= num_pid_m tile rows maps every program as G = num_pid_m does; passing at
  // most num_pid_m keeps G * num_pid_n (<= the program count) inside the kernels' 32 bits.
  a.group_m = r.group_m < r.num_pid_m ? r.group_m : r.num_pid_m;
  a.xcd_remap = r.xcd_remap;
  a.num_programs = r.num_programs;
  a.W = ws;
  a.ldw = cdiv(pt.N, 4) * 4;
  a.splits = r.splits;
  a.panels_per_split = r.splits > 1 ? r.split_depth / r.bk : 0;
  a.strip_n = r.strip_n;
  const bool odd = (((uintptr_t)a.A | (uintptr_t)a.B) & 3) != 0 || ((pr.lda | pr.ldb) & 1) != 0;
  hipError_t e = hipSuccess;
  switch (r.tile) {
#define GEMM_F16F32_TILE_CASE(id, bm, bn, bk, ns, rd, wm, wn, g) \
  case id: e = launch<bm, bn, bk, ns, rd, wm, wn>(r, a, odd, s); break;
    GEMM_F16F32_TILES(GEMM_F16F32_TILE_CASE)
#undef GEMM_F16F32_TILE_CASE
    default: return GEMM_F16F32_ERR_OPTS;
  }
  if (e == hipSuccess && r.splits > 1) {
    const int64_t threads = pt.M * (a.ldw / 4);
    hipLaunchKernelGGL(gk::splitk_reduce, dim3((uint32_t)cdiv(threads, 256)), dim3(256), 0, s,
                       (const float*)ws, a.ldw, (int)r.splits, a.M, a.N, a.C, a.ldc);
    e = hipGetLastError();
  }
  return e == hipSuccess ? GEMM_F16F32_OK : GEMM_F16F32_ERR_HIP;
}

Problem row_major_problem(int64_t M, int64_t N, int64_t K, const uint16_t* A, const uint16_t* B,
                          const uint16_t* C, int64_t lda, int64_t ldb, int64_t ldc) {
  return Problem{M, N, K, A, B, C, lda, ldb, ldc, true, false, false};
}

// Problem for caller strides (A: sam, sak; B: sbk, sbn; C: scm, scn).  A column-major C is
// turned into its transpose, C^T = B^T A^T, with the operands' roles exchanged: B^T is k-major
// exactly when B is stored column-major, and A^T exactly when A is stored row-major.
int strided_problem(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t sam,
                    int64_t sak, const uint16_t* B, int64_t sbk, int64_t sbn, const uint16_t* C,
                    int64_t scm, int64_t scn, Problem* pr) {
  const int64_t kMax = (int64_t)1 << 31;
  if (M < 0 || N < 0 || K < 0 || M >= kMax || N >= kMax || K >= kMax) return GEMM_F16F32_ERR_DIM;
  int64_t lda = 0, ldb = 0, ldc = 0;
  const int oa = order_of(M, K, sam, sak, &lda);
  const int ob = order_of(K, N, sbk, sbn, &ldb);
  const int oc = order_of(M, N, scm, scn, &ldc);
  if (oa < 0 || ob < 0 || oc < 0) return GEMM_F16F32_ERR_LD;
  if (oc == 0)
    *pr = Problem{M, N, K, A, B, C, lda, ldb, ldc, oa == 0, ob == 1, false};
  else
    *pr = Problem{N, M, K, B, A, C, ldb, lda, ldc, ob == 1, oa == 0, true};
  return GEMM_F16F32_OK;
}

// Plans, checks the workspace against the plan (ws_bytes < 0: the entry point has none),
// then launches every part.
int run(const Problem& pr, void* stream, const gemm_f16f32_opts* opts, void* ws,
        int64_t ws_bytes) {
  Part parts[4];
  int n = 0;
  int rc = plan_parts(pr, opts, ws_bytes, parts, &n);
  if (rc != GEMM_F16F32_OK) return rc;
  const gemm_f16f32_plan_info& r = parts[0].r;
  if (n > 0 && r.splits > 1) {
    if (ws == nullptr || ws_bytes < r.workspace_bytes || ((uintptr_t)ws & 15) != 0)
      return GEMM_F16F32_ERR_WORKSPACE;
    const uint64_t fw = (uint64_t)r.workspace_bytes;
    const uint64_t fc = footprint(pr.M, pr.N, pr.ldc);
    const uint64_t fa = pr.a_kmajor ? footprint(pr.M, pr.K, pr.lda) : footprint(pr.K, pr.M, pr.lda);
    const uint64_t fb = pr.b_kmajor ? footprint(pr.N, pr.K, pr.ldb) : footprint(pr.K, pr.N, pr.ldb);
    if (overlaps(ws, fw, pr.C, fc) || overlaps(ws, fw, pr.A, fa) || overlaps(ws, fw, pr.B, fb))
      return GEMM_F16F32_ERR_OVERLAP;
  }
  for (int i = 0; i < n && rc == GEMM_F16F32_OK; ++i)
    rc = launch_part(pr, parts[i], (float*)ws, (hipStream_t)stream);
  return rc;
}

int plan(const Problem& pr, const gemm_f16f32_opts* opts, gemm_f16f32_plan_info* info) {
  Part parts[4];
  int n = 0;
  // the plan reports the automatic split as if a large enough workspace were given
  const int rc = plan_parts(pr, opts, INT64_MAX, parts, &n);
  if (rc == GEMM_F16F32_OK && info) *info = parts[0].r;
  return rc;
}

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices] = {};

// The scratch array's device address on the device `stream` runs on, which must be the
// current device (looked up with that device current on its first use).
int scratch_for_stream(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return GEMM_F16F32_ERR_HIP;
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return GEMM_F16F32_ERR_HIP;
    if (sdev != dev) return GEMM_F16F32_ERR_SCRATCH;
  }
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return GEMM_F16F32_ERR_HIP;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return GEMM_F16F32_OK;
}

}  // namespace

extern "C" {

int gemm_f16f32_plan(int64_t M, int64_t N, int64_t K, const uint16_t* A, const uint16_t* B,
                     const uint16_t* C, int64_t lda, int64_t ldb, int64_t ldc,
                     const gemm_f16f32_opts* opts, gemm_f16f32_plan_info* info) {
  return plan(row_major_problem(M, N, K, A, B, C, lda, ldb, ldc), opts, info);
}

int gemm_f16f32_ex(int64_t M, int64_t N, int64_t K, const uint16_t* A, const uint16_t* B,
                   uint16_t* C, int64_t lda, int64_t ldb, int64_t ldc, void* stream,
                   const gemm_f16f32_opts* opts) {
  return run(row_major_problem(M, N, K, A, B, C, lda, ldb, ldc), stream, opts, nullptr, -1);
}

int gemm_f16f32(int64_t M, int64_t N, int64_t K, const uint16_t* A, const uint16_t* B,
                uint16_t* C, int64_t lda, int64_t ldb, int64_t ldc, void* stream) {
  return gemm_f16f32_ex(M, N, K, A, B, C, lda, ldb, ldc, stream, nullptr);
}

int gemm_f16f32_strided(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t stride_am,
                        int64_t stride_ak, const uint16_t* B, int64_t stride_bk,
                        int64_t stride_bn, uint16_t* C, int64_t stride_cm, int64_t stride_cn,
                        void* stream, const gemm_f16f32_opts* opts) {
  Problem pr;
  const int rc = strided_problem(M, N, K, A, stride_am, stride_ak, B, stride_bk, stride_bn, C,
                                 stride_cm, stride_cn, &pr);
  return rc != GEMM_F16F32_OK ? rc : run(pr, stream, opts, nullptr, -1);
}

int gemm_f16f32_strided_ws(int64_t M, int64_t N, int64_t K, const uint16_t* A,
                           int64_t stride_am, int64_t stride_ak, const uint16_t* B,
                           int64_t stride_bk, int64_t stride_bn, uint16_t* C, int64_t stride_cm,
                           int64_t stride_cn, void* workspace, int64_t workspace_bytes,
                           void* stream, const gemm_f16f32_opts* opts) {
  Problem pr;
  const int rc = strided_problem(M, N, K, A, stride_am, stride_ak, B, stride_bk, stride_bn, C,
                                 stride_cm, stride_cn, &pr);
  return rc != GEMM_F16F32_OK ? rc : run(pr, stream, opts, workspace, workspace_bytes);
}

int gemm_f16f32_strided_scratch(int64_t M, int64_t N, int64_t K, const uint16_t* A,
                                int64_t stride_am, int64_t stride_ak, const uint16_t* B,
                                int64_t stride_bk, int64_t stride_bn, uint16_t* C,
                                int64_t stride_cm, int64_t stride_cn, void* stream,
                                const gemm_f16f32_opts* opts) {
  Problem pr;
  int rc = strided_problem(M, N, K, A, stride_am, stride_ak, B, stride_bk, stride_bn, C,
                           stride_cm, stride_cn, &pr);
  if (rc != GEMM_F16F32_OK) return rc;
  // An explicit split larger than the array is refused, not silently run unsplit.
  if (opts != nullptr && opts->split_k >= 2) {
    Part parts[4];
    int n = 0;
    rc = plan_parts(pr, opts, INT64_MAX, parts, &n);
    if (rc != GEMM_F16F32_OK) return rc;
    if (n > 0 && parts[0].r.workspace_bytes > GEMM_F16F32_SCRATCH_BYTES)
      return GEMM_F16F32_ERR_SCRATCH;
  }
  void* ws = nullptr;
  rc = scratch_for_stream((hipStream_t)stream, &ws);
  if (rc != GEMM_F16F32_OK) return rc;
  return run(pr, stream, opts, ws, GEMM_F16F32_SCRATCH_BYTES);
}

int gemm_f16f32_strided_plan(int64_t M, int64_t N, int64_t K, const uint16_t* A,
                             int64_t stride_am, int64_t stride_ak, const uint16_t* B,
                             int64_t stride_bk, int64_t stride_bn, const uint16_t* C,
                             int64_t stride_cm, int64_t stride_cn, const gemm_f16f32_opts* opts,
                             gemm_f16f32_plan_info* info) {
  Problem pr;
  const int rc = strided_problem(M, N, K, A, stride_am, stride_ak, B, stride_bk, stride_bn, C,
                                 stride_cm, stride_cn, &pr);
  return rc != GEMM_F16F32_OK ? rc : plan(pr, opts, info);
}

int gemm_f16f32_tile_map(int32_t num_pid_m, int32_t num_pid_n, int32_t group_m,
                         int32_t xcd_remap, int32_t* out_dev, void* stream) {
  if (num_pid_m < 1 || num_pid_n < 1) return GEMM_F16F32_ERR_DIM;
  const int64_t P = (int64_t)num_pid_m * num_pid_n;
  if (P >= ((int64_t)1 << 31)) return GEMM_F16F32_ERR_DIM;
  if (group_m < 1 || xcd_remap < 0 || xcd_remap > 2) return GEMM_F16F32_ERR_OPTS;
  if (out_dev == nullptr) return GEMM_F16F32_ERR_NULL;
  hipLaunchKernelGGL(gk::tile_map_kernel, dim3((uint32_t)P), dim3(64), 0, (hipStream_t)stream,
                     (int)P, num_pid_m, num_pid_n, group_m < num_pid_m ? group_m : num_pid_m,
                     xcd_remap == 1 ? 1 : 0, out_dev);
  return hipGetLastError() == hipSuccess ? GEMM_F16F32_OK : GEMM_F16F32_ERR_HIP;
}

const char* gemm_f16f32_strerror(int code) {
  switch (code) {
    case GEMM_F16F32_OK: return "success";
    case GEMM_F16F32_ERR_DIM: return "M, N or K negative or too large";
    case GEMM_F16F32_ERR_NULL: return "NULL pointer for a non-empty operand";
    case GEMM_F16F32_ERR_LD: return "unsupported strides: leading dimension too small or no unit stride";
    case GEMM_F16F32_ERR_OVERLAP: return "C overlaps A or B";
    case GEMM_F16F32_ERR_OPTS: return "invalid option or misaligned pointer";
    case GEMM_F16F32_ERR_TOO_LARGE: return "leading dimension too large for 32-bit tile offsets";
    case GEMM_F16F32_ERR_HIP: return "HIP runtime rejected the launch";
    case GEMM_F16F32_ERR_WORKSPACE:
      return "split K needs a 16-byte aligned workspace of at least plan_info.workspace_bytes";
    case GEMM_F16F32_ERR_SCRATCH:
      return "split K needs more than the library's 16 MiB static scratch, or the stream is "
             "not on the current device";
    default: return "unknown error code";
  }
}

int gemm_f16f32_version(void) { return kVersion; }

}  // extern "C"
