// Device code for the fp16-operand / fp32-accumulate / fp16-result GEMM on gfx950.
//
// What is computed: C = A B with fp16 operands, an fp32 accumulator that stays in registers
// for the whole k loop, and one narrowing to fp16 (round to nearest even) on the store --
// phobos "03: Matrix multiplication", the `matmul` kernel and the paragraph after it.  One
// workgroup owns one BM x BN tile of C and walks K in BK = 64 deep panels; each panel of A and
// of B is staged in LDS and multiplied on the matrix cores; the LDS panels are double
// buffered so that panel s+1 streams in while panel s is multiplied.
//
// Which tile a workgroup owns follows the grouped order of the kernl notebook "Computing
// coordinates on Triton GEMM example" (introduction excerpt, cells In[4]-In[7]), applied to a
// program id that is first permuted so that the workgroups one XCD receives (the hardware
// deals them round-robin over the 8 XCDs) get consecutive program ids.
//
// gfx950 specifics used here (each checked on the hardware with one-hot / index probes):
//  * v_mfma_f32_32x32x16_f16: lane l supplies A[l%32][8(l/32) .. 8(l/32)+7] and
//    B[8(l/32) .. +7][l%32]; result element v of lane l is C[8(v/4) + 4(l/32) + v%4][l%32].
//  * ds_read_b64_tr_b16: inside each group of 16 lanes, lane i receives, as its 4 halves, the
//    i-th 16-bit column of the 4 x 16 block whose row e is the 4 x 64 bits addressed by lanes
//    4e .. 4e+3 of the group.  Row-major B panels therefore yield MFMA B operands (k-runs at a
//    fixed column) without any transpose in memory.
//  * global_load_lds_dwordx4: lane l's 16 bytes land at the (wave-uniform) LDS address plus
//    16 l; the instruction's immediate offset would move both addresses, so it stays 0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace gk {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define GK_LDS __attribute__((address_space(3)))

constexpr int kXcds = 8;       // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int kThreads = 256;  // 4 wavefronts of 64 lanes in a 2 x 2 arrangement
constexpr int kBK = 64;        // k depth of one staged panel

struct Args {
  const uint16_t* A;
  const uint16_t* B;
  uint16_t* C;
  int64_t lda, ldb, ldc;
  int32_t M, N, K;
  int32_t num_pid_m, num_pid_n, group_m, xcd_remap, num_programs;
};

// ---------------------------------------------------------------------------------------
// Program map.  h: hardware workgroup id.  Optional XCD permutation, then the grouped map:
// groups of G tile-rows, column-major inside a group, a smaller last group, and the row
// offset inside the group taken as pid % group_size (as the notebook prints it).
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ void program_tile(int h, int P, int num_pid_m, int num_pid_n, int G,
                                             int remap, int& pid, int& pid_m, int& pid_n) {
  if (remap) {
    const int q = P / kXcds, r = P % kXcds, x = h % kXcds;
    pid = x * q + (x < r ? x : r) + h / kXcds;
  } else {
    pid = h;
  }
  const int in_group = G * num_pid_n;
  const int group = pid / in_group;
  const int first_m = group * G;
  const int rows_left = num_pid_m - first_m;
  const int size_m = rows_left < G ? rows_left : G;
  pid_m = first_m + pid % size_m;
  pid_n = (pid % in_group) / size_m;
}

// ---------------------------------------------------------------------------------------
// Tile geometry.
// ---------------------------------------------------------------------------------------
template <int BM_, int BN_, int BK_ = kBK>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int WTM = BM / 2, WTN = BN / 2;   // per-wave block of C
  static constexpr int TM = WTM / 32, TN = WTN / 32; // 32x32 MFMA blocks per wave
  static constexpr int CA = BK / 8;                  // 16-byte chunks per LDS row of A
  static constexpr int CB = BN / 8;                  // 16-byte chunks per LDS row of B
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int B_BYTES = BK * BN * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_LD = A_BYTES / (kThreads * 16);  // 16-byte loads per thread
  static constexpr int B_LD = B_BYTES / (kThreads * 16);
  static_assert(TM >= 1 && TN >= 1 && (CA == 8 || CA == 4), "tile shape");
  static_assert(A_LD >= 1 && B_LD >= 1, "tile too small for 256 threads");
};

// The hardware range-checks each dword of a buffer load on its own and returns 0 for a dword
// that reaches past num_records, even partly.  The extent is therefore rounded up to whole
// dwords: a matrix whose last element ends 2 bytes into a dword still gets that element.  The
// 2 extra bytes share a dword (hence a page) with valid data, and they only ever land in
// slots that are masked (k >= K) or never stored (columns >= N).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  // Saturate to [0, 2^32 - 4] with 32-bit scalar operations only (no 64-bit compares, which
  // the scalar unit lacks and would move to the vector unit).
  const uint64_t b = (uint64_t)(bytes + 3) & ~(uint64_t)3;
  const uint32_t hi = (uint32_t)(b >> 32), lo = (uint32_t)b;
  const uint32_t n = (hi & 0x80000000u) ? 0u : (hi ? 0xFFFFFFFCu : lo);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

// 16-byte buffer -> LDS load: lane l's 16 bytes from (resource, voff) land at dst + 16 l.
// The builtin exists only for the device; in the host pass of this single-source file the
// call must not appear at all, or the kernels' host launch stubs are not emitted.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, void GK_LDS* dst,
                                                  uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, 0);
#endif
}

// LDS layouts.  A panel: BM rows of BK halves (CA = BK/8 chunks of 16 B); chunk c of row r is
// stored at chunk position c ^ swz_a(r).  An MFMA A-operand read has 32 lanes on 32
// consecutive rows at one logical chunk; the hardware serves such a read 8 lanes (128 B) or
// 16 lanes (256 B) at a time, so any 8 (and any 16) consecutive rows must land on distinct
// bank groups:
//  * 128-byte rows (BK = 64): swz = (r mod 8) xor bit 3 of r -- 8 rows give 8 distinct chunk
//    positions, 16 rows 16 distinct (row parity, position) pairs;
//  * 64-byte rows (BK = 32): two rows share a bank line; swz = (bits 1-2 of r) xor (bits 3-4)
//    gives distinct (r mod 2, position) over 8 rows and distinct (r mod 4, position) over 16.
// Both depend on r mod 32 only, so rows 32 apart (the next 32-row MFMA block) share the
// swizzle and their addresses differ by a constant.
template <int CA>
__device__ __forceinline__ int swz_a(int r) {
  if constexpr (CA == 8)
    return (r & 7) ^ ((r >> 3) & 1);
  else
    return ((r >> 1) ^ (r >> 3)) & 3;
}

// B panel: BK rows (k) of BN halves; chunk c of row k sits at c ^ swz_b(k).  A transposing
// read covers 4 consecutive rows x 2 (16 lanes) or x 4 (32 lanes) consecutive chunks; the
// XOR values 0, 10, 4, 14 for k % 4 = 0..3 spread both footprints over distinct banks.
template <int CB>
__device__ __forceinline__ int swz_b(int k) {
  return ((0xE4A0 >> (4 * (k & 3))) & 0xF) & (CB - 1);
}

template <class T>
__device__ __forceinline__ int lds_a(int r, int c) {
  return r * (T::CA * 16) + ((c ^ swz_a<T::CA>(r)) << 4);
}
template <class T>
__device__ __forceinline__ int lds_b(int k, int n) {
  return k * (T::CB * 16) + ((((n >> 3) ^ swz_b<T::CB>(k))) << 4) + ((n & 7) << 1);
}

// ---------------------------------------------------------------------------------------
// MFMA operands of one 16-deep k step for one wave: TM A blocks (32 rows x 16 k) and TN B
// blocks (16 k x 32 columns), read from a staged panel.
// ---------------------------------------------------------------------------------------
template <class T>
struct Frag {
  half8 a[T::TM];
  half8 b[T::TN];
};

// Per-lane LDS byte offsets of a wave's operand reads inside one stage.  A: one per k step
// (block tm adds 32 rows, which keep the swizzle, so that is an immediate).  B: one per 32-column block (k step kk and the second
// 4-deep read add whole rows, which keep row % 4 and hence the swizzle; also immediates).
template <class T>
struct LaneOffsets {
  int a[T::BK / 16];
  int b[T::TN];
};

template <class T>
__device__ __forceinline__ LaneOffsets<T> lane_offsets(int wm, int wn, int lane) {
  LaneOffsets<T> o;
#pragma unroll
  for (int kk = 0; kk < T::BK / 16; ++kk)
    o.a[kk] = lds_a<T>(wm * T::WTM + (lane & 31), kk * 2 + (lane >> 5));
  const int g = lane >> 4, i = lane & 15;
#pragma unroll
  for (int tn = 0; tn < T::TN; ++tn)
    o.b[tn] = T::A_BYTES +
              lds_b<T>((g >> 1) * 8 + (i >> 2), wn * T::WTN + tn * 32 + (g & 1) * 16 + (i & 3) * 4);
  return o;
}

// Reads the operands of k step kk from the stage at `st`.
template <class T>
__device__ __forceinline__ void read_frags(Frag<T>& f, const char GK_LDS* st,
                                           const LaneOffsets<T>& o, int kk) {
#pragma unroll
  for (int tm = 0; tm < T::TM; ++tm)
    f.a[tm] = *(const half8 GK_LDS*)(st + o.a[kk] + tm * 32 * (T::CA * 16));
#pragma unroll
  for (int tn = 0; tn < T::TN; ++tn) {
    const char GK_LDS* pb = st + o.b[tn] + kk * 16 * (T::CB * 16);
    short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((short4v GK_LDS*)pb);
    short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((short4v GK_LDS*)(pb + 4 * T::CB * 16));
    f.b[tn] = __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
}

template <class T>
__device__ __forceinline__ void mfma_step(float16v (&acc)[T::TM][T::TN], const Frag<T>& f) {
#pragma unroll
  for (int tm = 0; tm < T::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < T::TN; ++tn)
      acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a[tm], f.b[tn], acc[tm][tn], 0, 0, 0);
}

// One whole staged panel, operands read just before use (generic path).
template <class T>
__device__ __forceinline__ void mma_panel(const char GK_LDS* st, float16v (&acc)[T::TM][T::TN],
                                          const LaneOffsets<T>& o) {
#pragma unroll
  for (int kk = 0; kk < T::BK / 16; ++kk) {
    Frag<T> f;
    read_frags<T>(f, st, o, kk);
    mfma_step<T>(acc, f);
  }
}

// ---------------------------------------------------------------------------------------
// Epilogue: narrow once (fp32 -> fp16, round to nearest even) and store the wave's block.
// Stores go through a buffer resource that ends at C's last element, so rows past M are
// dropped by the hardware; columns past N (which would land in the ldc padding) are masked.
// Per lane, one VGPR holds the byte offset of its first element; row steps are scalar
// offsets and 32-column steps immediates.
// ---------------------------------------------------------------------------------------
template <class T>
__device__ __forceinline__ void store_tile(const Args& p, const float16v (&acc)[T::TM][T::TN],
                                           int m0, int n0, int wm, int wn, int lane) {
  const int64_t c0 = (int64_t)m0 * p.ldc + n0;
  const int64_t extC = (int64_t)(p.M - 1) * p.ldc + p.N;
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.C + c0, 2 * (extC - c0));
  const int col = wn * T::WTN + (lane & 31);
  const uint32_t vbase =
      2u * ((uint32_t)(wm * T::WTM + (lane >> 5) * 4) * (uint32_t)p.ldc + (uint32_t)col);
  const uint32_t ldc2 = 2u * (uint32_t)p.ldc;
  const int ncols = p.N - n0;   // columns of this tile that exist
#pragma unroll
  for (int tn = 0; tn < T::TN; ++tn) {
    if (col + tn * 32 < ncols) {
#pragma unroll
      for (int tm = 0; tm < T::TM; ++tm) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const uint32_t rowstep = (uint32_t)(tm * 32 + (v >> 2) * 8 + (v & 3)) * ldc2;
          const _Float16 h = (_Float16)acc[tm][tn][v];
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, h), rc,
                                                vbase + tn * 64, rowstep, 0);
        }
      }
    }
  }
}

// Wait for this wave's LDS accesses, then meet the other waves.  Written as one asm block so
// that no LDS access is moved across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---------------------------------------------------------------------------------------
// Instruction interleaving inside one k step (one scheduling region): NM MFMAs, with ND LDS
// reads and NV global loads spread evenly between them.
// ---------------------------------------------------------------------------------------
template <int MASK, int COUNT>
__device__ __forceinline__ void sched_group() {
  if constexpr (COUNT > 0) __builtin_amdgcn_sched_group_barrier(MASK, COUNT, 0);
}

template <int NM, int ND, int NV, int... I>
__device__ __forceinline__ void sched_step(std::integer_sequence<int, I...>) {
  ((sched_group<0x008, 1>(), sched_group<0x100, (I + 1) * ND / NM - I * ND / NM>(),
    sched_group<0x020, (I + 1) * NV / NM - I * NV / NM>()),
   ...);
}

template <int NM, int ND, int NV>
__device__ __forceinline__ void sched_step() {
  sched_step<NM, ND, NV>(std::make_integer_sequence<int, NM>{});
  __builtin_amdgcn_sched_barrier(0);
}

// s_waitcnt vmcnt(N) for a compile-time N: wait until at most N vector-memory loads of this
// wave are outstanding (loads complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ---------------------------------------------------------------------------------------
// DMA path (any shape, any 2-byte alignment, any leading dimension).
//
// Panels are BK deep.  When BK does not divide K, panel 0 is a "head" that holds the first
// K mod BK values of k at its end and zeros in front: the run is then the same, bit for bit,
// as a run on operands zero-padded in front of k to a multiple of BK, and every later panel
// is a full one.  Full panels are loaded with 16-byte buffer->LDS DMA (A: rows of 16-byte
// chunks, B: 16-byte chunks of rows); the buffer resources end at the matrices' last
// elements, so rows past M read as zeros and nothing past the matrices is read.  Columns
// past N read whatever lies there and only feed results that are never stored.  The head is
// loaded through registers, A element by element (so nothing before A's first element is
// ever addressed), and written to LDS in the same layout.
//
// Pipeline (per wave), NS LDS stages, panel s in stage s mod NS: the operands of k step kk+1
// are read from LDS while the MFMAs of step kk run.  The one barrier per panel sits in the
// last k step, after that step's operands are in registers; past it the first operands of
// panel s+1 are read.  Stage refills: see `panel` below.  The stages are separate LDS objects
// and the loop is unrolled by NS, so the compiler can see that a refill never aliases the
// stage being read and does not wait for it.  Panels past the end get empty buffer
// resources: they load zeros, touch no memory and add exactly +0, which keeps the loop free
// of branches.
// ---------------------------------------------------------------------------------------
template <int BM, int BN, int BK, int NS>
__global__ void __launch_bounds__(kThreads) gemm_dma(Args p) {
  using T = Tile<BM, BN, BK>;
  constexpr int KS = BK / 16;              // k steps per panel
  constexpr int NM = T::TM * T::TN;        // MFMAs per k step
  constexpr int ND = T::TM + 2 * T::TN;    // LDS reads per k step
  constexpr int NV = T::A_LD + T::B_LD;    // buffer->LDS loads per panel
  static_assert(KS % 2 == 0 && NS >= 2 && NS <= 5, "pipeline shape");
  static_assert(NS * T::STAGE <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) char stage0[T::STAGE];
  __shared__ __attribute__((aligned(16))) char stage1[T::STAGE];
  __shared__ __attribute__((aligned(16))) char stage2[NS > 2 ? T::STAGE : 16];
  __shared__ __attribute__((aligned(16))) char stage3[NS > 3 ? T::STAGE : 16];
  __shared__ __attribute__((aligned(16))) char stage4[NS > 4 ? T::STAGE : 16];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w >> 1, wn = w & 1;

  int pid, pid_m, pid_n;
  program_tile(blockIdx.x, p.num_programs, p.num_pid_m, p.num_pid_n, p.group_m, p.xcd_remap,
               pid, pid_m, pid_n);
  const int m0 = pid_m * BM, n0 = pid_n * BN;

  // This thread's load slots: slot q = (i*4 + w)*64 + lane of a stage holds logical chunk
  // (row, chunk) of A (or B) as given by the swizzles.  Byte offsets relative to the panel's
  // corner.
  uint32_t offA[T::A_LD], offB[T::B_LD];
#pragma unroll
  for (int i = 0; i < T::A_LD; ++i) {
    const int q = (i * 4 + w) * 64 + lane;
    const int r = q / T::CA, c = (q % T::CA) ^ swz_a<T::CA>(r);
    offA[i] = 2u * ((uint32_t)r * (uint32_t)p.lda + (uint32_t)(c * 8));
  }
#pragma unroll
  for (int i = 0; i < T::B_LD; ++i) {
    const int q = (i * 4 + w) * 64 + lane;
    const int k = q / T::CB, c = (q % T::CB) ^ swz_b<T::CB>(k);
    offB[i] = 2u * ((uint32_t)k * (uint32_t)p.ldb + (uint32_t)(c * 8));
  }

  // Extents (elements from each matrix's first element to one past its last).
  const int64_t extA = (int64_t)(p.M - 1) * p.lda + p.K;
  const int64_t extB = (int64_t)(p.K - 1) * p.ldb + p.N;
  const int rk = p.K % BK;                       // depth of the head panel (0: none)
  const int np = p.K / BK + (rk ? 1 : 0);        // panels
  const int kofs = rk ? rk - BK : 0;             // panel s covers k in [kofs + s BK, + BK)

  // The last panel's copies of A's last element A[M-1][K-1] and B's last element
  // B[K-1][N-1].  A 16-byte load that starts 2 bytes into a dword is range-checked dword by
  // dword from its own start, so when a matrix ends on a 4-byte boundary the dword holding its
  // last element reaches 2 bytes past the end and reads as zero.  The thread whose load slot
  // holds that element (local k = BK-1 of the last panel, for tiles that contain row M-1 or
  // column N-1) rewrites it from an exact 2-byte load once the panel has landed.
  int patch_a = -1, patch_b = -1;    // LDS byte offsets within a stage, or -1
  uint16_t last_a = 0, last_b = 0;
  {
    const int t = threadIdx.x;
    const int rl = p.M - 1 - m0;
    if (p.K > 0 && rl < BM) {
      const int q = rl * T::CA + ((T::CA - 1) ^ swz_a<T::CA>(rl));
      if ((q & (kThreads - 1)) == t) {
        patch_a = q * 16 + 7 * 2;
        last_a = __builtin_amdgcn_raw_buffer_load_b16(
            make_rsrc(p.A, 2 * extA), 2u * (uint32_t)((int64_t)(p.M - 1) * p.lda + p.K - 1), 0, 0);
      }
    }
    const int cl = p.N - 1 - n0;
    if (p.K > 0 && cl < BN) {
      const int q = (BK - 1) * T::CB + ((cl >> 3) ^ swz_b<T::CB>(BK - 1));
      if ((q & (kThreads - 1)) == t) {
        patch_b = T::A_BYTES + q * 16 + (cl & 7) * 2;
        last_b = __builtin_amdgcn_raw_buffer_load_b16(
            make_rsrc(p.B, 2 * extB), 2u * (uint32_t)((int64_t)(p.K - 1) * p.ldb + p.N - 1), 0, 0);
      }
    }
  }
  auto patch = [&](char GK_LDS* base) __attribute__((always_inline)) {
    if (patch_a >= 0) *(uint16_t GK_LDS*)(base + patch_a) = last_a;
    if (patch_b >= 0) *(uint16_t GK_LDS*)(base + patch_b) = last_b;
  };

  // Full panel s (k0 = kofs + s BK >= 0): DMA into `base`.  Panels past the end get an empty
  // resource: their loads touch no memory and deposit zeros.
  auto issue = [&](int s, char GK_LDS* base) __attribute__((always_inline)) {
    const bool live = s < np;
    const int64_t k0 = (int64_t)kofs + (int64_t)s * BK;
    const int64_t a0 = (int64_t)m0 * p.lda + k0;
    const int64_t b0 = k0 * p.ldb + n0;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A + (live ? a0 : 0), live ? 2 * (extA - a0) : 0);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B + (live ? b0 : 0), live ? 2 * (extB - b0) : 0);
#pragma unroll
    for (int i = 0; i < T::A_LD; ++i)
      buffer_load_lds16(ra, (void GK_LDS*)(base + (i * 4 + w) * 1024), offA[i]);
#pragma unroll
    for (int i = 0; i < T::B_LD; ++i)
      buffer_load_lds16(rb, (void GK_LDS*)(base + T::A_BYTES + (i * 4 + w) * 1024), offB[i]);
  };

  // Head panel (k0 = kofs < 0): the same slots, through registers; k < 0 is zero.
  auto head = [&](char GK_LDS* base) __attribute__((always_inline)) {
    const int64_t a0 = (int64_t)m0 * p.lda;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A + a0, 2 * (extA - a0));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B + n0, 2 * (extB - n0));
    u32x4 va[T::A_LD], vb[T::B_LD];
#pragma unroll
    for (int i = 0; i < T::A_LD; ++i) {
      const int q = (i * 4 + w) * 64 + lane;
      const int r = q / T::CA, c = (q % T::CA) ^ swz_a<T::CA>(r);
      uint16_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = kofs + c * 8 + e;
        h[e] = k >= 0 ? __builtin_amdgcn_raw_buffer_load_b16(
                            ra, 2u * ((uint32_t)r * (uint32_t)p.lda + (uint32_t)k), 0, 0)
                      : (uint16_t)0;
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) va[i][d] = (uint32_t)h[2 * d] | ((uint32_t)h[2 * d + 1] << 16);
    }
#pragma unroll
    for (int i = 0; i < T::B_LD; ++i) {
      const int q = (i * 4 + w) * 64 + lane;
      const int k = q / T::CB, c = (q % T::CB) ^ swz_b<T::CB>(k);
      const int kr = kofs + k;
      vb[i] = kr >= 0 ? __builtin_amdgcn_raw_buffer_load_b128(
                            rb, 2u * ((uint32_t)kr * (uint32_t)p.ldb + (uint32_t)(c * 8)), 0, 0)
                      : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < T::A_LD; ++i)
      *(u32x4 GK_LDS*)(base + ((i * 4 + w) * 64 + lane) * 16) = va[i];
#pragma unroll
    for (int i = 0; i < T::B_LD; ++i)
      *(u32x4 GK_LDS*)(base + T::A_BYTES + ((i * 4 + w) * 64 + lane) * 16) = vb[i];
  };

  float16v acc[T::TM][T::TN];
#pragma unroll
  for (int tm = 0; tm < T::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < T::TN; ++tn)
      acc[tm][tn] = float16v{};

  char GK_LDS* const S[5] = {(char GK_LDS*)stage0, (char GK_LDS*)stage1, (char GK_LDS*)stage2,
                             (char GK_LDS*)stage3, (char GK_LDS*)stage4};
  const LaneOffsets<T> lo = lane_offsets<T>(wm, wn, lane);
  Frag<T> f[2];

  // One panel from stage `cur`, with panel s+1 in `nxt`; `prev` held panel s-1.
  //  * NS == 2: past the barrier in the last k step, `cur` (just consumed) is refilled with
  //    panel s+2.
  //  * NS >= 3: `prev` is refilled with panel s+NS-1 at the start of the panel, its loads
  //    spread over the first k step's MFMAs.  Every wave finished reading `prev` before the
  //    previous panel's barrier (which waits for the wave's own LDS reads), so no further
  //    synchronisation is needed, and this panel's barrier only has to see panel s+1 land.
  auto panel = [&](int s, char GK_LDS* cur, char GK_LDS* nxt, char GK_LDS* prev)
                   __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk + 1 < KS; ++kk) {
      if constexpr (NS >= 3) {
        if (kk == 0) issue(s + NS - 1, prev);
      }
      read_frags<T>(f[(kk + 1) & 1], cur, lo, kk + 1);
      mfma_step<T>(acc, f[kk & 1]);
      if constexpr (NS >= 3) {
        if (kk == 0)
          sched_step<NM, ND, NV>();
        else
          sched_step<NM, ND, 0>();
      } else {
        sched_step<NM, ND, 0>();
      }
    }
    wait_vmcnt<(NS - 2) * NV>();   // panel s+1 has landed (this wave's part)
    if (s + 2 == np) patch(nxt);   // panel s+1 is the last one
    lds_barrier();                 // ... every wave's part
    if constexpr (NS == 2) issue(s + NS, cur);
    read_frags<T>(f[0], nxt, lo, 0);
    mfma_step<T>(acc, f[1]);
    sched_step<NM, ND, NS == 2 ? NV : 0>();
  };

  if (np > 0) {
    // NS == 2 starts with both stages filled; NS >= 3 with all but the last (the first
    // panel refills it).
    constexpr int kPre = NS == 2 ? 2 : NS - 1;
    if (rk)
      head(S[0]);
    else
      issue(0, S[0]);
#pragma unroll
    for (int j = 1; j < kPre; ++j) issue(j, S[j]);
    wait_vmcnt<(kPre - 1) * NV>();
    if (np == 1) patch(S[0]);
    lds_barrier();
    read_frags<T>(f[0], S[0], lo, 0);
  }
  for (int s = 0; s < np; s += NS) {
#pragma unroll
    for (int j = 0; j < NS; ++j) panel(s + j, S[j], S[(j + 1) % NS], S[(j + NS - 1) % NS]);
  }
  // The last refills (of panels past the end) must land before the workgroup's LDS is freed.
  wait_vmcnt<0>();
  store_tile<T>(p, acc, m0, n0, wm, wn, lane);
}

// ---------------------------------------------------------------------------------------
// Generic path: any leading dimension, any 2-byte alignment, any K.  Panels are fetched with
// raw buffer loads whose resource ends at the matrix's last element, so reads past it return
// zero and never fault; A's elements at k >= K inside a row are zeroed explicitly.  kOdd:
// some row starts are only 2-byte aligned, so each 16-byte chunk is assembled from a
// 4-byte-aligned dwordx4 plus one more dword and a byte funnel shift.
// ---------------------------------------------------------------------------------------
template <bool kOdd>
__device__ __forceinline__ u32x4 load_chunk(__amdgpu_buffer_rsrc_t rs, uint32_t off_bytes) {
  if (!kOdd) {
    return __builtin_amdgcn_raw_buffer_load_b128(rs, off_bytes, 0, 0);
  } else {
    const uint32_t o = off_bytes & ~3u;
    const uint32_t sh = off_bytes & 3u;  // 0 or 2
    u32x4 d = __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, 0);
    uint32_t e = __builtin_amdgcn_raw_buffer_load_b32(rs, o + 16, 0, 0);
    u32x4 r;
    r[0] = __builtin_amdgcn_alignbyte(d[1], d[0], sh);
    r[1] = __builtin_amdgcn_alignbyte(d[2], d[1], sh);
    r[2] = __builtin_amdgcn_alignbyte(d[3], d[2], sh);
    r[3] = __builtin_amdgcn_alignbyte(e, d[3], sh);
    return r;
  }
}

// Zero the halves of a chunk whose k index (first + e) is >= K.
__device__ __forceinline__ u32x4 mask_k(u32x4 v, int first, int K) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int k0 = first + 2 * d;
    uint32_t m = (k0 < K ? 0x0000FFFFu : 0u) | (k0 + 1 < K ? 0xFFFF0000u : 0u);
    v[d] &= m;
  }
  return v;
}

template <int BM, int BN, bool kOdd>
__global__ void __launch_bounds__(kThreads) gemm_generic(Args p) {
  using T = Tile<BM, BN>;
  __shared__ __attribute__((aligned(16))) char smem[2 * T::STAGE];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w >> 1, wn = w & 1;

  int pid, pid_m, pid_n;
  program_tile(blockIdx.x, p.num_programs, p.num_pid_m, p.num_pid_n, p.group_m, p.xcd_remap,
               pid, pid_m, pid_n);
  const int m0 = pid_m * BM, n0 = pid_n * BN;
  const int nk = (p.K + T::BK - 1) / T::BK;

  // Extents in elements, from each matrix's first element to one past its last.
  const int64_t extA = (int64_t)(p.M - 1) * p.lda + p.K;
  const int64_t extB = (int64_t)(p.K - 1) * p.ldb + p.N;

  u32x4 ra[T::A_LD], rb[T::B_LD];

  auto fetch = [&](int s) {
    const int k0 = s * T::BK;
    const int64_t baseA = (int64_t)m0 * p.lda + k0;
    const int64_t baseB = (int64_t)k0 * p.ldb + n0;
    __amdgpu_buffer_rsrc_t rsA = make_rsrc(p.A + baseA, 2 * (extA - baseA));
    __amdgpu_buffer_rsrc_t rsB = make_rsrc(p.B + baseB, 2 * (extB - baseB));
    const bool tail = k0 + T::BK > p.K;
#pragma unroll
    for (int i = 0; i < T::A_LD; ++i) {
      const int q = i * kThreads + t;
      const int r = q / T::CA, c = q % T::CA;
      const uint32_t off = 2u * ((uint32_t)r * (uint32_t)p.lda + (uint32_t)(c * 8));
      ra[i] = load_chunk<kOdd>(rsA, off);
      if (tail) ra[i] = mask_k(ra[i], k0 + c * 8, p.K);
    }
#pragma unroll
    for (int i = 0; i < T::B_LD; ++i) {
      const int q = i * kThreads + t;
      const int k = q / T::CB, c = q % T::CB;
      const uint32_t off = 2u * ((uint32_t)k * (uint32_t)p.ldb + (uint32_t)(c * 8));
      rb[i] = load_chunk<kOdd>(rsB, off);
    }
  };
  auto deposit = [&](int stage) {
    char GK_LDS* base = (char GK_LDS*)smem + stage * T::STAGE;
#pragma unroll
    for (int i = 0; i < T::A_LD; ++i) {
      const int q = i * kThreads + t;
      const int r = q / T::CA, c = q % T::CA;
      *(u32x4 GK_LDS*)(base + lds_a<T>(r, c)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < T::B_LD; ++i) {
      const int q = i * kThreads + t;
      const int k = q / T::CB, c = q % T::CB;
      *(u32x4 GK_LDS*)(base + T::A_BYTES + lds_b<T>(k, c * 8)) = rb[i];
    }
  };

  const LaneOffsets<T> lo = lane_offsets<T>(wm, wn, lane);
  float16v acc[T::TM][T::TN];
#pragma unroll
  for (int tm = 0; tm < T::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < T::TN; ++tn)
      acc[tm][tn] = float16v{};

  if (nk > 0) {
    fetch(0);
    deposit(0);
  }
  for (int s = 0; s < nk; ++s) {
    __syncthreads();
    if (s + 1 < nk) fetch(s + 1);
    mma_panel<T>((const char GK_LDS*)smem + (s & 1) * T::STAGE, acc, lo);
    if (s + 1 < nk) deposit((s + 1) & 1);
  }
  store_tile<T>(p, acc, m0, n0, wm, wn, lane);
}

// ---------------------------------------------------------------------------------------
// Tile-map export: workgroup h writes (logical pid, pid_m, pid_n) from program_tile().
// ---------------------------------------------------------------------------------------
__global__ void __launch_bounds__(64) tile_map_kernel(int P, int num_pid_m, int num_pid_n, int G,
                                                      int remap, int32_t* out) {
  if (threadIdx.x != 0 || (int)blockIdx.x >= P) return;
  int pid, pm, pn;
  program_tile(blockIdx.x, P, num_pid_m, num_pid_n, G, remap, pid, pm, pn);
  out[3 * (int64_t)blockIdx.x + 0] = pid;
  out[3 * (int64_t)blockIdx.x + 1] = pm;
  out[3 * (int64_t)blockIdx.x + 2] = pn;
}

}  // namespace gk
