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
template <int BM_, int BN_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, BK = kBK;
  static constexpr int WTM = BM / 2, WTN = BN / 2;   // per-wave block of C
  static constexpr int TM = WTM / 32, TN = WTN / 32; // 32x32 MFMA blocks per wave
  static constexpr int CA = BK / 8;                  // 16-byte chunks per LDS row of A
  static constexpr int CB = BN / 8;                  // 16-byte chunks per LDS row of B
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int B_BYTES = BK * BN * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_LD = A_BYTES / (kThreads * 16);  // 16-byte loads per thread
  static constexpr int B_LD = B_BYTES / (kThreads * 16);
  static_assert(TM >= 1 && TN >= 1 && CA == 8, "tile shape");
  static_assert(A_LD >= 1 && B_LD >= 1, "tile too small for 256 threads");
};

// LDS layouts.  A panel: BM rows of 64 halves (8 chunks of 16 B); chunk c of row r is stored
// at chunk position c ^ swz_a(r).  Eight (and sixteen) consecutive rows read at the same
// logical chunk then hit distinct bank groups, which is what the MFMA A-operand read does.
__device__ __forceinline__ int swz_a(int r) { return (r ^ (r >> 3)) & 7; }

// B panel: 64 rows (k) of BN halves; chunk c of row k sits at c ^ swz_b(k).  A transposing
// read covers 4 consecutive rows x 2 (16 lanes) or x 4 (32 lanes) consecutive chunks; the
// XOR values 0, 10, 4, 14 for k % 4 = 0..3 spread both footprints over distinct banks.
template <int CB>
__device__ __forceinline__ int swz_b(int k) {
  return ((0xE4A0 >> (4 * (k & 3))) & 0xF) & (CB - 1);
}

template <class T>
__device__ __forceinline__ int lds_a(int r, int c) {
  return r * (T::CA * 16) + ((c ^ swz_a(r)) << 4);
}
template <class T>
__device__ __forceinline__ int lds_b(int k, int n) {
  return k * (T::CB * 16) + ((((n >> 3) ^ swz_b<T::CB>(k))) << 4) + ((n & 7) << 1);
}

// ---------------------------------------------------------------------------------------
// Compute one staged panel: BK/16 steps of TM x TN MFMAs per wave.
// ---------------------------------------------------------------------------------------
template <class T>
__device__ __forceinline__ void mma_panel(const char GK_LDS* sA, const char GK_LDS* sB,
                                          float16v (&acc)[T::TM][T::TN], int wm, int wn,
                                          int lane) {
#pragma unroll
  for (int kk = 0; kk < T::BK / 16; ++kk) {
    half8 a[T::TM];
    half8 b[T::TN];
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm) {
      const int r = wm * T::WTM + tm * 32 + (lane & 31);
      const int c = kk * 2 + (lane >> 5);
      a[tm] = *(const half8 GK_LDS*)(sA + lds_a<T>(r, c));
    }
#pragma unroll
    for (int tn = 0; tn < T::TN; ++tn) {
      const int g = lane >> 4, i = lane & 15;
      const int n = wn * T::WTN + tn * 32 + (g & 1) * 16 + (i & 3) * 4;
      const int k = kk * 16 + (g >> 1) * 8 + (i >> 2);
      short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (short4v GK_LDS*)(sB + lds_b<T>(k, n)));
      short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (short4v GK_LDS*)(sB + lds_b<T>(k + 4, n)));
      b[tn] = __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < T::TN; ++tn)
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[tm], b[tn], acc[tm][tn], 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------------------
// Epilogue: narrow once (fp32 -> fp16, round to nearest even) and store the wave's block.
// ---------------------------------------------------------------------------------------
template <class T>
__device__ __forceinline__ void store_tile(const Args& p, const float16v (&acc)[T::TM][T::TN],
                                           int m0, int n0, int wm, int wn, int lane) {
  const bool full = (m0 + T::BM <= p.M) && (n0 + T::BN <= p.N);
#pragma unroll
  for (int tm = 0; tm < T::TM; ++tm) {
#pragma unroll
    for (int tn = 0; tn < T::TN; ++tn) {
      const int j = n0 + wn * T::WTN + tn * 32 + (lane & 31);
      const int ib = m0 + wm * T::WTM + tm * 32 + (lane >> 5) * 4;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = ib + (v >> 2) * 8 + (v & 3);
        const _Float16 h = (_Float16)acc[tm][tn][v];
        if (full || (i < p.M && j < p.N))
          p.C[(int64_t)i * p.ldc + j] = __builtin_bit_cast(uint16_t, h);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Aligned path: A and B 16-byte aligned, lda % 8 == 0, ldb % 8 == 0, N % 8 == 0, K % 64 == 0.
// Each thread issues A_LD + B_LD direct global->LDS 16-byte loads per panel.  Rows past M
// and column chunks past N are clamped to the last valid ones (their results are never
// stored), so every load stays inside the caller's matrices.
// ---------------------------------------------------------------------------------------
template <int BM, int BN>
__global__ void __launch_bounds__(kThreads) gemm_aligned(Args p) {
  using T = Tile<BM, BN>;
  __shared__ __attribute__((aligned(16))) char smem[2 * T::STAGE];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w >> 1, wn = w & 1;

  int pid, pid_m, pid_n;
  program_tile(blockIdx.x, p.num_programs, p.num_pid_m, p.num_pid_n, p.group_m, p.xcd_remap,
               pid, pid_m, pid_n);
  const int m0 = pid_m * BM, n0 = pid_n * BN;

  // Per-thread element offsets of its load slots, relative to the panel's corner.
  int32_t offA[T::A_LD], offB[T::B_LD];
#pragma unroll
  for (int i = 0; i < T::A_LD; ++i) {
    const int q = (i * 4 + w) * 64 + lane;
    const int r = q / T::CA, c = (q % T::CA) ^ swz_a(r);
    const int row = min(m0 + r, p.M - 1) - m0;
    offA[i] = row * (int32_t)p.lda + c * 8;
  }
#pragma unroll
  for (int i = 0; i < T::B_LD; ++i) {
    const int q = (i * 4 + w) * 64 + lane;
    const int k = q / T::CB, c = (q % T::CB) ^ swz_b<T::CB>(k);
    const int col = min(n0 + c * 8, p.N - 8) - n0;
    offB[i] = k * (int32_t)p.ldb + col;
  }

  const uint16_t* gA = p.A + (int64_t)m0 * p.lda;
  const uint16_t* gB = p.B + n0;
  const int nk = p.K / T::BK;

  auto issue = [&](int s, int stage) {
    const uint16_t* pa = gA + s * T::BK;
    const uint16_t* pb = gB + (int64_t)s * T::BK * p.ldb;
    char GK_LDS* base = (char GK_LDS*)smem + stage * T::STAGE;
#pragma unroll
    for (int i = 0; i < T::A_LD; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(pa + offA[i]),
                                       (void GK_LDS*)(base + (i * 4 + w) * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < T::B_LD; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(pb + offB[i]),
                                       (void GK_LDS*)(base + T::A_BYTES + (i * 4 + w) * 1024),
                                       16, 0, 0);
  };

  float16v acc[T::TM][T::TN];
#pragma unroll
  for (int tm = 0; tm < T::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < T::TN; ++tn)
      acc[tm][tn] = float16v{};

  if (nk > 0) issue(0, 0);
  for (int s = 0; s < nk; ++s) {
    // Own loads of panel s have landed; after the barrier every wave's have, and every wave
    // has finished reading the other stage (panel s-1).
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (s + 1 < nk) issue(s + 1, (s + 1) & 1);
    const char GK_LDS* base = (const char GK_LDS*)smem + (s & 1) * T::STAGE;
    mma_panel<T>(base, base + T::A_BYTES, acc, wm, wn, lane);
  }
  store_tile<T>(p, acc, m0, n0, wm, wn, lane);
}

// ---------------------------------------------------------------------------------------
// Generic path: any leading dimension, any 2-byte alignment, any K.  Panels are fetched with
// raw buffer loads whose resource ends at the matrix's last element, so reads past it return
// zero and never fault; A's elements at k >= K inside a row are zeroed explicitly.  kOdd:
// some row starts are only 2-byte aligned, so each 16-byte chunk is assembled from a
// 4-byte-aligned dwordx4 plus one more dword and a byte funnel shift.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t lim = 0xFFFFFFFFll;
  const int n = (int)(uint32_t)(bytes < 0 ? 0 : (bytes > lim ? lim : bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

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
    const char GK_LDS* base = (const char GK_LDS*)smem + (s & 1) * T::STAGE;
    mma_panel<T>(base, base + T::A_BYTES, acc, wm, wn, lane);
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
