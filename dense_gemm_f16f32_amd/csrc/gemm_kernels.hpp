// Device code for the fp16-operand / fp32-accumulate / fp16-result GEMM on gfx950.
//
// What is computed: C = A B with fp16 operands, an fp32 accumulator that stays in registers
// for the whole k loop, and one narrowing to fp16 (round to nearest even) on the store --
// phobos "03: Matrix multiplication", the `matmul` kernel and the paragraph after it.  A
// workgroup of WM x WN wavefronts computes one BM x BN tile of C (or, in the persistent
// schedule, a sequence of them) and walks K in BK-deep panels; each panel of A and of B is
// staged in LDS in the operand's own storage order (k-contiguous or not) and multiplied on
// the matrix cores; NS LDS stages keep the next panels streaming in while one is multiplied.
//
// Split K (opt-in, with a caller workspace): the k range is cut into slices whose partial
// tile sums are stored in fp32 and added in slice order by a second kernel before the one
// narrowing -- still one fp32 sum per element, rounded once, in another order of additions.
//
// Which tile a workgroup owns follows the grouped order of the kernl notebook "Computing
// coordinates on Triton GEMM example" (introduction excerpt, cells In[4]-In[7]), applied to a
// program id that is first permuted so that the workgroups one XCD receives (the hardware
// deals them round-robin over the 8 XCDs) get consecutive program ids.
//
// gfx950 specifics used here (each checked on the hardware with one-hot / index probes):
//  * v_mfma_f32_32x32x16_f16: lane l supplies A[l%32][8(l/32) .. 8(l/32)+7] and
//    B[8(l/32) .. +7][l%32]; result element v of lane l is C[8(v/4) + 4(l/32) + v%4][l%32].
//  * v_mfma_f32_16x16x32_f16: lane l supplies A[l%16][8(l/16) .. +7] and B[8(l/16) .. +7][l%16];
//    result element v of lane l is C[4(l/16) + v][l%16].  A 32-deep step of it gives the same
//    fp32 result, bit for bit, as two 16-deep steps of the 32 x 32 instruction (checked on
//    whole 8192^3 outputs), so every tile still yields the same bits.
//  * ds_read_b64_tr_b16: inside each group of 16 lanes, lane i receives, as its 4 halves, the
//    i-th 16-bit column of the 4 x 16 block whose row e is the 4 x 64 bits addressed by lanes
//    4e .. 4e+3 of the group.  Panels stored with k as the row index therefore yield MFMA
//    operands (k-runs at a fixed row of A / column of B) without any transpose in memory.
//  * buffer_load_dwordx4 ... lds: lane l's 16 bytes land at the (wave-uniform) LDS address
//    plus 16 l; the instruction's immediate offset would move both addresses, so it stays 0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace gk {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define GK_LDS __attribute__((address_space(3)))

constexpr int kXcds = 8;       // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int kBK = 64;        // k depth of one staged panel (generic path; the widest)
constexpr int kMaxStages = 16; // LDS stages of the DMA path, at most

struct Args {
  const uint16_t* A;
  const uint16_t* B;
  uint16_t* C;
  int64_t lda, ldb, ldc;
  int32_t M, N, K;
  int32_t num_pid_m, num_pid_n, group_m, xcd_remap, num_programs;
  // Split K only (gemm_dma_splitk): slice z of every tile sums its k panels into the fp32
  // workspace W[z][i][j] at W + (z M + i) ldw + j instead of narrowing into C.
  float* W;
  int64_t ldw;
  int32_t splits, panels_per_split;
  // Ping-pong tile only (gemm_pp with a strip): the strip_n (1..16) columns of C right of the
  // N launched ones, computed by the launch's own workgroups (see pp_tile).
  int32_t strip_n;
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
// Operands.  Both MFMA operands have the same register shape: lane l holds the 8 k values
// 8(l/32) .. 8(l/32)+7 at position l % 32 along the operand's other axis X (the row of A, the
// column of B) -- with 16x16x32 MFMAs (XB = 16) the 8 k values 8(l/16) .. +7 of a 32-deep step
// at position l % 16.  They differ only in how the matrix is stored:
//  * k-major (KM): consecutive k are adjacent in memory -- A row-major (M x K), or B stored
//    transposed (N x K).  Element (x, k) is at x * ld + k.
//  * x-major: consecutive x are adjacent -- B row-major (K x N), or A stored transposed
//    (K x M).  Element (x, k) is at k * ld + x.
// An LDS panel keeps the operand's memory layout, in rows of 16-byte chunks:
//  * k-major: BX rows of BK halves; one MFMA operand is one 16-byte read per lane;
//  * x-major: BK rows of BX halves; one MFMA operand is two transposing reads per lane
//    (ds_read_b64_tr_b16, 4 k rows each).
// Chunk c of LDS row r sits at chunk position c ^ swz(r).
// ---------------------------------------------------------------------------------------
template <int BX_, int BK_, bool KM_, int W_, int NW_, int XB_ = 32>
struct Opnd {
  static constexpr int XB = XB_, KD = XB_ == 32 ? 16 : 32;  // MFMA block width, k depth
  static constexpr int BX = BX_, BK = BK_;
  static constexpr bool KM = KM_;
  static constexpr int W = W_;                       // waves along X
  static constexpr int NW = NW_;                     // waves in the workgroup
  static constexpr int ROWS = KM ? BX : BK;          // LDS rows of one panel
  static constexpr int CH = (KM ? BK : BX) / 8;      // 16-byte chunks per LDS row
  static constexpr int ROW_BYTES = CH * 16;
  static constexpr int BYTES = BX * BK * 2;
  static constexpr int LD = BYTES / (NW * 64 * 16); // 16-byte loads per thread per panel
  static constexpr int WX = BX / W;                  // extent of one wave's block along X
  static constexpr int T = WX / XB;                  // MFMA blocks per wave
  static constexpr int NOFF = KM ? BK / KD : T;      // per-lane LDS read offsets
  static constexpr int READS = KM ? T : 2 * T;       // LDS read instructions per k step
  static_assert(T >= 1 && LD >= 1 && WX % XB == 0, "operand tile too small for its waves");
  static_assert(!KM || CH == 16 || CH == 8 || CH == 4, "k-major LDS rows hold 128-32 halves");
  static_assert(KM || CH == 4 || CH == 8 || CH == 16 || CH == 32,
                "x-major LDS rows hold 32-256 halves");
};

// A BM x BN tile of C computed by WM x WN wavefronts, each owning a (BM/WM) x (BN/WN) block.
template <int BM_, int BN_, int BK_, bool AKM, bool BKM, int WM_, int WN_>
struct Tile {
  static constexpr int WM = WM_, WN = WN_, NW = WM * WN, NT = 64 * NW;  // waves, threads
  // The 256 x 256 x 64 tile on 2 x 2 wavefronts issues 16x16x32 MFMAs (see ring_tile and,
  // for its generic form, gemm_generic): on random operands that instruction does more work
  // per joule, and large GEMMs run at the chip's power limit.  Every other tile keeps 32x32x16.
  static constexpr bool M16 = BM_ == 256 && BN_ == 256 && BK_ == 64 && WM_ == 2 && WN_ == 2;
  static constexpr int XB = M16 ? 16 : 32, KD = M16 ? 32 : 16, VN = M16 ? 4 : 16;
  using Acc = std::conditional_t<M16, float4v, float16v>;
  using OA = Opnd<BM_, BK_, AKM, WM, NW, XB>;
  using OB = Opnd<BN_, BK_, BKM, WN, NW, XB>;
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int WTM = BM / WM, WTN = BN / WN; // per-wave block of C
  static constexpr int TM = OA::T, TN = OB::T;       // 32x32 MFMA blocks per wave
  static constexpr int A_BYTES = OA::BYTES, B_BYTES = OB::BYTES;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_LD = OA::LD, B_LD = OB::LD;
};

// Element offset of (x, k) inside an operand stored with leading dimension ld, and the
// extent (elements from the first element to one past the last, (X-1, K-1)).
template <bool KM>
__device__ __forceinline__ int64_t elem_off(int64_t x, int64_t k, int64_t ld) {
  return KM ? x * ld + k : k * ld + x;
}
template <bool KM>
__device__ __forceinline__ int64_t extent(int64_t X, int64_t K, int64_t ld) {
  return KM ? (X - 1) * ld + K : (K - 1) * ld + X;
}

// The hardware range-checks each dword of a buffer load on its own and returns 0 for a dword
// that reaches past num_records, even partly.  The extent is therefore rounded up to whole
// dwords: a matrix whose last element ends 2 bytes into a dword still gets that element.  The
// 2 extra bytes share a dword (hence a page) with valid data, and they only ever land in
// slots that are masked (k >= K) or never stored (rows >= M, columns >= N).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  // Saturate to [0, 2^32 - 4] with 32-bit scalar operations only (no 64-bit compares, which
  // the scalar unit lacks and would move to the vector unit).
  const uint64_t b = (uint64_t)(bytes + 3) & ~(uint64_t)3;
  const uint32_t hi = (uint32_t)(b >> 32), lo = (uint32_t)b;
  const uint32_t n = (hi & 0x80000000u) ? 0u : (hi ? 0xFFFFFFFCu : lo);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

// Buffer-resource fields of consecutive panels of one operand, stepped one panel at a time:
// the byte address of the panel's corner and the bytes from there to one past the matrix's
// last element, rounded up to a dword (the step is a multiple of 4 bytes, so the rounding
// stays exact).  Gives the same resource as make_rsrc(corner, bytes) for a live panel, and an
// empty one (no memory touched, zeros) for a panel past the end.
struct PanelSeq {
  uint64_t addr;
  int64_t rem, step;
  __device__ __forceinline__ void init(const uint16_t* base, int64_t e0, int64_t ext,
                                       int64_t step_elems) {
    addr = (uint64_t)(uintptr_t)base + 2 * (uint64_t)e0;
    rem = (2 * (ext - e0) + 3) & ~(int64_t)3;
    step = 2 * step_elems;
  }
  // A live panel starts before the matrix's end (rem > 0); more than 4 GiB saturates.  The
  // high word passes through an empty asm so that the test stays one 32-bit scalar compare
  // (a 64-bit compare would go to the vector unit).
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(bool live) const {
    uint32_t hi = (uint32_t)((uint64_t)rem >> 32);
    asm("" : "+s"(hi));
    const uint32_t lo = (uint32_t)rem;
    const uint32_t n = live ? (hi != 0 ? 0xFFFFFFFCu : lo) : 0u;
    return __builtin_amdgcn_make_buffer_rsrc((void*)addr, (short)0, (int)n, 0x00020000);
  }
  __device__ __forceinline__ void next() {
    addr += (uint64_t)step;
    rem -= step;
  }
};

// 16-byte buffer -> LDS load: lane l's 16 bytes from (resource, voff) land at dst + 16 l.
// The builtin exists only for the device; in the host pass of this single-source file the
// call must not appear at all, or the kernels' host launch stubs are not emitted.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, void GK_LDS* dst,
                                                  uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, 0);
#else
  (void)r, (void)dst, (void)voff;
#endif
}

// Swizzles.  How gfx950 serves LDS reads (measured with one-wave probes and the
// SQ_LDS_BANK_CONFLICT counter): 64 banks of 4 bytes, i.e. a 256-byte bank line of 16
// 16-byte bank groups.  ds_read_b128 takes 4 cycles of 16 lanes each, and the 16 lanes of a
// cycle are not consecutive: within each half of the wave (lanes 0-31, 32-63) the 4-lane
// quads are split by the parity of the quad index (bits 2-4 of the lane), so lanes 0-3,
// 12-15, 20-23 and 24-27 share a cycle, and so do 4-7, 8-11, 16-19 and 28-31.
// ds_read_b64_tr_b16 takes 2 cycles, lanes 0-31 and 32-63.  A conflict-free read gives the
// lanes of each cycle 16 distinct bank groups (32 distinct 8-byte halves for the transposing
// read).
//  * k-major, 256-byte rows (BK = 128): every row starts on the same bank, and swz = r mod 16
//    puts 16 consecutive rows on the 16 bank groups.
//  * k-major, 128-byte rows (BK = 64): two rows per bank line; swz = bits 1-3 of r.  With
//    32x32x16 MFMAs a cycle reads rows {4q .. 4q+3} for four quads q of one parity at one
//    chunk; with 16x16x32 MFMAs rows 0-15 at two chunks.  Both land on 16 distinct groups.
//  * k-major, 64-byte rows (BK = 32): four rows per bank line; swz = (b2, b2 xor b3) from
//    bits 2 and 3 of r, which serves both MFMA layouts.
//    All three depend on r mod 16, so rows 16 or 32 apart (the next MFMA block) share the
//    swizzle and their addresses differ by a constant.
//  * x-major: a transposing read covers 4 consecutive rows x 2 (16 lanes) chunks per 16-lane
//    group; the XOR values 0, 10, 4, 14 for r % 4 = 0..3 (masked to the row's chunk count)
//    spread the 32 lanes of a cycle over distinct banks.  With 16x16x32 MFMAs the two groups
//    of a cycle read rows 8 apart, which an extra XOR of 2 by bit 3 of r separates.  Rows of 4
//    chunks (64 bytes) need none: 4 consecutive rows already fill one 256-byte bank line.
template <class O>
__device__ __forceinline__ int swz(int r) {
  if constexpr (O::KM) {
    if constexpr (O::CH == 16)
      return r & 15;
    else if constexpr (O::CH == 8)
      return (r >> 1) & 7;
    else
      return ((r >> 2) & 1) | ((((r >> 2) ^ (r >> 3)) & 1) << 1);
  } else if constexpr (O::CH == 4) {
    return 0;
  } else {
    const int base = ((0xE4A0 >> (4 * (r & 3))) & 0xF) & (O::CH - 1);
    if constexpr (O::XB == 16)
      return base ^ ((((r >> 3) & 1) << 1) & (O::CH - 1));
    return base;
  }
}

// LDS byte offset of logical chunk c of row r of a panel.
template <class O>
__device__ __forceinline__ int lds_chunk(int r, int c) {
  return r * O::ROW_BYTES + ((c ^ swz<O>(r)) << 4);
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

// Per-lane LDS byte offsets of a wave's operand reads inside one stage.  k-major: one per k
// step (block t adds 32 rows, which keep the swizzle, so that is an immediate).  x-major: one
// per 32-wide block (k step kk and the second 4-deep read add whole rows, which keep
// row % 4 and hence the swizzle; also immediates).
template <class T>
struct LaneOffsets {
  int a[T::OA::NOFF];
  int b[T::OB::NOFF];
};

template <class O>
__device__ __forceinline__ void operand_offsets(int (&o)[O::NOFF], int wx, int lane, int base) {
  if constexpr (O::KM) {
#pragma unroll
    for (int kk = 0; kk < O::BK / O::KD; ++kk) {
      if constexpr (O::XB == 32)
        o[kk] = base + lds_chunk<O>(wx * O::WX + (lane & 31), kk * 2 + (lane >> 5));
      else
        o[kk] = base + lds_chunk<O>(wx * O::WX + (lane & 15), kk * 4 + (lane >> 4));
    }
  } else {
    // Lane 4e + j of a 16-lane group g addresses row (g/2)*8 + e and the 4 halves at
    // x = (g%2)*16 + 4j of its block: the group's 4 x 16 block then transposes into lane
    // i <- column i, i.e. lane l gets x = l % 32 and k = 8(l/32) + 0..3.
    const int g = lane >> 4, i = lane & 15;
#pragma unroll
    for (int t = 0; t < O::T; ++t) {
      if constexpr (O::XB == 32) {
        const int x = wx * O::WX + t * 32 + (g & 1) * 16 + (i & 3) * 4;
        o[t] = base + lds_chunk<O>((g >> 1) * 8 + (i >> 2), x >> 3) + ((x & 7) << 1);
      } else {
        // group g holds k = 8g .. 8g+7 of columns t*16 + 0..15
        const int x = wx * O::WX + t * 16 + (i & 3) * 4;
        o[t] = base + lds_chunk<O>(g * 8 + (i >> 2), x >> 3) + ((x & 7) << 1);
      }
    }
  }
}

template <class T>
__device__ __forceinline__ LaneOffsets<T> lane_offsets(int wm, int wn, int lane) {
  LaneOffsets<T> o;
  operand_offsets<typename T::OA>(o.a, wm, lane, 0);
  operand_offsets<typename T::OB>(o.b, wn, lane, T::A_BYTES);
  return o;
}

// Operand block t of k step kk from the stage at `st`.
template <class O>
__device__ __forceinline__ half8 read_operand(const char GK_LDS* st, const int (&o)[O::NOFF],
                                              int t, int kk) {
  if constexpr (O::KM) {
    return *(const half8 GK_LDS*)(st + o[kk] + t * O::XB * O::ROW_BYTES);
  } else {
    const char GK_LDS* p = st + o[t] + kk * O::KD * O::ROW_BYTES;
    short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((short4v GK_LDS*)p);
    short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((short4v GK_LDS*)(p + 4 * O::ROW_BYTES));
    return __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
}

// Reads the operands of k step kk from the stage at `st`.
template <class T>
__device__ __forceinline__ void read_frags(Frag<T>& f, const char GK_LDS* st,
                                           const LaneOffsets<T>& o, int kk) {
#pragma unroll
  for (int tm = 0; tm < T::TM; ++tm) f.a[tm] = read_operand<typename T::OA>(st, o.a, tm, kk);
#pragma unroll
  for (int tn = 0; tn < T::TN; ++tn) f.b[tn] = read_operand<typename T::OB>(st, o.b, tn, kk);
}

// One 16x16x32 MFMA accumulating in place on accumulator registers.  Written as inline asm:
// through the builtin the compiler copied every 4-register accumulator once per MFMA.  The
// compiler's hazard checks do not see inside the asm, so the code around it provides the wait
// states the hardware needs (CDNA3/CDNA4 ISA guides, "Dependency Resolution: Required
// Independent Instructions"); every asm here is volatile, and volatile asms keep their order:
//  * VALU or v_accvgpr_write of an accumulator, then an MFMA reading it as SrcC (a few wait
//    states): `mfma16_pin_zero` pins the zeroed accumulators in place and issues 8 wait
//    states after them, before any MFMA of the tile.
//  * MFMA result, then v_accvgpr_read or any other read of it (the longest entry of the
//    table, for a 16-pass MFMA, is under 20 wait states): `mfma16_drain` issues 32 wait
//    states after the tile's last MFMA and only then hands the accumulators back to the
//    compiler, so no read is scheduled above it.
//  * An LDS load overwriting an MFMA's A or B operand registers while it may still read them:
//    the operand ring holds two k steps, and a register is reloaded at the earliest 8 MFMAs
//    (over 100 cycles) after the last MFMA that read it (see `panel` in ring_tile).
//  * MFMA result fed to the next MFMA on the same accumulator (SrcC = vdst, same size): back
//    to back is allowed; here 63 other MFMAs lie between.
__device__ __forceinline__ void mfma16(float4v& acc, const half8& a, const half8& b) {
  asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

template <class T>
__device__ __forceinline__ void mfma16_pin_zero(typename T::Acc (&acc)[T::TM][T::TN]) {
#pragma unroll
  for (int tm = 0; tm < T::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < T::TN; ++tn) asm volatile("" : "+a"(acc[tm][tn]));
  asm volatile("s_nop 7" ::: "memory");
}

template <class T>
__device__ __forceinline__ void mfma16_drain(typename T::Acc (&acc)[T::TM][T::TN]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int tm = 0; tm < T::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < T::TN; ++tn) asm volatile("" : "+a"(acc[tm][tn]));
}

template <class T>
__device__ __forceinline__ void mfma_step(typename T::Acc (&acc)[T::TM][T::TN], const Frag<T>& f) {
#pragma unroll
  for (int tm = 0; tm < T::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < T::TN; ++tn) {
      if constexpr (T::M16)   // in place on accumulator registers (see mfma16)
        mfma16(acc[tm][tn], f.a[tm], f.b[tn]);
      else
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a[tm], f.b[tn], acc[tm][tn], 0, 0, 0);
    }
}

// One whole staged panel, operands read just before use (generic path).
template <class T>
__device__ __forceinline__ void mma_panel(const char GK_LDS* st, typename T::Acc (&acc)[T::TM][T::TN],
                                          const LaneOffsets<T>& o) {
#pragma unroll
  for (int kk = 0; kk < T::BK / T::KD; ++kk) {
    Frag<T> f;
    read_frags<T>(f, st, o, kk);
    mfma_step<T>(acc, f);
  }
}

// ---------------------------------------------------------------------------------------
// Epilogue: narrow once (fp32 -> fp16, round to nearest even) and store the wave's block.
// Only C[i][j] with i < M and j < N is written: columns past N are masked per 32-column block
// and, in the last tile row, rows past M per element.  (The buffer resource's range check is
// not relied on: its extent is rounded up to a whole dword, so a store one element past C's
// last element would still land.)  Per lane, one VGPR holds the byte offset of its first
// element; row steps are scalar offsets and 32-column steps immediates.
// ---------------------------------------------------------------------------------------
template <class T>
__device__ __forceinline__ void store_tile(const Args& p, const typename T::Acc (&acc)[T::TM][T::TN],
                                           int m0, int n0, int wm, int wn, int lane) {
  const int64_t c0 = (int64_t)m0 * p.ldc + n0;
  const int64_t extC = (int64_t)(p.M - 1) * p.ldc + p.N;
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.C + c0, 2 * (extC - c0));
  const int col = wn * T::WTN + (lane & (T::XB - 1));
  const int row = wm * T::WTM + (lane / T::XB) * 4;
  const uint32_t vbase = 2u * ((uint32_t)row * (uint32_t)p.ldc + (uint32_t)col);
  const uint32_t ldc2 = 2u * (uint32_t)p.ldc;
  const int ncols = p.N - n0;   // columns of this tile that exist
  const int nrows = p.M - m0;   // rows of this tile that exist
  auto store = [&](int tm, int tn, int v) __attribute__((always_inline)) {
    const int r = T::M16 ? tm * 16 + v : tm * 32 + (v >> 2) * 8 + (v & 3);
    const _Float16 h = (_Float16)acc[tm][tn][v];
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, h), rc,
                                          vbase + tn * T::XB * 2, (uint32_t)r * ldc2, 0);
  };
  if (nrows >= T::BM && ncols >= T::BN) {
    // Whole tile: row by row of the wave's block, so that the stores completing each
    // 128-byte line of C follow one another.
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm)
#pragma unroll
      for (int v = 0; v < T::VN; ++v)
#pragma unroll
        for (int tn = 0; tn < T::TN; ++tn) store(tm, tn, v);
  } else {
#pragma unroll
    for (int tn = 0; tn < T::TN; ++tn) {
      if (col + tn * T::XB < ncols) {
#pragma unroll
        for (int tm = 0; tm < T::TM; ++tm) {
#pragma unroll
          for (int v = 0; v < T::VN; ++v) {
            const int r = T::M16 ? tm * 16 + v : tm * 32 + (v >> 2) * 8 + (v & 3);
            if (row + r < nrows) store(tm, tn, v);
          }
        }
      }
    }
  }
}

// Split-K epilogue: the fp32 accumulators of one k slice, unrounded, into the workspace (same
// lane layout and masks as store_tile; the slice's M x N block starts at `w`).
template <class T>
__device__ __forceinline__ void store_partial(const Args& p, float* w,
                                             const typename T::Acc (&acc)[T::TM][T::TN], int m0,
                                             int n0, int wm, int wn, int lane) {
  const int64_t w0 = (int64_t)m0 * p.ldw + n0;
  const int64_t extW = (int64_t)(p.M - 1) * p.ldw + p.N;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(w + w0, 4 * (extW - w0));
  const int col = wn * T::WTN + (lane & (T::XB - 1));
  const int row = wm * T::WTM + (lane / T::XB) * 4;
  const uint32_t vbase = 4u * ((uint32_t)row * (uint32_t)p.ldw + (uint32_t)col);
  const uint32_t ldw4 = 4u * (uint32_t)p.ldw;
  const int ncols = p.N - n0, nrows = p.M - m0;
#pragma unroll
  for (int tn = 0; tn < T::TN; ++tn) {
    if (col + tn * T::XB < ncols) {
#pragma unroll
      for (int tm = 0; tm < T::TM; ++tm) {
#pragma unroll
        for (int v = 0; v < T::VN; ++v) {
          const int r = T::M16 ? tm * 16 + v : tm * 32 + (v >> 2) * 8 + (v & 3);
          // the element by value first: a bit_cast of the subscript itself reads element 0
          const float x = acc[tm][tn][v];
          if (row + r < nrows)
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), rw,
                                                  vbase + tn * T::XB * 4, (uint32_t)r * ldw4, 0);
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
// Operand loading for the DMA path.
//
// Load slot q = (i*NW + w)*64 + lane of a panel (NW waves; thread q mod 64 NW owns it) holds
// the chunk at position q % CH of LDS row q / CH, i.e. logical chunk (q % CH) ^ swz(row).
// Relative to the panel's corner in global memory that chunk starts 2 (row * ld + 8 chunk)
// bytes in, for either storage order (an LDS row is an x row of a k-major operand, a k row
// of an x-major one).
// ---------------------------------------------------------------------------------------
template <class O>
__device__ __forceinline__ void slot_offsets(uint32_t (&off)[O::LD], int w, int lane,
                                             int64_t ld) {
#pragma unroll
  for (int i = 0; i < O::LD; ++i) {
    const int q = (i * O::NW + w) * 64 + lane;
    const int r = q / O::CH, c = (q % O::CH) ^ swz<O>(r);
    off[i] = 2u * ((uint32_t)r * (uint32_t)ld + (uint32_t)(c * 8));
  }
}

// Full panel at (x0, k0), k0 >= 0: 16-byte DMA into the operand's part of a stage (load slots
// I0 <= i < I1 of each thread; all of them by default).  A panel that is not live gets an empty
// resource: its loads touch no memory and deposit zeros.
template <class O, int I0 = 0, int I1 = O::LD>
__device__ __forceinline__ void dma_panel(const uint16_t* ptr, int64_t ld, int64_t ext, int x0,
                                          int64_t k0, bool live, const uint32_t (&off)[O::LD],
                                          char GK_LDS* dst, int w) {
  const int64_t e0 = elem_off<O::KM>(x0, k0, ld);
  const __amdgpu_buffer_rsrc_t r = make_rsrc(ptr + (live ? e0 : 0), live ? 2 * (ext - e0) : 0);
#pragma unroll
  for (int i = I0; i < I1; ++i)
    buffer_load_lds16(r, (void GK_LDS*)(dst + (i * O::NW + w) * 1024), off[i]);
}

// Head panel at (x0, kofs), kofs < 0: the same slots, through registers, with k < 0 read as
// zero and never addressed (nothing before the matrix's first element is touched).  k-major:
// element by element, since a chunk may straddle k = 0; x-major: whole chunks of the rows
// with k >= 0.
template <class O>
__device__ __forceinline__ void head_load(u32x4 (&v)[O::LD], const uint16_t* ptr, int64_t ld,
                                          int64_t ext, int x0, int kofs, int w, int lane) {
  const int64_t e0 = elem_off<O::KM>(x0, 0, ld);
  const __amdgpu_buffer_rsrc_t r = make_rsrc(ptr + e0, 2 * (ext - e0));
#pragma unroll
  for (int i = 0; i < O::LD; ++i) {
    const int q = (i * O::NW + w) * 64 + lane;
    const int row = q / O::CH, c = (q % O::CH) ^ swz<O>(row);
    if constexpr (O::KM) {
      uint16_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = kofs + c * 8 + e;
        h[e] = k >= 0 ? __builtin_amdgcn_raw_buffer_load_b16(
                            r, 2u * ((uint32_t)row * (uint32_t)ld + (uint32_t)k), 0, 0)
                      : (uint16_t)0;
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) v[i][d] = (uint32_t)h[2 * d] | ((uint32_t)h[2 * d + 1] << 16);
    } else {
      const int k = kofs + row;
      v[i] = k >= 0 ? __builtin_amdgcn_raw_buffer_load_b128(
                          r, 2u * ((uint32_t)k * (uint32_t)ld + (uint32_t)(c * 8)), 0, 0)
                    : u32x4{0u, 0u, 0u, 0u};
    }
  }
}

template <class O>
__device__ __forceinline__ void head_store(const u32x4 (&v)[O::LD], char GK_LDS* dst, int w,
                                           int lane) {
#pragma unroll
  for (int i = 0; i < O::LD; ++i)
    *(u32x4 GK_LDS*)(dst + ((i * O::NW + w) * 64 + lane) * 16) = v[i];
}

// The operand's last element (X-1, K-1) in the last panel.  A 16-byte load that starts 2
// bytes into a dword is range-checked dword by dword from its own start, so when the matrix
// ends on a 4-byte boundary the dword holding its last element reaches 2 bytes past the end
// and reads as zero.  The thread whose load slot holds that element (local k = BK-1 of the
// last panel, in the tile that contains x = X-1) rewrites it from an exact 2-byte load once
// the panel has landed.  Returns the element's LDS byte offset within the operand's part of
// a stage (and its value), or -1 for every other thread.
template <class O>
__device__ __forceinline__ int last_element_slot(int x0, int X, int K, const uint16_t* ptr,
                                                 int64_t ext, int tid, uint16_t& value) {
  const int xl = X - 1 - x0;
  if (K <= 0 || xl >= O::BX) return -1;
  int q, byte;
  if constexpr (O::KM) {
    q = xl * O::CH + ((O::CH - 1) ^ swz<O>(xl));
    byte = 7 * 2;
  } else {
    q = (O::BK - 1) * O::CH + ((xl >> 3) ^ swz<O>(O::BK - 1));
    byte = (xl & 7) * 2;
  }
  if ((q & (O::NW * 64 - 1)) != tid) return -1;
  value = __builtin_amdgcn_raw_buffer_load_b16(make_rsrc(ptr + ext - 1, 2), 0u, 0, 0);
  return q * 16 + byte;
}

// ---------------------------------------------------------------------------------------
// DMA path (any shape, any 2-byte alignment, any leading dimension, either storage order of
// each operand).
//
// Panels are BK deep.  When BK does not divide K, panel 0 is a "head" that holds the first
// K mod BK values of k at its end and zeros in front: the run is then the same, bit for bit,
// as a run on operands zero-padded in front of k to a multiple of BK, and every later panel
// is a full one.  Full panels are loaded with 16-byte buffer->LDS DMA; the buffer resources
// end at the matrices' last elements, so nothing past a matrix is read (it reads as zero).
// Rows and columns past M or N only feed results that are never stored.  The head is loaded
// through registers and written to LDS in the same layout.
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
// The NS LDS stages of a DMA kernel: separate __shared__ objects (so that the compiler can
// tell a refill of one stage from reads of another and does not wait for the refill), and
// the array S of their addresses.
#define GK_DECLARE_STAGES(NS, BYTES)                                                          \
  __shared__ __attribute__((aligned(16))) char stage0[BYTES];                                 \
  __shared__ __attribute__((aligned(16))) char stage1[BYTES];                                 \
  __shared__ __attribute__((aligned(16))) char stage2[(NS) > 2 ? (BYTES) : 16];               \
  __shared__ __attribute__((aligned(16))) char stage3[(NS) > 3 ? (BYTES) : 16];               \
  __shared__ __attribute__((aligned(16))) char stage4[(NS) > 4 ? (BYTES) : 16];               \
  __shared__ __attribute__((aligned(16))) char stage5[(NS) > 5 ? (BYTES) : 16];               \
  __shared__ __attribute__((aligned(16))) char stage6[(NS) > 6 ? (BYTES) : 16];               \
  __shared__ __attribute__((aligned(16))) char stage7[(NS) > 7 ? (BYTES) : 16];               \
  __shared__ __attribute__((aligned(16))) char stage8[(NS) > 8 ? (BYTES) : 16];               \
  __shared__ __attribute__((aligned(16))) char stage9[(NS) > 9 ? (BYTES) : 16];               \
  __shared__ __attribute__((aligned(16))) char stage10[(NS) > 10 ? (BYTES) : 16];             \
  __shared__ __attribute__((aligned(16))) char stage11[(NS) > 11 ? (BYTES) : 16];             \
  __shared__ __attribute__((aligned(16))) char stage12[(NS) > 12 ? (BYTES) : 16];             \
  __shared__ __attribute__((aligned(16))) char stage13[(NS) > 13 ? (BYTES) : 16];             \
  __shared__ __attribute__((aligned(16))) char stage14[(NS) > 14 ? (BYTES) : 16];             \
  __shared__ __attribute__((aligned(16))) char stage15[(NS) > 15 ? (BYTES) : 16];             \
  char GK_LDS* const S[kMaxStages] = {                                                        \
      (char GK_LDS*)stage0,  (char GK_LDS*)stage1,  (char GK_LDS*)stage2,                     \
      (char GK_LDS*)stage3,  (char GK_LDS*)stage4,  (char GK_LDS*)stage5,                     \
      (char GK_LDS*)stage6,  (char GK_LDS*)stage7,  (char GK_LDS*)stage8,                     \
      (char GK_LDS*)stage9,  (char GK_LDS*)stage10, (char GK_LDS*)stage11,                    \
      (char GK_LDS*)stage12, (char GK_LDS*)stage13, (char GK_LDS*)stage14,                    \
      (char GK_LDS*)stage15};

// One BM x BN tile of C with corner (m0, n0) on the LDS stages S: the k loop over all panels
// and the store narrowed into C, or (SPLIT) over panels [p0, p1) with the fp32 partial stored
// into the workspace block `ws`.
template <int BM, int BN, int BK, int NS, int RD, int WM, int WN, bool AKM, bool BKM,
          bool SPLIT = false>
__device__ __forceinline__ void dma_tile(const Args& p, int m0, int n0,
                                         char GK_LDS* const (&S)[kMaxStages], int p0 = 0,
                                         int p1 = 0, float* ws = nullptr) {
  using T = Tile<BM, BN, BK, AKM, BKM, WM, WN>;
  using OA = typename T::OA;
  using OB = typename T::OB;
  constexpr int KS = BK / T::KD;           // k steps per panel
  constexpr int NM = T::TM * T::TN;        // MFMAs per k step
  constexpr int ND = OA::READS + OB::READS;  // LDS reads per k step
  constexpr int NV = T::A_LD + T::B_LD;    // buffer->LDS loads per panel
  // NS == 2, RD == 1: a quarter of each refill is issued one k step later (see `panel`)
  constexpr bool kSplitRefill = NS == 2 && RD == 1 && T::B_LD >= 2;
  static_assert(KS % 2 == 0 && NS >= 2 && NS <= kMaxStages, "pipeline shape");
  static_assert(NS * T::STAGE <= 160 * 1024, "LDS");
  static_assert((NS - 2) * NV <= 63, "vmcnt range");
  static_assert(RD >= 1 && RD < KS && (NS * KS) % (RD + 1) == 0, "read-ahead distance");

  // The thread index passes through an empty asm so that nothing derived from it (LDS and
  // global offsets) is hoisted out of a persistent tile loop, where it would stay live across
  // the whole k loop and push the accumulators' registers into scratch.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / WN, wn = w % WN;

  uint32_t offA[T::A_LD], offB[T::B_LD];
  slot_offsets<OA>(offA, w, lane, p.lda);
  slot_offsets<OB>(offB, w, lane, p.ldb);

  const int64_t extA = extent<AKM>(p.M, p.K, p.lda);
  const int64_t extB = extent<BKM>(p.N, p.K, p.ldb);
  const int rk0 = p.K % BK;                      // depth of the head panel (0: none)
  const int np_all = p.K / BK + (rk0 ? 1 : 0);   // panels of the whole k range
  // Split K: this call's panels are [p0, p1) of the whole sequence (0 < p0 < p1 <= np_all or
  // p0 == 0), renumbered from 0.  Only the slice holding panel 0 has the head; only the one
  // holding the last panel patches.
  const int np = SPLIT ? p1 - p0 : np_all;       // panels of this call
  const int rk = SPLIT && p0 != 0 ? 0 : rk0;
  const bool has_last = !SPLIT || p1 == np_all;
  // panel s covers k in [kofs + s BK, + BK)
  const int kofs = (rk0 ? rk0 - BK : 0) + (SPLIT ? p0 * BK : 0);

  uint16_t last_a = 0, last_b = 0;
  const int patch_a = last_element_slot<OA>(m0, p.M, p.K, p.A, extA, tid, last_a);
  const int patch_b = last_element_slot<OB>(n0, p.N, p.K, p.B, extB, tid, last_b);
  auto patch = [&](char GK_LDS* base) __attribute__((always_inline)) {
    if (patch_a >= 0) *(uint16_t GK_LDS*)(base + patch_a) = last_a;
    if (patch_b >= 0) *(uint16_t GK_LDS*)(base + T::A_BYTES + patch_b) = last_b;
  };

  // Full panel s (k0 = kofs + s BK >= 0) into `base`; panels s >= np load zeros.  `part`
  // splits it: 1 = A's slots and the first half of B's, 2 = the rest of B's (0 = all).
  constexpr int kBHalf = T::B_LD / 2;
  auto issue = [&](int s, char GK_LDS* base, int part = 0) __attribute__((always_inline)) {
    const bool live = s < np;
    const int64_t k0 = (int64_t)kofs + (int64_t)s * BK;
    if (part != 2) dma_panel<OA>(p.A, p.lda, extA, m0, k0, live, offA, base, w);
    if (part == 0)
      dma_panel<OB>(p.B, p.ldb, extB, n0, k0, live, offB, base + T::A_BYTES, w);
    else if (part == 1)
      dma_panel<OB, 0, kBHalf>(p.B, p.ldb, extB, n0, k0, live, offB, base + T::A_BYTES, w);
    else
      dma_panel<OB, kBHalf, T::B_LD>(p.B, p.ldb, extB, n0, k0, live, offB, base + T::A_BYTES, w);
  };

  // Head panel (k0 = kofs < 0).
  auto head = [&](char GK_LDS* base) __attribute__((always_inline)) {
    u32x4 va[T::A_LD], vb[T::B_LD];
    head_load<OA>(va, p.A, p.lda, extA, m0, kofs, w, lane);
    head_load<OB>(vb, p.B, p.ldb, extB, n0, kofs, w, lane);
    head_store<OA>(va, base, w, lane);
    head_store<OB>(vb, base + T::A_BYTES, w, lane);
  };

  typename T::Acc acc[T::TM][T::TN];
#pragma unroll
  for (int tm = 0; tm < T::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < T::TN; ++tn)
      acc[tm][tn] = typename T::Acc{};

  const LaneOffsets<T> lo = lane_offsets<T>(wm, wn, lane);
  // Operands are read RD k steps ahead of the MFMAs that use them: a ring of RD + 1
  // fragments, indexed by the k step's position in the NS-panel unrolled loop.
  Frag<T> f[RD + 1];
  static_assert(!T::M16, "the 16x16x32 tile runs on ring_tile");

  // Panel s from stage `cur` (position j in the unrolled loop), with panel s+1 in `nxt`;
  // `prev` held panel s-1.  K step kk multiplies the operands of step kk and reads those of
  // step kk + RD, which from kk = KS - RD on lie in panel s+1: that is where this panel's
  // barrier sits (after it every wave has read all of panel s, and panel s+1 has landed).
  //  * NS == 2: right past the barrier, `cur` is refilled with panel s+2.  With RD == 1 the
  //    barrier sits in the last k step, which then also issues 16 MFMAs, the next panel's first
  //    operand reads and the refill; a quarter of the refill (the second half of B's slots) is
  //    moved to the first k step of panel s+1, which thins that step out and still leaves the
  //    loads three k steps before they are waited for (measured: 1.2 % faster at 8192^3 on
  //    random and on all-zero operands, same results).  Moving more of it one k step later,
  //    or part of it two k steps later, measured slower at 8192^3 on low-activity data, where
  //    the clock is highest and the loads run out of slack.
  //  * NS >= 3: `prev` is refilled with panel s+NS-1 at the start of the panel, its loads
  //    spread over the first k step's MFMAs.  Every wave finished reading `prev` before the
  //    previous panel's barrier (which waits for the wave's own LDS reads), so no further
  //    synchronisation is needed, and this panel's barrier only has to see panel s+1 land.
  auto panel = [&](int s, int j, char GK_LDS* cur, char GK_LDS* nxt, char GK_LDS* prev)
                   __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      if constexpr (NS >= 3) {
        if (kk == 0) issue(s + NS - 1, prev);
      }
      if constexpr (kSplitRefill) {
        // the rest of panel s+1's refill, started at the previous panel's barrier (panel 1 was
        // loaded whole before the loop)
        if (kk == 0 && s > 0) issue(s + 1, nxt, 2);
      }
      if (kk == KS - RD) {
        wait_vmcnt<(NS - 2) * NV>();   // panel s+1 has landed (this wave's part)
        if (has_last && s + 2 == np) patch(nxt);   // panel s+1 is the last one
        lds_barrier();                 // ... every wave's part
        if constexpr (NS == 2) issue(s + NS, cur, kSplitRefill ? 1 : 0);
      }
      const int ka = kk + RD;
      if (ka < KS)
        read_frags<T>(f[(j * KS + ka) % (RD + 1)], cur, lo, ka);
      else
        read_frags<T>(f[(j * KS + ka) % (RD + 1)], nxt, lo, ka - KS);
      mfma_step<T>(acc, f[(j * KS + kk) % (RD + 1)]);
      if constexpr (NS >= 3) {
        if (kk == 0)
          sched_step<NM, ND, NV>();
        else
          sched_step<NM, ND, 0>();
      } else if constexpr (kSplitRefill) {
        if (kk == KS - RD)
          sched_step<NM, ND, T::A_LD + kBHalf>();
        else if (kk == 0)
          sched_step<NM, ND, T::B_LD - kBHalf>();
        else
          sched_step<NM, ND, 0>();
      } else {
        if (kk == KS - RD)
          sched_step<NM, ND, NV>();
        else
          sched_step<NM, ND, 0>();
      }
    }
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
    if (has_last && np == 1) patch(S[0]);
    lds_barrier();
#pragma unroll
    for (int d = 0; d < RD; ++d) read_frags<T>(f[d], S[0], lo, d);
  }
  for (int s = 0; s < np; s += NS) {
#pragma unroll
    for (int j = 0; j < NS; ++j)
      panel(s + j, j, S[j], S[(j + 1) % NS], S[(j + NS - 1) % NS]);
  }
  // The last refills (of panels past the end) must land before the workgroup's LDS is freed
  // (or reused for another tile).
  wait_vmcnt<0>();
  if constexpr (SPLIT)
    store_partial<T>(p, ws, acc, m0, n0, wm, wn, lane);
  else
    store_tile<T>(p, acc, m0, n0, wm, wn, lane);
}

// ---------------------------------------------------------------------------------------
// The 256 x 256 x 64 tile on 16x16x32 MFMAs (one workgroup per program, each tile of the
// persistent schedule, and the split-K slices): the operand panels in five LDS slots of 32 KiB
// (all 160 KiB), B's in a ring of three and A's in a ring of two.
// With two 64 KiB stages a panel's whole refill can only start at the barrier that frees its
// stage; here B of panel s+2 goes to the slot that held B of panel s-1 -- free since panel
// s-1's barrier -- and is loaded during panel s's first k step, and A of panel s+2 goes to
// A's slot of panel s after panel s's barrier.  Each k step then issues 8 loads per wave,
// one every 8 MFMAs, instead of 12 in one step and 4 in the other, and B's loads have two k
// steps to land.  (B gets the early slot: measured 3.3-3.8 % fewer cycles than with A in it,
// at G = 4 and 8; an XCD's 4 x 8 block of tiles at G = 4 reads 8 B panels and 4 A panels per
// k step.)  Per panel s:
//   first k step:  MFMAs of step 0 (operands in registers), reads of step 1's operands from
//                  panel s's slots, B of panel s+2 loaded; A's resource of panel s+2 computed.
//   barrier:       this wave's loads of panel s+1 have landed (only B of panel s+2 may be in
//                  flight), then every wave's.
//   second k step: MFMAs of step 1, reads of panel s+1's step 0 operands, A of panel s+2
//                  loaded; B's resource of panel s+3 computed.
// Slot indices repeat every 6 panels, so the loop is unrolled by 6 and leaves after the last
// panel.  The k order of every element's sum is the one of the other schedules: same bits.
// As in dma_tile, SPLIT runs panels [p0, p1) only and stores the fp32 partial into `ws`.
// ---------------------------------------------------------------------------------------
template <bool AKM, bool BKM, bool SPLIT = false>
__device__ __forceinline__ void ring_tile(const Args& p, int m0, int n0,
                                          char GK_LDS* const (&SA)[2],
                                          char GK_LDS* const (&SB)[3], int p0 = 0, int p1 = 0,
                                          float* ws = nullptr) {
  using T = Tile<256, 256, 64, AKM, BKM, 2, 2>;
  using OA = typename T::OA;
  using OB = typename T::OB;
  constexpr int BK = 64;
  static_assert(T::M16 && OA::BYTES == 32768 && OB::BYTES == 32768 && T::A_LD == 8 &&
                T::B_LD == 8 && T::TM == 8 && T::TN == 8, "ring tile shape");
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / 2, wn = w % 2;
  uint32_t offA[T::A_LD], offB[T::B_LD];
  slot_offsets<OA>(offA, w, lane, p.lda);
  slot_offsets<OB>(offB, w, lane, p.ldb);
  const int64_t extA = extent<AKM>(p.M, p.K, p.lda);
  const int64_t extB = extent<BKM>(p.N, p.K, p.ldb);
  const int rk0 = p.K % BK;                     // depth of the head panel (0: none)
  const int np_all = p.K / BK + (rk0 ? 1 : 0);  // panels of the whole k range
  // split K (see dma_tile): panels [p0, p1) renumbered from 0, the head only in the first
  // slice, the last element's patch only in the last
  const int np = SPLIT ? p1 - p0 : np_all;
  const int rk = SPLIT && p0 != 0 ? 0 : rk0;
  const bool has_last = !SPLIT || p1 == np_all;
  // panel s covers k in [kofs + s BK, + BK)
  const int kofs = (rk0 ? rk0 - BK : 0) + (SPLIT ? p0 * BK : 0);
  uint16_t last_a = 0, last_b = 0;
  const int patch_a = last_element_slot<OA>(m0, p.M, p.K, p.A, extA, tid, last_a);
  const int patch_b = last_element_slot<OB>(n0, p.N, p.K, p.B, extB, tid, last_b);
  auto patch = [&](char GK_LDS* a, char GK_LDS* b) __attribute__((always_inline)) {
    if (!has_last) return;
    if (patch_a >= 0) *(uint16_t GK_LDS*)(a + patch_a) = last_a;
    if (patch_b >= 0) *(uint16_t GK_LDS*)(b + patch_b) = last_b;
  };

  typename T::Acc acc[T::TM][T::TN];
#pragma unroll
  for (int tm = 0; tm < T::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < T::TN; ++tn) acc[tm][tn] = typename T::Acc{};
  mfma16_pin_zero<T>(acc);

  int oa[OA::NOFF], ob[OB::NOFF];   // per-lane read offsets inside a slot
  operand_offsets<OA>(oa, wm, lane, 0);
  operand_offsets<OB>(ob, wn, lane, 0);
  Frag<T> f[2];                     // f[0]: step 0's operands, f[1]: step 1's

  // refill resources: B's of panel s+2 (s+3 once stepped in the second k step), A's of s+2
  PanelSeq qa{}, qb{};
  {
    const int64_t k2 = (int64_t)kofs + 2 * BK;
    qa.init(p.A, elem_off<OA::KM>(m0, k2, p.lda), extA, OA::KM ? BK : (int64_t)BK * p.lda);
    qb.init(p.B, elem_off<OB::KM>(n0, k2, p.ldb), extB, OB::KM ? BK : (int64_t)BK * p.ldb);
  }
  __amdgpu_buffer_rsrc_t rb = qb.rsrc(2 < np), ra = rb;
  qb.next();

  if (np > 0) {
    if (rk) {
      u32x4 va[T::A_LD], vb[T::B_LD];
      head_load<OA>(va, p.A, p.lda, extA, m0, kofs, w, lane);
      head_load<OB>(vb, p.B, p.ldb, extB, n0, kofs, w, lane);
      head_store<OA>(va, SA[0], w, lane);
      head_store<OB>(vb, SB[0], w, lane);
    } else {
      dma_panel<OA>(p.A, p.lda, extA, m0, kofs, true, offA, SA[0], w);
      dma_panel<OB>(p.B, p.ldb, extB, n0, kofs, true, offB, SB[0], w);
    }
    const int64_t k1 = (int64_t)kofs + BK;
    dma_panel<OA>(p.A, p.lda, extA, m0, k1, 1 < np, offA, SA[1], w);
    dma_panel<OB>(p.B, p.ldb, extB, n0, k1, 1 < np, offB, SB[1], w);
    wait_vmcnt<T::A_LD + T::B_LD>();   // panel 0 has landed
    if (np == 1) patch(SA[0], SB[0]);
    lds_barrier();
#pragma unroll
    for (int t = 0; t < T::TN; ++t) f[0].b[t] = read_operand<OB>(SB[0], ob, t, 0);
#pragma unroll
    for (int t = 0; t < T::TM; ++t) f[0].a[t] = read_operand<OA>(SA[0], oa, t, 0);
  }

  // Panel s at position j of the unrolled loop: A in SA[j % 2], B in SB[j % 3].  Each k step
  // is scheduled by hand (the MFMAs are asm): one operand read of the next step after every
  // fourth MFMA, B fragments first, and one refill load every 8 MFMAs from MFMA 2 on.
  auto panel = [&](int s, int j) __attribute__((always_inline)) {
    char GK_LDS* const a_cur = SA[j % 2];
    char GK_LDS* const b_cur = SB[j % 3];
    char GK_LDS* const a_nxt = SA[(j + 1) % 2];
    char GK_LDS* const b_nxt = SB[(j + 1) % 3];
    char GK_LDS* const b_new = SB[(j + 2) % 3];   // B of panel s+2 (held B of panel s-1)
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      if (i >= 2 && (i - 2) % 8 == 0) {
        const int q = (i - 2) / 8;
        buffer_load_lds16(rb, (void GK_LDS*)(b_new + (q * OB::NW + w) * 1024), offB[q]);
      }
      mfma16(acc[i / 8][i % 8], f[0].a[i / 8], f[0].b[i % 8]);
      // A's resource of panel s+2; the empty asms keep this scalar work between MFMAs 16
      // and 24, where the matrix core has queued work, rather than next to the barrier
      if (i == 16) {
        asm volatile("" : "+s"(qa.addr), "+s"(qa.rem));
        ra = qa.rsrc(s + 2 < np);
        qa.next();
      }
      if (i == 24) asm volatile("" : "+s"(ra));
      if (i % 4 == 0) {
        const int r = i / 4;
        if (r < 8)
          f[1].b[r] = read_operand<OB>(b_cur, ob, r, 1);
        else
          f[1].a[r - 8] = read_operand<OA>(a_cur, oa, r - 8, 1);
      }
    }
    wait_vmcnt<T::B_LD>();   // panel s+1 has landed (this wave's part) ...
    if (s + 2 == np) patch(a_nxt, b_nxt);   // panel s+1 is the last one
    lds_barrier();           // ... every wave's part; and every wave has read A of panel s
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      if (i >= 2 && (i - 2) % 8 == 0) {
        const int q = (i - 2) / 8;
        buffer_load_lds16(ra, (void GK_LDS*)(a_cur + (q * OA::NW + w) * 1024), offA[q]);
      }
      mfma16(acc[i / 8][i % 8], f[1].a[i / 8], f[1].b[i % 8]);
      if (i == 16) {   // B's resource of panel s+3, for the next panel's first k step
        asm volatile("" : "+s"(qb.addr), "+s"(qb.rem));
        rb = qb.rsrc(s + 3 < np);
        qb.next();
      }
      if (i == 24) asm volatile("" : "+s"(rb));
      if (i % 4 == 0) {
        const int r = i / 4;
        if (r < 8)
          f[0].b[r] = read_operand<OB>(b_nxt, ob, r, 0);
        else
          f[0].a[r - 8] = read_operand<OA>(a_nxt, oa, r - 8, 0);
      }
    }
  };
  for (int s = 0; s < np; s += 6) {
#pragma unroll
    for (int j = 0; j < 6; ++j) {
      if (s + j >= np) break;
      panel(s + j, j);
    }
  }
  // The last refills (of panels past the end: empty resources) must land before the
  // workgroup's LDS is freed or reused for another tile.
  wait_vmcnt<0>();
  mfma16_drain<T>(acc);
  if constexpr (SPLIT)
    store_partial<T>(p, ws, acc, m0, n0, wm, wn, lane);
  else
    store_tile<T>(p, acc, m0, n0, wm, wn, lane);
}

// The five LDS slots of ring_tile: separate LDS objects, whose pointers are assigned one by
// one (an initializer list of LDS addresses would become a static table).
#define GK_DECLARE_RING()                                                                     \
  __shared__ __attribute__((aligned(16))) char slot0[32768];                                  \
  __shared__ __attribute__((aligned(16))) char slot1[32768];                                  \
  __shared__ __attribute__((aligned(16))) char slot2[32768];                                  \
  __shared__ __attribute__((aligned(16))) char slot3[32768];                                  \
  __shared__ __attribute__((aligned(16))) char slot4[32768];                                  \
  char GK_LDS* SA[2];                                                                         \
  char GK_LDS* SB[3];                                                                         \
  SA[0] = (char GK_LDS*)slot3;                                                                \
  SA[1] = (char GK_LDS*)slot4;                                                                \
  SB[0] = (char GK_LDS*)slot0;                                                                \
  SB[1] = (char GK_LDS*)slot1;                                                                \
  SB[2] = (char GK_LDS*)slot2;

// Whether a DMA kernel's tile runs on ring_tile (the 256 x 256 x 64 tile on 2 x 2 wavefronts).
template <int BM, int BN, int BK, int NS, int WM, int WN>
constexpr bool kRing = BM == 256 && BN == 256 && BK == 64 && NS == 2 && WM == 2 && WN == 2;

// One workgroup per program: hardware id -> program id -> tile.
template <int BM, int BN, int BK, int NS, int RD, int WM, int WN, bool AKM, bool BKM>
__global__ void __launch_bounds__(64 * WM * WN) gemm_dma(Args p) {
  int pid, pid_m, pid_n;
  program_tile(blockIdx.x, p.num_programs, p.num_pid_m, p.num_pid_n, p.group_m, p.xcd_remap,
               pid, pid_m, pid_n);
  if constexpr (kRing<BM, BN, BK, NS, WM, WN>) {
    GK_DECLARE_RING()
    ring_tile<AKM, BKM>(p, pid_m * BM, pid_n * BN, SA, SB);
  } else {
    GK_DECLARE_STAGES(NS, (Tile<BM, BN, BK, AKM, BKM, WM, WN>::STAGE))
    dma_tile<BM, BN, BK, NS, RD, WM, WN, AKM, BKM>(p, pid_m * BM, pid_n * BN, S);
  }
}

// Persistent grouped schedule: a grid of G workgroups (a multiple of 8, at most the number
// of programs) in which workgroup h computes the tiles of programs h, h + G, h + 2G, ...
// Each of those ids goes through the same map as a hardware id of the one-workgroup-per-
// program launch -- and as G is a multiple of 8 it is dealt to the same XCD -- so every tile
// is computed exactly once and, at any moment, the tiles in flight are those of consecutive
// ids in the grouped order.  Every workgroup leaves the loop after at most
// ceil(P / G) tiles.
template <int BM, int BN, int BK, int NS, int RD, int WM, int WN, bool AKM, bool BKM>
__global__ void __launch_bounds__(64 * WM * WN) gemm_dma_persistent(Args p) {
  if constexpr (kRing<BM, BN, BK, NS, WM, WN>) {
    GK_DECLARE_RING()
    for (int v = blockIdx.x; v < p.num_programs; v += gridDim.x) {
      int pid, pid_m, pid_n;
      program_tile(v, p.num_programs, p.num_pid_m, p.num_pid_n, p.group_m, p.xcd_remap, pid,
                   pid_m, pid_n);
      ring_tile<AKM, BKM>(p, pid_m * BM, pid_n * BN, SA, SB);
      __syncthreads();   // every wave is done with the slots before the next tile's prologue
    }
  } else {
    GK_DECLARE_STAGES(NS, (Tile<BM, BN, BK, AKM, BKM, WM, WN>::STAGE))
    for (int v = blockIdx.x; v < p.num_programs; v += gridDim.x) {
      int pid, pid_m, pid_n;
      program_tile(v, p.num_programs, p.num_pid_m, p.num_pid_n, p.group_m, p.xcd_remap, pid,
                   pid_m, pid_n);
      dma_tile<BM, BN, BK, NS, RD, WM, WN, AKM, BKM>(p, pid_m * BM, pid_n * BN, S);
      __syncthreads();   // every wave is done with the stages before the next tile's prologue
    }
  }
}

// Split K: the k range is cut into `splits` slices at k = K - L, K - 2L, ... (L a multiple of
// 128 k values, so every tile's panel boundaries fall on the cuts and the slices' sums do not
// depend on the tile): slices 1 .. splits-1 hold panels_per_split = L / BK panels each,
// counted back from the last panel, and slice 0 holds the panels in front of them, head panel
// included.  Workgroup b = z P + h (P programs) computes slice z of the tile of program h, h
// going through the same map as a hardware id of the one-workgroup-per-program launch; the
// fp32 partial goes to W[z].  `splitk_reduce` then adds the slices in order and narrows once.
template <int BM, int BN, int BK, int NS, int RD, int WM, int WN, bool AKM, bool BKM>
__global__ void __launch_bounds__(64 * WM * WN) gemm_dma_splitk(Args p) {
  const int z = blockIdx.x / p.num_programs;
  const int h = blockIdx.x - z * p.num_programs;
  int pid, pid_m, pid_n;
  program_tile(h, p.num_programs, p.num_pid_m, p.num_pid_n, p.group_m, p.xcd_remap, pid, pid_m,
               pid_n);
  const int np_all = p.K / BK + (p.K % BK ? 1 : 0);
  const int p1 = np_all - (p.splits - 1 - z) * p.panels_per_split;
  const int p0 = z == 0 ? 0 : p1 - p.panels_per_split;
  float* const ws = p.W + (int64_t)z * p.M * p.ldw;
  if constexpr (kRing<BM, BN, BK, NS, WM, WN>) {
    GK_DECLARE_RING()
    ring_tile<AKM, BKM, true>(p, pid_m * BM, pid_n * BN, SA, SB, p0, p1, ws);
  } else {
    GK_DECLARE_STAGES(NS, (Tile<BM, BN, BK, AKM, BKM, WM, WN>::STAGE))
    dma_tile<BM, BN, BK, NS, RD, WM, WN, AKM, BKM, true>(p, pid_m * BM, pid_n * BN, S, p0, p1,
                                                         ws);
  }
}

// ---------------------------------------------------------------------------------------
// Ping-pong schedule of the 256 x 256 x 32 tile: 8 wavefronts, two per SIMD (the hardware
// deals a workgroup's waves to the 4 SIMDs in order, so waves w and w + 4 share one).  Each
// wave owns a 128 x 64 block of C (16x16x32 MFMAs, 8 x 4 accumulator blocks) and holds the
// operands of one 32-deep panel in registers.  Every wave runs the same sequence per panel
// u -- fetch (its operands of panel u from LDS, and its share of the DMA refill), barrier,
// multiply (32 MFMAs back to back), barrier -- but waves 4-7 start one barrier later, so the
// two waves of a SIMD take turns: in every phase one of them multiplies while the other
// fetches, and the matrix core always has one wave's uninterrupted run of MFMAs to work on.
//
// Panels live in 4 LDS stages (panel u in stage u mod 4).  With waves 0-3 fetching panel u
// in phase 2u and waves 4-7 in phase 2u+1, panel u-1 was last read in phase 2u-1, so while
// fetching panel u every wave refills that stage with its share (4 loads) of panel u+3.
// At the end of its fetch of panel u a wave waits for its share of panel u+1 (the loads of
// u+2 and u+3 may stay in flight), four phases after issuing it; the next barrier then
// precedes the first read of panel u+1.  Loads of panels past the end get empty buffer
// resources (zeros, no memory traffic) so that every wave always has the same loads in
// flight.  The k order of every element's sum is the same sequence of 32-deep MFMA steps as
// in the other schedules, so the results are the same bits.
// ---------------------------------------------------------------------------------------
struct PPTile {   // one wave's block, in the terms store_tile uses
  static constexpr int BM = 256, BN = 256, BK = 32, WM = 2, WN = 4;
  static constexpr int WTM = 128, WTN = 64, XB = 16, KD = 32, TM = 8, TN = 4, VN = 4;
  static constexpr bool M16 = true;
  using Acc = float4v;
};

// The strip.  When the last tile column would hold only a few (1..16) columns, the planner
// launches the grid over the columns left of them, and the workgroups of each tile row compute
// those columns too: 16 rows each, the workgroup in tile column c taking the rows
// 16c .. 16c+15 of its tile row (so the 16 workgroups of a tile row cover its 256 rows).  The
// rows' A operands are already in the registers of one wave (wave c / 8, the one holding rows
// 128 (c/8) .. +127), which issues one more MFMA per panel: that A block times a 32-deep
// B block whose column j is the strip's column j (and whose columns past the strip only feed
// results that are never stored).  That B block is staged per panel by the same wave in 1 KiB
// beside the stage, by one more DMA load.  The sum of a strip element is the same sequence
// of 32-deep MFMA steps as in any tile, so the strip's bits are those of a separate launch.
template <bool BKM>
struct StripB {
  // Load slot of lane l in the 1 KiB staging area: x-major B -> k row l/2, 8 columns at
  // 8 (l%2); k-major B -> strip column l/4, 8 k values at 8 (l%4).
  __device__ static int64_t elem(int lane, int64_t x0, int64_t k0, int64_t ld) {
    return BKM ? (x0 + (lane >> 2)) * ld + k0 + 8 * (lane & 3)
               : (k0 + (lane >> 1)) * ld + x0 + 8 * (lane & 1);
  }
  // LDS byte offset, inside the area, of element (strip column j, panel k value kk).
  __device__ static int at(int j, int kk) { return BKM ? j * 64 + kk * 2 : kk * 32 + j * 2; }
};

template <bool AKM, bool BKM, bool SPLIT = false, bool STRIP = false>
__device__ __forceinline__ void pp_tile(const Args& p, int m0, int n0,
                                        char GK_LDS* const (&S)[kMaxStages], int p0 = 0,
                                        int p1 = 0, float* ws = nullptr) {
  static_assert(!(SPLIT && STRIP), "no strip with split K");
  using T = PPTile;
  using OA = Opnd<256, 32, AKM, 2, 8, 16>;   // operand reads: 2 waves along M
  using OB = Opnd<256, 32, BKM, 4, 8, 16>;   // operand reads: 4 waves along N
  constexpr int BK = 32, NS = 4, TM = T::TM, TN = T::TN;
  constexpr int A_BYTES = OA::BYTES;
  constexpr int NL = OA::LD + OB::LD;          // loads per wave per panel
  static_assert(OA::T == TM && OB::T == TN && OA::KD == BK && NL == 4, "ping-pong tile shape");

  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w & 1, wn = w >> 1;

  uint32_t offA[OA::LD], offB[OB::LD];
  slot_offsets<OA>(offA, w, lane, p.lda);
  slot_offsets<OB>(offB, w, lane, p.ldb);
  const int64_t extA = extent<AKM>(p.M, p.K, p.lda);
  const int64_t extB = extent<BKM>(p.N, p.K, p.ldb);
  const int rk0 = p.K % BK;                     // depth of the head panel (0: none)
  const int np_all = p.K / BK + (rk0 ? 1 : 0);  // panels of the whole k range
  // Split K: this call's panels are [p0, p1) of the whole sequence, renumbered from 0 (as in
  // dma_tile); only the slice holding panel 0 has the head, only the last one patches.
  const int np = SPLIT ? p1 - p0 : np_all;
  const int rk = SPLIT && p0 != 0 ? 0 : rk0;
  const bool has_last = !SPLIT || p1 == np_all;
  // panel u covers k in [kofs + u BK, + BK)
  const int kofs = (rk0 ? rk0 - BK : 0) + (SPLIT ? p0 * BK : 0);

  // the last element of each operand, rewritten by the thread whose load slot holds it
  uint16_t last_a = 0, last_b = 0;
  const int patch_a = last_element_slot<OA>(m0, p.M, p.K, p.A, extA, tid, last_a);
  const int patch_b = last_element_slot<OB>(n0, p.N, p.K, p.B, extB, tid, last_b);
  // The strip (see StripB): this tile column's 16-row block sb, if any, is computed by wave
  // sb / 8.  Its last element (the matrix's last) is rewritten like the operands' (see
  // last_element_slot) by the lane whose load slot holds it.
  constexpr int STRIP_AT = A_BYTES + OB::BYTES;   // staging area inside a stage
  const int sb = n0 / 256;
  const bool strip_wave = STRIP && sb < 16 && w == (sb >> 3);
  const int strip_tm = sb & 7;
  const int64_t sx0 = p.N;                        // first strip column
  const int64_t extBs = STRIP ? extent<BKM>(p.N + p.strip_n, p.K, p.ldb) : 0;
  int patch_s = -1;
  uint16_t last_s = 0;
  if (strip_wave && p.K > 0) {
    const int j = p.strip_n - 1, kk = (p.K - 1 - kofs) % BK;
    const int q = BKM ? 4 * j + (kk >> 3) : 2 * kk + (j >> 3);
    if (q == lane) {
      patch_s = StripB<BKM>::at(j, kk);
      last_s = __builtin_amdgcn_raw_buffer_load_b16(make_rsrc(p.B + extBs - 1, 2), 0u, 0, 0);
    }
  }
  auto patch = [&](char GK_LDS* base) __attribute__((always_inline)) {
    if (!has_last) return;
    if (patch_a >= 0) *(uint16_t GK_LDS*)(base + patch_a) = last_a;
    if (patch_b >= 0) *(uint16_t GK_LDS*)(base + A_BYTES + patch_b) = last_b;
    if (STRIP && patch_s >= 0) *(uint16_t GK_LDS*)(base + STRIP_AT + patch_s) = last_s;
  };
  // This wave's share of full panel u (k0 >= 0); panels past the end load zeros.
  auto issue = [&](int u, char GK_LDS* base) __attribute__((always_inline)) {
    const bool live = u < np;
    const int64_t k0 = (int64_t)kofs + (int64_t)u * BK;
    dma_panel<OA>(p.A, p.lda, extA, m0, k0, live, offA, base, w);
    dma_panel<OB>(p.B, p.ldb, extB, n0, k0, live, offB, base + A_BYTES, w);
  };
  auto head = [&](char GK_LDS* base) __attribute__((always_inline)) {
    u32x4 va[OA::LD], vb[OB::LD];
    head_load<OA>(va, p.A, p.lda, extA, m0, kofs, w, lane);
    head_load<OB>(vb, p.B, p.ldb, extB, n0, kofs, w, lane);
    head_store<OA>(va, base, w, lane);
    head_store<OB>(vb, base + A_BYTES, w, lane);
  };

  auto issue_strip = [&](int u, char GK_LDS* base) __attribute__((always_inline)) {
    const bool live = u < np;
    const int64_t k0 = (int64_t)kofs + (int64_t)u * BK;
    const int64_t e0 = BKM ? sx0 * p.ldb + k0 : k0 * p.ldb + sx0;
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc(p.B + (live ? e0 : 0), live ? 2 * (extBs - e0) : 0);
    const int64_t off = StripB<BKM>::elem(lane, sx0, k0, p.ldb) - e0;
    buffer_load_lds16(r, (void GK_LDS*)(base + STRIP_AT), 2u * (uint32_t)off);
  };
  // head panel of the strip (k0 = kofs < 0): through registers, k < 0 read as zero
  auto head_strip = [&](char GK_LDS* base) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(p.B, 2 * extBs);
    uint16_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t k = BKM ? (int64_t)kofs + 8 * (lane & 3) + e : (int64_t)kofs + (lane >> 1);
      const int64_t x = BKM ? sx0 + (lane >> 2) : sx0 + 8 * (lane & 1) + e;
      h[e] = k >= 0 ? __builtin_amdgcn_raw_buffer_load_b16(
                          r, (uint32_t)(2 * elem_off<BKM>(x, k, p.ldb)), 0, 0)
                    : (uint16_t)0;
    }
    u32x4 v;
#pragma unroll
    for (int d = 0; d < 4; ++d) v[d] = (uint32_t)h[2 * d] | ((uint32_t)h[2 * d + 1] << 16);
    *(u32x4 GK_LDS*)(base + STRIP_AT + lane * 16) = v;
  };
  half8 rs;   // the strip's B operand of the current panel
  auto fetch_strip = [&](const char GK_LDS* st) __attribute__((always_inline)) {
    if constexpr (BKM) {
      rs = *(const half8 GK_LDS*)(st + STRIP_AT + StripB<BKM>::at(lane & 15, 8 * (lane >> 4)));
    } else {
      const int g = lane >> 4, i = lane & 15;
      const char GK_LDS* q = st + STRIP_AT + StripB<BKM>::at((i & 3) * 4, g * 8 + (i >> 2));
      short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((short4v GK_LDS*)q);
      short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((short4v GK_LDS*)(q + 4 * 32));
      rs = __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };

  int oa[OA::NOFF], ob[OB::NOFF];
  operand_offsets<OA>(oa, wm, lane, 0);
  operand_offsets<OB>(ob, wn, lane, A_BYTES);
  half8 ra[TM], rb[TN];
  auto fetch = [&](const char GK_LDS* st) __attribute__((always_inline)) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) ra[tm] = read_operand<OA>(st, oa, tm, 0);
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) rb[tn] = read_operand<OB>(st, ob, tn, 0);
  };

  // Waits until this wave's share of the panel before the last two it issued has landed
  // (the strip's wave has one load more per panel).
  auto wait_panel = [&]() __attribute__((always_inline)) {
    if (STRIP && strip_wave)
      wait_vmcnt<2 * (NL + 1)>();
    else
      wait_vmcnt<2 * NL>();
  };

  // Prologue: panels 0, 1 and 2 (the head through registers), then panel 0 has landed.
  if (np > 0) {
    if (rk)
      head(S[0]);
    else
      issue(0, S[0]);
    if (STRIP && strip_wave) {
      if (rk)
        head_strip(S[0]);
      else
        issue_strip(0, S[0]);
    }
#pragma unroll
    for (int u = 1; u < 3; ++u) {
      issue(u, S[u]);
      if (STRIP && strip_wave) issue_strip(u, S[u]);
    }
    wait_panel();
    if (np == 1) patch(S[0]);
  }

  typename T::Acc acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = typename T::Acc{};
  typename T::Acc acc_s = typename T::Acc{};   // the strip block (strip wave only)

  // The MFMAs go through the builtin here, so that the compiler sees them: this kernel's
  // register allocation moves accumulators between register files around them, and the
  // compiler then keeps the wait states such moves need.
  // The builtins touch no memory, so scheduling barriers keep them inside their phase.
  auto multiply = [&]() __attribute__((always_inline)) {
    // While it multiplies, the wave has the higher issue priority on its SIMD.
    asm volatile("s_setprio 1" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ra[tm], rb[tn], acc[tm][tn], 0, 0, 0);
    if (STRIP && strip_wave) {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
        if (tm == strip_tm) acc_s = __builtin_amdgcn_mfma_f32_16x16x32_f16(ra[tm], rs, acc_s, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_setprio 0" ::: "memory");
  };
  // Panel u from stage j = u mod 4.
  auto panel = [&](int u, int j) __attribute__((always_inline)) {
    fetch(S[j]);
    if (STRIP && strip_wave) fetch_strip(S[j]);
    issue(u + 3, S[(j + 3) % NS]);     // panel u-1's stage, read by every wave by now
    if (STRIP && strip_wave) issue_strip(u + 3, S[(j + 3) % NS]);
    wait_panel();                      // this wave's share of panel u+1 has landed
    if (u + 2 == np) patch(S[(j + 1) % NS]);   // panel u+1 is the last one
    lds_barrier();
    multiply();
    lds_barrier();
  };
  if (np > 0) {
    lds_barrier();                     // panel 0 has landed
    if (w >= 4) lds_barrier();         // waves 4-7 run one phase behind
    for (int u = 0; u < np; u += NS) {
#pragma unroll
      for (int j = 0; j < NS; ++j)
        if (u + j < np) panel(u + j, j);
    }
    if (w < 4) lds_barrier();          // the same number of barriers in every wave
  }
  wait_vmcnt<0>();                     // the empty loads past the end, before LDS is freed
  if constexpr (SPLIT) {
    store_partial<T>(p, ws, acc, m0, n0, wm, wn, lane);
  } else {
    store_tile<T>(p, acc, m0, n0, wm, wn, lane);
    if constexpr (STRIP) {
      if (strip_wave) {
        // lane l holds rows 4 (l/16) + v, v = 0..3, of the block, strip column l % 16
        const int j = lane & 15, r0 = m0 + 16 * sb + 4 * (lane >> 4);
        const int64_t extC = (int64_t)(p.M - 1) * p.ldc + p.N + p.strip_n;
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.C, 2 * extC);
        if (j < p.strip_n) {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (r0 + v < p.M) {
              const _Float16 h = (_Float16)acc_s[v];
              __builtin_amdgcn_raw_buffer_store_b16(
                  __builtin_bit_cast(uint16_t, h), rc,
                  (uint32_t)(2 * ((int64_t)(r0 + v) * p.ldc + p.N + j)), 0, 0);
            }
        }
      }
    }
  }
}

template <bool AKM, bool BKM, bool STRIP>
__global__ void __launch_bounds__(512) gemm_pp(Args p) {
  GK_DECLARE_STAGES(4, 32768 + (STRIP ? 1024 : 0))
  int pid, pid_m, pid_n;
  program_tile(blockIdx.x, p.num_programs, p.num_pid_m, p.num_pid_n, p.group_m, p.xcd_remap,
               pid, pid_m, pid_n);
  pp_tile<AKM, BKM, false, STRIP>(p, pid_m * 256, pid_n * 256, S);
}

// The persistent grouped schedule (see gemm_dma_persistent) on the ping-pong tile.
template <bool AKM, bool BKM>
__global__ void __launch_bounds__(512) gemm_pp_persistent(Args p) {
  GK_DECLARE_STAGES(4, 32768)
  for (int v = blockIdx.x; v < p.num_programs; v += gridDim.x) {
    int pid, pid_m, pid_n;
    program_tile(v, p.num_programs, p.num_pid_m, p.num_pid_n, p.group_m, p.xcd_remap, pid,
                 pid_m, pid_n);
    pp_tile<AKM, BKM>(p, pid_m * 256, pid_n * 256, S);
    __syncthreads();   // every wave is done with the stages before the next tile's prologue
  }
}

// Split K (see gemm_dma_splitk) on the ping-pong tile.
template <bool AKM, bool BKM>
__global__ void __launch_bounds__(512) gemm_pp_splitk(Args p) {
  GK_DECLARE_STAGES(4, 32768)
  const int z = blockIdx.x / p.num_programs;
  const int h = blockIdx.x - z * p.num_programs;
  int pid, pid_m, pid_n;
  program_tile(h, p.num_programs, p.num_pid_m, p.num_pid_n, p.group_m, p.xcd_remap, pid, pid_m,
               pid_n);
  const int np_all = p.K / 32 + (p.K % 32 ? 1 : 0);
  const int p1 = np_all - (p.splits - 1 - z) * p.panels_per_split;
  const int p0 = z == 0 ? 0 : p1 - p.panels_per_split;
  pp_tile<AKM, BKM, true>(p, pid_m * 256, pid_n * 256, S, p0, p1,
                          p.W + (int64_t)z * p.M * p.ldw);
}

// C[i][j] = fp16(W[0][i][j] + W[1][i][j] + ... + W[splits-1][i][j]): the slices added in
// order in fp32, then one narrowing (round to nearest even).  Thread t covers row
// i = t / (ldw / 4), columns j .. j + 3 with j = 4 (t mod (ldw / 4)); ldw is a multiple of 4
// and W 16-byte aligned, so the reads are whole float4s (columns past N are read, not stored).
__global__ void __launch_bounds__(256) splitk_reduce(const float* W, int64_t ldw, int splits,
                                                     int M, int N, uint16_t* C, int64_t ldc) {
  const uint32_t q4 = (uint32_t)(ldw >> 2);   // M q4 < 2^31 (checked on the host)
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  if (t >= (uint32_t)M * q4) return;
  const uint32_t i = t / q4;
  const int j = (int)(t - i * q4) * 4;
  const int64_t slice = (int64_t)M * ldw;
  const float* w = W + (int64_t)i * ldw + j;
  // loads issued 8 at a time (in flight together), added strictly in slice order
  float4v sum = *(const float4v*)w;
  int z = 1;
  for (; z + 8 <= splits; z += 8) {
    float4v v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *(const float4v*)(w + (z + u) * slice);
#pragma unroll
    for (int u = 0; u < 8; ++u) sum += v[u];
  }
  for (; z < splits; ++z) sum += *(const float4v*)(w + z * slice);
  uint16_t* c = C + (int64_t)i * ldc + j;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const _Float16 h = (_Float16)sum[e];
    if (j + e < N) c[e] = __builtin_bit_cast(uint16_t, h);
  }
}

// ---------------------------------------------------------------------------------------
// Generic path: any leading dimension, any 2-byte alignment, any K, either storage order of
// each operand.  Panels are fetched with raw buffer loads whose resource ends at the
// matrix's last element, so reads past it return zero and never fault; the last panel's
// slots with k >= K (chunks of a k-major operand, rows of an x-major one) are zeroed
// explicitly.
// kOdd: some row starts are only 2-byte aligned, so each 16-byte chunk is assembled from a
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

// Slot q = i*NT + t of a panel (NT threads) holds logical chunk q % CH of LDS row q / CH.
template <class O, bool kOdd>
__device__ __forceinline__ void generic_fetch(u32x4 (&v)[O::LD], const uint16_t* ptr,
                                              int64_t ld, int64_t ext, int x0, int k0, int K,
                                              int t) {
  const int64_t e0 = elem_off<O::KM>(x0, k0, ld);
  const __amdgpu_buffer_rsrc_t r = make_rsrc(ptr + e0, 2 * (ext - e0));
  const bool tail = k0 + O::BK > K;
#pragma unroll
  for (int i = 0; i < O::LD; ++i) {
    const int q = i * O::NW * 64 + t;
    const int row = q / O::CH, c = q % O::CH;
    v[i] = load_chunk<kOdd>(r, 2u * ((uint32_t)row * (uint32_t)ld + (uint32_t)(c * 8)));
    if constexpr (O::KM) {
      if (tail) v[i] = mask_k(v[i], k0 + c * 8, K);
    } else {
      // Rows k >= K start past the matrix's last element, but the resource's extent is
      // rounded up to a whole dword, which can admit the one element after it: with unpadded
      // rows (ld = X) that is row K, x = 0.  Whatever it holds would be multiplied by the zero
      // of the other operand at k = K, and Inf or NaN times zero is NaN, so those rows are
      // zeroed like the k-major chunks past K.
      if (tail && k0 + row >= K) v[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

template <class O>
__device__ __forceinline__ void generic_deposit(const u32x4 (&v)[O::LD], char GK_LDS* dst,
                                                int t) {
#pragma unroll
  for (int i = 0; i < O::LD; ++i) {
    const int q = i * O::NW * 64 + t;
    *(u32x4 GK_LDS*)(dst + lds_chunk<O>(q / O::CH, q % O::CH)) = v[i];
  }
}

template <int BM, int BN, bool kOdd, int WM, int WN, bool AKM, bool BKM>
__global__ void __launch_bounds__(64 * WM * WN) gemm_generic(Args p) {
  using T = Tile<BM, BN, kBK, AKM, BKM, WM, WN>;
  using OA = typename T::OA;
  using OB = typename T::OB;
  __shared__ __attribute__((aligned(16))) char smem[2 * T::STAGE];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w / WN, wn = w % WN;

  int pid, pid_m, pid_n;
  program_tile(blockIdx.x, p.num_programs, p.num_pid_m, p.num_pid_n, p.group_m, p.xcd_remap,
               pid, pid_m, pid_n);
  const int m0 = pid_m * BM, n0 = pid_n * BN;
  const int nk = (p.K + T::BK - 1) / T::BK;
  const int64_t extA = extent<AKM>(p.M, p.K, p.lda);
  const int64_t extB = extent<BKM>(p.N, p.K, p.ldb);

  u32x4 ra[T::A_LD], rb[T::B_LD];
  auto fetch = [&](int s) __attribute__((always_inline)) {
    generic_fetch<OA, kOdd>(ra, p.A, p.lda, extA, m0, s * T::BK, p.K, t);
    generic_fetch<OB, kOdd>(rb, p.B, p.ldb, extB, n0, s * T::BK, p.K, t);
  };
  auto deposit = [&](int stage) __attribute__((always_inline)) {
    char GK_LDS* base = (char GK_LDS*)smem + stage * T::STAGE;
    generic_deposit<OA>(ra, base, t);
    generic_deposit<OB>(rb, base + T::A_BYTES, t);
  };

  const LaneOffsets<T> lo = lane_offsets<T>(wm, wn, lane);
  typename T::Acc acc[T::TM][T::TN];
#pragma unroll
  for (int tm = 0; tm < T::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < T::TN; ++tn)
      acc[tm][tn] = typename T::Acc{};
  if constexpr (T::M16) mfma16_pin_zero<T>(acc);

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
  if constexpr (T::M16) mfma16_drain<T>(acc);
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
