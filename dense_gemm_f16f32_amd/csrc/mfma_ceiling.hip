// Matrix-core rate probe, for measurement only (bench.py --mfma-ceiling); no part of the GEMM
// calls it.  Every wavefront issues MFMAs back to back on operands held in registers, in the
// pattern of the GEMM's 256 x 256 x 64 tile: a 128 x 128 block of C per wavefront held in 256
// accumulator registers, 64-deep k per iteration split into k steps whose operands differ, and
// per k step each A fragment used by consecutive MFMAs with every B fragment.  There are no
// loads, no LDS traffic and no barriers, so on the GEMM's grid (one wavefront per SIMD) its rate
// is what the matrix cores reach at the clock the board allows for that data: the ceiling for
// the GEMM's own MFMAs.
//
// Two instruction shapes, the same flops per iteration and the same 128 operand registers:
//   v_mfma_f32_16x16x32_f16 (the GEMM's): 64 blocks of 16 x 16, 2 k steps of 32, per k step
//     8 A fragments x 8 B fragments;
//   v_mfma_f32_32x32x16_f16: 16 blocks of 32 x 32, 4 k steps of 16, per k step 4 x 4.
//
// Operands are either +0 or uniform on [-0.5, 0.5) in fp16 (the 8192^3 workload's
// distribution), drawn per thread and element from a 32-bit integer hash of (seed, index).
// The accumulators random-walk as the GEMM's do, since every product is added to them.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));

// Multiply-xorshift integer hash; only needs to give every element its own bits.
__device__ __forceinline__ uint32_t hash32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__device__ __forceinline__ half8 operand(uint32_t seed, uint32_t index, bool zeros) {
  half8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t h = hash32(seed ^ hash32(index * 8u + (uint32_t)e));
    const float u = (float)(h >> 8) * (1.0f / 16777216.0f) - 0.5f;   // [-0.5, 0.5)
    v[e] = (_Float16)(zeros ? 0.0f : u);
  }
  return v;
}

// In place on accumulator registers, as in the GEMM kernel (the builtin would copy them).
__device__ __forceinline__ void mfma(float4v& acc, const half8& a, const half8& b) {
  asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma(float16v& acc, const half8& a, const half8& b) {
  asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// F: the MFMA shape's block count per side of the wavefront's 128 x 128 block (8 for 16 x 16,
// 4 for 32 x 32); S = 16 / F k steps per iteration; ACC its accumulator type.
// Wait states around the asm MFMAs as in the GEMM kernel: 8 after the accumulators are zeroed
// and pinned, 32 after the last MFMA before any accumulator is read; the same accumulator is
// used again only 16 (32 x 32) or 64 (16 x 16) MFMAs later.
template <int F, typename ACC>
__device__ __forceinline__ void probe(float* out, int iters, int zeros, uint32_t seed) {
  constexpr int S = 16 / F;
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  half8 a[S][F], b[S][F];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int i = 0; i < F; ++i) {
      a[s][i] = operand(seed, t * 64u + (uint32_t)(s * F + i), zeros != 0);
      b[s][i] = operand(seed, t * 64u + 32u + (uint32_t)(s * F + i), zeros != 0);
    }
  ACC acc[F][F];
#pragma unroll
  for (int i = 0; i < F; ++i)
#pragma unroll
    for (int j = 0; j < F; ++j) {
      acc[i][j] = ACC{};
      asm volatile("" : "+a"(acc[i][j]));
    }
  asm volatile("s_nop 7" ::: "memory");
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int i = 0; i < F * F; ++i) mfma(acc[i / F][i % F], a[s][i / F], b[s][i % F]);
  }
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < F; ++i)
#pragma unroll
    for (int j = 0; j < F; ++j) {
      asm volatile("" : "+a"(acc[i][j]));
#pragma unroll
      for (int e = 0; e < 256 / (F * F); ++e) sum += acc[i][j][e];
    }
  out[t] = sum;
}

}  // namespace

// out: one float per thread, the sum of its accumulators (so that no MFMA is dead code).
extern "C" __global__ void __launch_bounds__(256) mfma_ceiling(float* out, int iters, int zeros,
                                                              uint32_t seed) {
  probe<8, float4v>(out, iters, zeros, seed);
}
extern "C" __global__ void __launch_bounds__(256) mfma_ceiling_32x32x16(float* out, int iters,
                                                                       int zeros, uint32_t seed) {
  probe<4, float16v>(out, iters, zeros, seed);
}

// blocks workgroups of 256 threads; out holds blocks * 256 floats; shape 0 runs
// v_mfma_f32_16x16x32_f16, 1 v_mfma_f32_32x32x16_f16 (each iteration 128 of the first or 64
// of the second per wavefront, the same flops).  Returns the hipError_t of the launch.
extern "C" int mfma_ceiling_launch(float* out, int blocks, int iters, int shape, int zeros,
                                   uint32_t seed, void* stream) {
  if (out == nullptr || blocks <= 0 || iters < 0 || shape < 0 || shape > 1)
    return (int)hipErrorInvalidValue;
  if (shape == 0)
    hipLaunchKernelGGL(mfma_ceiling, dim3((uint32_t)blocks), dim3(256), 0, (hipStream_t)stream,
                       out, iters, zeros, seed);
  else
    hipLaunchKernelGGL(mfma_ceiling_32x32x16, dim3((uint32_t)blocks), dim3(256), 0,
                       (hipStream_t)stream, out, iters, zeros, seed);
  return (int)hipGetLastError();
}
