// Matrix-core rate probe, for measurement only (bench.py --mfma-ceiling); no part of the GEMM
// calls it.  Every wavefront issues v_mfma_f32_16x16x32_f16 back to back on operands held in
// registers, in the pattern of the GEMM's 256 x 256 x 64 tile: 64 accumulator blocks of
// 16 x 16, two k steps whose operands differ, and per k step 8 A fragments each used by 8
// consecutive MFMAs with 8 different B fragments.  There are no loads, no LDS traffic and no
// barriers, so on the GEMM's grid (one wavefront per SIMD) its rate is what the matrix cores
// reach at the clock the board allows for that data: the ceiling for the GEMM's own MFMAs.
//
// Operands are either +0 or uniform on [-0.5, 0.5) in fp16 (the 8192^3 workload's
// distribution), drawn per thread and element from a 32-bit integer hash of (seed, index).
// The accumulators random-walk as the GEMM's do, since every product is added to them.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

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

}  // namespace

// out: one float per thread, the sum of its accumulators (so that no MFMA is dead code).
// Wait states around the asm MFMAs as in the GEMM kernel: 8 after the accumulators are
// zeroed and pinned, 32 after the last MFMA before any accumulator is read; the same
// accumulator is used again only 64 MFMAs later.
extern "C" __global__ void __launch_bounds__(256) mfma_ceiling(float* out, int iters, int zeros,
                                                              uint32_t seed) {
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  half8 a[2][8], b[2][8];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[s][i] = operand(seed, t * 64u + (uint32_t)(s * 8 + i), zeros != 0);
      b[s][i] = operand(seed, t * 64u + 32u + (uint32_t)(s * 8 + i), zeros != 0);
    }
  float4v acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc[i][j] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
      asm volatile("" : "+a"(acc[i][j]));
    }
  asm volatile("s_nop 7" ::: "memory");
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 64; ++i) mfma(acc[i / 8][i % 8], a[s][i / 8], b[s][i % 8]);
  }
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      asm volatile("" : "+a"(acc[i][j]));
      sum += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
    }
  out[t] = sum;
}

// blocks workgroups of 256 threads; out holds blocks * 256 floats.  Returns the hipError_t
// of the launch.
extern "C" int mfma_ceiling_launch(float* out, int blocks, int iters, int zeros, uint32_t seed,
                                   void* stream) {
  if (out == nullptr || blocks <= 0 || iters < 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_ceiling, dim3((uint32_t)blocks), dim3(256), 0, (hipStream_t)stream,
                     out, iters, zeros, seed);
  return (int)hipGetLastError();
}
