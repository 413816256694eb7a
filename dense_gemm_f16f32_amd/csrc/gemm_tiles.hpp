// The tile configurations of the GEMM kernels (ids as in include/gemm_f16f32.h).  Together
// with gemm_kernels.hpp this file fixes the code of every kernel the library can launch;
// the planner (gemm_f16f32.hip) chooses among them.
#pragma once

#include "gemm_f16f32.h"

// The tile configurations: id, BM x BN x BK, NS LDS stages of the DMA kernel, operands read
// RD k steps ahead, WM x WN wavefronts, default GROUP_SIZE_M.  RD = 0 marks the ping-pong
// schedule (gemm_pp), which has no read-ahead of its own.  (The generic kernel stages
// 64-deep panels through registers for every tile.)
#define GEMM_F16F32_TILES(X)                                              \
  X(GEMM_F16F32_TILE_256x256x64, 256, 256, 64, 2, 1, 2, 2, 8)            \
  X(GEMM_F16F32_TILE_128x128x64, 128, 128, 64, 2, 3, 2, 2, 4)            \
  X(GEMM_F16F32_TILE_128x64x64, 128, 64, 64, 2, 1, 2, 2, 4)              \
  X(GEMM_F16F32_TILE_256x128x64, 256, 128, 64, 2, 3, 2, 2, 8)            \
  X(GEMM_F16F32_TILE_256x256x32, 256, 256, 32, 4, 1, 2, 2, 8)            \
  X(GEMM_F16F32_TILE_64x64x32, 64, 64, 32, 5, 1, 2, 2, 4)                \
  X(GEMM_F16F32_TILE_128x64x32, 128, 64, 32, 5, 1, 2, 2, 4)              \
  X(GEMM_F16F32_TILE_256x256x64_W8, 256, 256, 64, 2, 1, 2, 4, 8)         \
  X(GEMM_F16F32_TILE_64x64x64, 64, 64, 64, 4, 3, 2, 2, 4)                \
  X(GEMM_F16F32_TILE_32x32x64, 32, 32, 64, 4, 3, 1, 1, 4)                \
  X(GEMM_F16F32_TILE_32x64x64, 32, 64, 64, 4, 3, 1, 2, 4)                \
  X(GEMM_F16F32_TILE_64x32x64, 64, 32, 64, 4, 3, 2, 1, 4)                \
  X(GEMM_F16F32_TILE_32x64x128, 32, 64, 128, 4, 3, 1, 2, 4)              \
  X(GEMM_F16F32_TILE_64x64x128, 64, 64, 128, 3, 3, 2, 2, 4)              \
  X(GEMM_F16F32_TILE_32x32x128, 32, 32, 128, 4, 3, 1, 1, 4)              \
  X(GEMM_F16F32_TILE_64x32x128, 64, 32, 128, 4, 3, 2, 1, 4)             \
  X(GEMM_F16F32_TILE_256x256x32_PP, 256, 256, 32, 4, 0, 2, 4, 8)
