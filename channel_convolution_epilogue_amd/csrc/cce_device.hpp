// Device helpers shared by the gfx950 kernels of libcce.
//
// Matrix-core contraction: every kernel runs its convolution as an implicit
// GEMM on v_mfma_f32_16x16x4_f32 (16 pixels x 16 output channels x 4 taps per
// instruction, fp32 in and out).  Lane layout of that instruction, as used
// throughout (lane l of a 64-wide wave):
//   A operand  lane l supplies A[m = l % 16][k = l / 16]     (pixel m, tap k)
//   B operand  lane l supplies B[k = l / 16][n = l % 16]     (tap k, channel n)
//   D result   lane l holds   D[m = 4 * (l / 16) + r][n = l % 16], r = 0..3
// so each lane ends with four consecutive pixels of one output channel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cce {

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f mfma16x16x4(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v4f splat4(float v) { return v4f{v, v, v, v}; }

__device__ __forceinline__ float clampf(float v, float lo, float hi) {
  return fminf(fmaxf(v, lo), hi);
}

// 16-byte global store of four consecutive floats (address 16-byte aligned).
__device__ __forceinline__ void store4(float *p, v4f v) {
  *reinterpret_cast<v4f *>(p) = v;
}

}  // namespace cce
