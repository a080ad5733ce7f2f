// The fixed-order pieces of the RMSNorm row reduction, shared by the norm
// kernels and by the small-batch GEMM that normalises its own rows of A, so
// that both evaluate the same expressions in the same order ("Batch
// invariance and reproducible inference": rms_norm reduces each row inside
// one block; "Lockstep", "The fix": every forward-pass reduction in one
// fixed order).  256 lanes per row: lane t folds vectors t, t + 256, ... of
// 8 consecutive elements into a = fma(x, x, a), element by element; each
// 64-lane wave then reduces by xor butterfly 32, 16, 8, 4, 2, 1; the four
// wave sums are added in wave order.
#pragma once

#include "common.h"

namespace bi {

// a after folding the 8 elements of one vector
__device__ __forceinline__ float rn_fold8(const float* x, float a) {
#pragma unroll
  for (int e = 0; e < 8; ++e) a = __builtin_fmaf(x[e], x[e], a);
  return a;
}

// the sum over the 64 lanes of a wave (every lane gets it)
__device__ __forceinline__ float rn_wave_sum(float a) {
  a = a + __shfl_xor(a, 32);
  a = a + __shfl_xor(a, 16);
  a = a + __shfl_xor(a, 8);
  a = a + __shfl_xor(a, 4);
  a = a + __shfl_xor(a, 2);
  a = a + __shfl_xor(a, 1);
  return a;
}

// 1 / sqrt(mean + eps) from the four wave sums of a row of d elements
__device__ __forceinline__ float rn_inv_rms(const float* ws, int d, float eps) {
  const float ss = ((ws[0] + ws[1]) + ws[2]) + ws[3];
  const float mean = ss / (float)d;
  return 1.0f / sqrtf(mean + eps);
}

// y = (x * r) * gamma for one vector of 8
__device__ __forceinline__ void rn_scale8(const float* x, const float* g, float r, float* y) {
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = (x[e] * r) * g[e];
}

}  // namespace bi
