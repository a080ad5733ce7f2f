// Batch-adaptive twins of RMSNorm and GEMM.  They compute the same
// mathematics as bi_rmsnorm / bi_gemm but choose their split points from the
// batch and the device's 256 compute units, as ordinary serving kernels do
// ("Batch invariance and reproducible inference", "From batch size to
// reduction tree" and "2 . Cross-block accumulation": split-K merged by
// atomics leaves the order to whichever workgroup lands first).  They exist
// to price invariance and as the harness's negative control.
#include "api.h"
#include "common.h"

namespace bi {

void gemm_splitk_atomic(const void* A, const void* W, float* C32, int M, int N, int K,
                        int splits, int kslice, hipStream_t s);
void gemm_dispatch(const void* A, const void* W, void* C, int M, int N, int K, int out_f32,
                   hipStream_t s);

constexpr int kCUs = 256;

__global__ void k_fill(float* __restrict__ p, long n) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) p[i] = 0.f;
}

template <int OUT_DT>
__global__ void k_convert(const float* __restrict__ src, void* __restrict__ dst, long n) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256)
    Elem<OUT_DT>::st(dst, i, src[i]);
}

// ---- RMSNorm twin ---------------------------------------------------------
// Partial sums of squares of row segments, added into ss[row] by atomics.
template <int DT>
__global__ __launch_bounds__(256) void k_rms_partial(const void* __restrict__ x,
                                                     float* __restrict__ ss, int d, int parts) {
  const long row = blockIdx.x / parts;
  const int part = blockIdx.x % parts;
  const int seg = (d + parts - 1) / parts;
  const int b = part * seg, e = min(d, b + seg);
  float a = 0.f;
  for (int i = b + threadIdx.x; i < e; i += 256) {
    const float v = Elem<DT>::ld(x, row * d + i);
    a = __builtin_fmaf(v, v, a);
  }
  for (int off = 32; off >= 1; off >>= 1) a += __shfl_down(a, off);
  __shared__ float w[4];
  if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) atomicAdd(ss + row, (w[0] + w[1]) + (w[2] + w[3]));
}

template <int DT>
__global__ __launch_bounds__(256) void k_rms_apply(const void* x, const void* __restrict__ g,
                                                   void* y, const float* __restrict__ ss, int d,
                                                   float eps) {
  const long row = blockIdx.x;
  const float r = 1.0f / sqrtf(ss[row] / (float)d + eps);
  for (int i = threadIdx.x; i < d; i += 256)
    Elem<DT>::st(y, row * d + i, (Elem<DT>::ld(x, row * d + i) * r) * Elem<DT>::ld(g, i));
}

// One workgroup per row, contiguous segments per lane and a shfl-down tree
// (an order different from the invariant kernel's).
template <int DT>
__global__ __launch_bounds__(256) void k_rms_onepass(const void* x, const void* __restrict__ g,
                                                     void* y, int d, float eps) {
  const long row = blockIdx.x;
  const int seg = (d + 255) / 256;
  const int b = threadIdx.x * seg, e = min(d, b + seg);
  float a = 0.f;
  for (int i = b; i < e; ++i) {
    const float v = Elem<DT>::ld(x, row * d + i);
    a = __builtin_fmaf(v, v, a);
  }
  for (int off = 32; off >= 1; off >>= 1) a += __shfl_down(a, off);
  __shared__ float w[4];
  if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = a;
  __syncthreads();
  const float ss = (w[0] + w[1]) + (w[2] + w[3]);
  const float r = 1.0f / sqrtf(ss / (float)d + eps);
  for (int i = threadIdx.x; i < d; i += 256)
    Elem<DT>::st(y, row * d + i, (Elem<DT>::ld(x, row * d + i) * r) * Elem<DT>::ld(g, i));
}

}  // namespace bi

using namespace bi;

extern "C" size_t bi_rmsnorm_free_workspace_bytes(int M, int d) {
  (void)d;
  return M > 0 ? (size_t)M * sizeof(float) : 0;
}

extern "C" bi_status bi_rmsnorm_free(const void* x, const void* gamma, void* y, int M, int d,
                                     float eps, int dtype, void* workspace,
                                     size_t workspace_bytes, bi_stream stream) {
  BI_REQUIRE(M >= 0 && d >= 1, BI_ERR_INVALID, "bi_rmsnorm_free: bad shape");
  BI_REQUIRE(dtype == BI_F32 || dtype == BI_BF16, BI_ERR_UNSUPPORTED, "bi_rmsnorm_free: dtype");
  if (M == 0) return BI_OK;
  BI_REQUIRE(x && gamma && y, BI_ERR_INVALID, "bi_rmsnorm_free: null pointer");
  hipStream_t s = as_stream(stream);
  if (M >= kCUs) {
    if (dtype == BI_BF16) hipLaunchKernelGGL(k_rms_onepass<1>, dim3(M), dim3(256), 0, s, x, gamma, y, d, eps);
    else hipLaunchKernelGGL(k_rms_onepass<0>, dim3(M), dim3(256), 0, s, x, gamma, y, d, eps);
    return launched("bi_rmsnorm_free");
  }
  BI_REQUIRE(workspace && workspace_bytes >= bi_rmsnorm_free_workspace_bytes(M, d),
             BI_ERR_WORKSPACE, "bi_rmsnorm_free: workspace too small");
  float* ss = static_cast<float*>(workspace);
  int parts = (2 * kCUs + M - 1) / M;       // enough workgroups to fill the device
  const int maxp = (d + 255) / 256;
  parts = parts < maxp ? parts : maxp;
  parts = parts > 1 ? parts : 1;
  hipLaunchKernelGGL(k_fill, dim3(1), dim3(256), 0, s, ss, (long)M);
  if (dtype == BI_BF16) {
    hipLaunchKernelGGL(k_rms_partial<1>, dim3(M * parts), dim3(256), 0, s, x, ss, d, parts);
    hipLaunchKernelGGL(k_rms_apply<1>, dim3(M), dim3(256), 0, s, x, gamma, y, ss, d, eps);
  } else {
    hipLaunchKernelGGL(k_rms_partial<0>, dim3(M * parts), dim3(256), 0, s, x, ss, d, parts);
    hipLaunchKernelGGL(k_rms_apply<0>, dim3(M), dim3(256), 0, s, x, gamma, y, ss, d, eps);
  }
  return launched("bi_rmsnorm_free");
}

extern "C" size_t bi_gemm_free_workspace_bytes(int M, int N, int K) {
  (void)K;
  return (M > 0 && N > 0) ? (size_t)M * N * sizeof(float) : 0;
}

extern "C" bi_status bi_gemm_free(const void* A, const void* W, void* C, int M, int N, int K,
                                  int in_dtype, int out_dtype, void* workspace,
                                  size_t workspace_bytes, bi_stream stream) {
  BI_REQUIRE(M >= 0 && N >= 1 && K >= 1, BI_ERR_INVALID, "bi_gemm_free: bad shape");
  if (in_dtype != BI_BF16 || M == 0 || M > 64 || K % 32 != 0)
    return bi_gemm(A, W, C, M, N, K, in_dtype, out_dtype, stream);
  BI_REQUIRE(out_dtype == BI_BF16 || out_dtype == BI_F32, BI_ERR_UNSUPPORTED,
             "bi_gemm_free: out dtype %d", out_dtype);
  BI_REQUIRE(A && W && C, BI_ERR_INVALID, "bi_gemm_free: null pointer");
  // Workgroups the small-M kernels would launch along N; split K until the
  // device holds a target that grows as the batch shrinks (fewer rows leave
  // each workgroup less work to hide its latency behind).
  const long tiles = (N + 15) / 16;
  const long target = (M <= 16 ? 4L : 2L) * kCUs;
  if (tiles >= target || K < 1024)
    return bi_gemm(A, W, C, M, N, K, in_dtype, out_dtype, stream);
  BI_REQUIRE(workspace && workspace_bytes >= bi_gemm_free_workspace_bytes(M, N, K),
             BI_ERR_WORKSPACE, "bi_gemm_free: workspace too small");
  int splits = (int)((target + tiles - 1) / tiles);
  splits = splits < 8 ? splits : 8;
  int kslice = (K + splits - 1) / splits;
  kslice = (kslice + 255) & ~255;               // whole pipeline stages
  splits = (K + kslice - 1) / kslice;
  hipStream_t s = as_stream(stream);
  float* c32 = static_cast<float*>(workspace);
  const long n = (long)M * N;
  hipLaunchKernelGGL(k_fill, dim3((unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096)),
                     dim3(256), 0, s, c32, n);
  gemm_splitk_atomic(A, W, c32, M, N, K, splits, kslice, s);
  const unsigned g = (unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
  if (out_dtype == BI_BF16) hipLaunchKernelGGL(k_convert<1>, dim3(g), dim3(256), 0, s, c32, C, n);
  else hipLaunchKernelGGL(k_convert<0>, dim3(g), dim3(256), 0, s, c32, C, n);
  return launched("bi_gemm_free");
}
