// Batch-adaptive twins of RMSNorm and GEMM.  They compute the same
// mathematics as bi_rmsnorm / bi_gemm but choose their split points from the
// batch and the device's 256 compute units, as ordinary serving kernels do
// ("Batch invariance and reproducible inference", "From batch size to
// reduction tree" and "2 . Cross-block accumulation": split-K whose split
// count follows the batch, and a norm whose partial sums meet through atomics
// in whatever order the workgroups land).  They exist to price invariance and
// as the harness's negative control.
#include "api.h"
#include "common.h"

namespace bi {

bool gemm_splitk_slices(const void* A, const void* W, float* C32, int M, int N, int K, int mb,
                        int ct, int splits, int kslice, hipStream_t s);
void gemm_dispatch(const void* A, const void* W, void* C, int M, int N, int K, int out_f32,
                   hipStream_t s);

constexpr int kCUs = 256;

__global__ void k_fill(float* __restrict__ p, long n) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) p[i] = 0.f;
}

// out[i] = sum over the split-K slices j = 0 .. splits-1 of part[j n + i]
// (slices in order), converted to the output type.
template <int OUT_DT>
__global__ void k_splitk_reduce(const float* __restrict__ part, void* __restrict__ out, long n,
                                int splits) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    float a = part[i];
    for (int j = 1; j < splits; ++j) a += part[(long)j * n + i];
    Elem<OUT_DT>::st(out, i, a);
  }
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

// The twin's split-K configuration for M <= 256: the tile (mb 8-row blocks by
// ct 16-column strips) and split count s that move the fewest bytes into the
// busiest CU -- rounds of 256 workgroups x (8 mb + 16 ct) rows x K / s -- plus
// the partial sums written and read back; s = 1 means no split.  The row
// count sets how many row groups share the device, so the split count (and
// with it each output's sum tree) follows the batch: at N = K = 4096, eight
// slices up to 64 rows, four at 128.
namespace bi {
struct SplitPick {
  int mb, ct, s, kslice;
};
static SplitPick split_pick(int M, int N, int K) {
  SplitPick best{0, 0, 1, K};
  double best_cost = -1;
  for (int mb : {1, 2, 4, 8}) {
    const long rg = (M + 8 * mb - 1) / (8 * mb);
    if (mb > 1 && 8 * (mb / 2) >= M) continue;   // a smaller block already holds every row
    for (int ct : {2, 4, 8}) {
      for (int s : {1, 2, 4, 8}) {
        const int kslice = ((K + s - 1) / s + 63) / 64 * 64;
        const int se = (K + kslice - 1) / kslice;
        const long wgs = rg * ((N + 16 * ct - 1) / (16 * ct)) * se;
        const double rounds = (double)((wgs + kCUs - 1) / kCUs);
        double cost = rounds * (8.0 * mb + 16.0 * ct) * kslice * 2.0;
        if (se > 1) cost += 2.0 * se * (double)M * N * 4.0 / kCUs;
        if (best_cost < 0 || cost < best_cost) {
          best_cost = cost;
          best = SplitPick{mb, ct, se, kslice};
        }
      }
    }
  }
  return best;
}
}  // namespace bi

constexpr int kSplitMaxRows = 256;

extern "C" size_t bi_gemm_free_workspace_bytes(int M, int N, int K) {
  if (M <= 0 || N <= 0 || K <= 0 || M > kSplitMaxRows) return 0;
  const SplitPick sp = split_pick(M, N, K);
  return sp.s > 1 ? (size_t)sp.s * M * N * sizeof(float) : 0;
}

extern "C" bi_status bi_gemm_free(const void* A, const void* W, void* C, int M, int N, int K,
                                  int in_dtype, int out_dtype, void* workspace,
                                  size_t workspace_bytes, bi_stream stream) {
  BI_REQUIRE(M >= 0 && N >= 1 && K >= 1, BI_ERR_INVALID, "bi_gemm_free: bad shape");
  if (in_dtype != BI_BF16 || M == 0 || M > kSplitMaxRows || K % 8 != 0)
    return bi_gemm(A, W, C, M, N, K, in_dtype, out_dtype, stream);
  BI_REQUIRE(out_dtype == BI_BF16 || out_dtype == BI_F32, BI_ERR_UNSUPPORTED,
             "bi_gemm_free: out dtype %d", out_dtype);
  BI_REQUIRE(A && W && C, BI_ERR_INVALID, "bi_gemm_free: null pointer");
  const SplitPick sp = split_pick(M, N, K);
  if (sp.s == 1) return bi_gemm(A, W, C, M, N, K, in_dtype, out_dtype, stream);
  BI_REQUIRE(workspace && workspace_bytes >= (size_t)sp.s * M * N * sizeof(float),
             BI_ERR_WORKSPACE, "bi_gemm_free: workspace too small");
  hipStream_t s = as_stream(stream);
  float* part = static_cast<float*>(workspace);
  if (!gemm_splitk_slices(A, W, part, M, N, K, sp.mb, sp.ct, sp.s, sp.kslice, s))
    return fail(BI_ERR_UNSUPPORTED, "bi_gemm_free: no split kernel for mb %d ct %d", sp.mb,
                sp.ct);
  const long n = (long)M * N;
  const unsigned g = (unsigned)((n + 255) / 256 < 2048 ? (n + 255) / 256 : 2048);
  if (out_dtype == BI_BF16)
    hipLaunchKernelGGL(k_splitk_reduce<1>, dim3(g), dim3(256), 0, s, part, C, n, sp.s);
  else
    hipLaunchKernelGGL(k_splitk_reduce<0>, dim3(g), dim3(256), 0, s, part, C, n, sp.s);
  return launched("bi_gemm_free");
}
