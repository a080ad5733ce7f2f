// bi_rmsnorm: one workgroup of 256 lanes per row, one fixed reduction tree.
//
// "Batch invariance and reproducible inference" lists rms_norm among the
// kernels that run one block per row with no cross-block reduction, so the
// order cannot follow the batch; "Lockstep", "The fix", asks exactly that of
// every forward-pass reduction.  The order (vectors of 8, lane-strided fma,
// xor butterfly per wave, waves added in order) depends on d only.
#include "api.h"
#include "common.h"
#include "rownorm.h"

namespace bi {

// rows of up to 256 x kNormRegVecs vectors of 8 stay in registers
constexpr int kNormRegVecs = 4;

template <int DT>
__global__ __launch_bounds__(256) void k_rmsnorm(const void* x, const void* __restrict__ gamma,
                                                 void* y, int d, float eps) {
  const long row = blockIdx.x;
  const int t = threadIdx.x;
  const long base = row * (long)d;
  const int nv = (d + 7) >> 3;
  const bool vec = (d & 7) == 0;

  float a = 0.0f;
  for (int v = t; v < nv; v += 256) {
    float xs[8];
    const int i0 = v << 3;
    if (vec) {
      load8<DT>(x, base + i0, xs);
      a = rn_fold8(xs, a);
    } else {
      const int n = min(8, d - i0);
      for (int e = 0; e < n; ++e) {
        const float xv = Elem<DT>::ld(x, base + i0 + e);
        a = __builtin_fmaf(xv, xv, a);
      }
    }
  }
  a = rn_wave_sum(a);
  __shared__ float ws[4];
  if ((t & 63) == 0) ws[t >> 6] = a;
  __syncthreads();
  const float r = rn_inv_rms(ws, d, eps);

  for (int v = t; v < nv; v += 256) {
    const int i0 = v << 3;
    if (vec) {
      float xs[8], gs[8], ys[8];
      load8<DT>(x, base + i0, xs);
      load8<DT>(gamma, i0, gs);
      rn_scale8(xs, gs, r, ys);
      store8<DT>(y, base + i0, ys);
    } else {
      const int n = min(8, d - i0);
      for (int e = 0; e < n; ++e) {
        const float xv = Elem<DT>::ld(x, base + i0 + e);
        Elem<DT>::st(y, base + i0 + e, (xv * r) * Elem<DT>::ld(gamma, i0 + e));
      }
    }
  }
}

// Residual add fused with the next RMSNorm: h = round(h + o) is stored back,
// then y = RMSNorm(h) by the k_rmsnorm tree over the rounded h.  Lane t
// handles the same vectors in both passes, so its second pass re-reads what
// it stored itself.  Bit for bit the two kernels bi_add then bi_rmsnorm.
template <int DT>
__global__ __launch_bounds__(256) void k_add_rmsnorm(void* h, const void* __restrict__ o,
                                                     const void* __restrict__ gamma, void* y,
                                                     int d, float eps) {
  const long row = blockIdx.x;
  const int t = threadIdx.x;
  const long base = row * (long)d;
  const int nv = (d + 7) >> 3;
  const bool vec = (d & 7) == 0;
  if (vec && nv <= 256 * kNormRegVecs) {
    // the row in registers between the two passes (same lanes, same order)
    float xs[kNormRegVecs][8], gs[kNormRegVecs][8];
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < kNormRegVecs; ++j) {
      const int v = t + 256 * j;
      if (v < nv) {
        float os[8];
        load8<DT>(h, base + 8 * v, xs[j]);
        load8<DT>(o, base + 8 * v, os);
        load8<DT>(gamma, 8 * v, gs[j]);
#pragma unroll
        for (int e = 0; e < 8; ++e) xs[j][e] = xs[j][e] + os[e];
        store8<DT>(h, base + 8 * v, xs[j]);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (Elem<DT>::bytes == 2)
            xs[j][e] = bf16_bits_to_f32((uint16_t)f32_to_bf16_bits(xs[j][e]));
        a = rn_fold8(xs[j], a);
      }
    }
    a = rn_wave_sum(a);
    __shared__ float wr[4];
    if ((t & 63) == 0) wr[t >> 6] = a;
    __syncthreads();
    const float r = rn_inv_rms(wr, d, eps);
#pragma unroll
    for (int j = 0; j < kNormRegVecs; ++j) {
      const int v = t + 256 * j;
      if (v < nv) {
        float ys[8];
        rn_scale8(xs[j], gs[j], r, ys);
        store8<DT>(y, base + 8 * v, ys);
      }
    }
    return;
  }

  float a = 0.0f;
  for (int v = t; v < nv; v += 256) {
    const int i0 = v << 3;
    if (vec) {
      float hs[8], os[8], rs[8];
      load8<DT>(h, base + i0, hs);
      load8<DT>(o, base + i0, os);
#pragma unroll
      for (int e = 0; e < 8; ++e) rs[e] = hs[e] + os[e];
      store8<DT>(h, base + i0, rs);
      float xs[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        xs[e] = Elem<DT>::bytes == 2 ? bf16_bits_to_f32((uint16_t)f32_to_bf16_bits(rs[e])) : rs[e];
      a = rn_fold8(xs, a);
    } else {
      const int n = min(8, d - i0);
      for (int e = 0; e < n; ++e) {
        Elem<DT>::st(h, base + i0 + e, Elem<DT>::ld(h, base + i0 + e) + Elem<DT>::ld(o, base + i0 + e));
        const float xv = Elem<DT>::ld(h, base + i0 + e);
        a = __builtin_fmaf(xv, xv, a);
      }
    }
  }
  a = rn_wave_sum(a);
  __shared__ float ws[4];
  if ((t & 63) == 0) ws[t >> 6] = a;
  __syncthreads();
  const float r = rn_inv_rms(ws, d, eps);

  for (int v = t; v < nv; v += 256) {
    const int i0 = v << 3;
    if (vec) {
      float xs[8], gs[8], ys[8];
      load8<DT>(h, base + i0, xs);
      load8<DT>(gamma, i0, gs);
      rn_scale8(xs, gs, r, ys);
      store8<DT>(y, base + i0, ys);
    } else {
      const int n = min(8, d - i0);
      for (int e = 0; e < n; ++e) {
        const float xv = Elem<DT>::ld(h, base + i0 + e);
        Elem<DT>::st(y, base + i0 + e, (xv * r) * Elem<DT>::ld(gamma, i0 + e));
      }
    }
  }
}

}  // namespace bi

extern "C" bi_status bi_add_rmsnorm(void* h, const void* o, const void* gamma, void* y, int M,
                                    int d, float eps, int dtype, bi_stream stream) {
  using namespace bi;
  BI_REQUIRE(M >= 0 && d >= 1, BI_ERR_INVALID, "bi_add_rmsnorm: bad shape M=%d d=%d", M, d);
  BI_REQUIRE(dtype == BI_F32 || dtype == BI_BF16, BI_ERR_UNSUPPORTED,
             "bi_add_rmsnorm: dtype %d not supported", dtype);
  if (M == 0) return BI_OK;
  BI_REQUIRE(h && o && gamma && y, BI_ERR_INVALID, "bi_add_rmsnorm: null pointer");
  BI_REQUIRE(aligned16(h) && aligned16(o) && aligned16(gamma) && aligned16(y), BI_ERR_INVALID,
             "bi_add_rmsnorm: pointers must be 16-byte aligned");
  BI_REQUIRE(y != h && y != o, BI_ERR_INVALID, "bi_add_rmsnorm: y must not alias h or o");
  BI_REQUIRE(eps >= 0.0f, BI_ERR_INVALID, "bi_add_rmsnorm: eps must be >= 0");
  hipStream_t s = as_stream(stream);
  if (dtype == BI_BF16)
    hipLaunchKernelGGL(k_add_rmsnorm<1>, dim3(M), dim3(256), 0, s, h, o, gamma, y, d, eps);
  else
    hipLaunchKernelGGL(k_add_rmsnorm<0>, dim3(M), dim3(256), 0, s, h, o, gamma, y, d, eps);
  return launched("bi_add_rmsnorm");
}

extern "C" bi_status bi_rmsnorm(const void* x, const void* gamma, void* y, int M, int d,
                                float eps, int dtype, bi_stream stream) {
  using namespace bi;
  BI_REQUIRE(M >= 0 && d >= 1, BI_ERR_INVALID, "bi_rmsnorm: bad shape M=%d d=%d", M, d);
  BI_REQUIRE(dtype == BI_F32 || dtype == BI_BF16, BI_ERR_UNSUPPORTED,
             "bi_rmsnorm: dtype %d not supported", dtype);
  if (M == 0) return BI_OK;
  BI_REQUIRE(x && gamma && y, BI_ERR_INVALID, "bi_rmsnorm: null pointer");
  BI_REQUIRE(aligned16(x) && aligned16(gamma) && aligned16(y), BI_ERR_INVALID,
             "bi_rmsnorm: pointers must be 16-byte aligned");
  BI_REQUIRE(eps >= 0.0f, BI_ERR_INVALID, "bi_rmsnorm: eps must be >= 0");
  hipStream_t s = as_stream(stream);
  if (dtype == BI_BF16)
    hipLaunchKernelGGL(k_rmsnorm<1>, dim3(M), dim3(256), 0, s, x, gamma, y, d, eps);
  else
    hipLaunchKernelGGL(k_rmsnorm<0>, dim3(M), dim3(256), 0, s, x, gamma, y, d, eps);
  return launched("bi_rmsnorm");
}
