// Elementwise glue of a Llama-shaped layer: embedding gather, RoPE + KV page
// append, residual add, SwiGLU, argmax.  None of these reduces across the
// batch, so each row's result depends on that row alone; argmax is exact
// (largest value, lowest index on ties) in any evaluation order.
#include "api.h"
#include "common.h"

namespace bi {

template <int DT>
__global__ __launch_bounds__(256) void k_embed(const void* __restrict__ table,
                                               const int32_t* __restrict__ ids,
                                               void* __restrict__ out, int d) {
  const long row = blockIdx.y;
  const long src = (long)ids[row] * d;
  const int vecs = d / 8;
  for (int v = blockIdx.x * 256 + threadIdx.x; v < vecs; v += gridDim.x * 256) {
    float x[8];
    load8<DT>(table, src + 8 * v, x);
    store8<DT>(out, row * d + 8 * v, x);
  }
}

// One thread per rotation pair of one head of one row.
template <int DT>
__global__ __launch_bounds__(256) void k_rope_kv_append(
    const void* __restrict__ qkv, int M, int h, int h_kv, int d_h,
    const int32_t* __restrict__ pos, const float* __restrict__ cos_t,
    const float* __restrict__ sin_t, const int32_t* __restrict__ slot_mapping, int page_size,
    void* __restrict__ q_out, void* __restrict__ k_pool, void* __restrict__ v_pool) {
  const int half = d_h / 2;
  const int heads = h + 2 * h_kv;
  const long tid = (long)blockIdx.x * 256 + threadIdx.x;
  if (tid >= (long)M * heads * half) return;
  const int i = (int)(tid % half);
  const long rh = tid / half;
  const int hh = (int)(rh % heads);
  const long row = rh / heads;
  const long in = row * heads * d_h + (long)hh * d_h;
  const float a = Elem<DT>::ld(qkv, in + i), b = Elem<DT>::ld(qkv, in + i + half);
  float ya = a, yb = b;
  if (hh < h + h_kv && cos_t != nullptr) {
    const long t = (long)pos[row] * half + i;
    const float c = cos_t[t], s = sin_t[t];
    ya = __builtin_fmaf(a, c, -(b * s));
    yb = __builtin_fmaf(b, c, a * s);
  }
  if (hh < h) {
    const long o = (row * h + hh) * (long)d_h;
    Elem<DT>::st(q_out, o + i, ya);
    Elem<DT>::st(q_out, o + i + half, yb);
    return;
  }
  const int g = hh < h + h_kv ? hh - h : hh - h - h_kv;
  const long slot = slot_mapping[row];
  const int t = (int)(slot % page_size);
  const long blk = ((slot / page_size) * h_kv + g) * page_size * (long)d_h;   // (page, head) block
  if (hh < h + h_kv) {   // K: unit-major block (common.h)
    Elem<DT>::st(k_pool, blk + k_block_elem(t, i, page_size, Elem<DT>::bytes), ya);
    Elem<DT>::st(k_pool, blk + k_block_elem(t, i + half, page_size, Elem<DT>::bytes), yb);
  } else {               // V: token-major rows
    Elem<DT>::st(v_pool, blk + (long)t * d_h + i, ya);
    Elem<DT>::st(v_pool, blk + (long)t * d_h + i + half, yb);
  }
}

template <int DT>
__global__ __launch_bounds__(256) void k_add(const void* a, const void* b, void* y, long n) {
  const long nv = n / 8;
  for (long v = (long)blockIdx.x * 256 + threadIdx.x; v < nv; v += (long)gridDim.x * 256) {
    float xa[8], xb[8], r[8];
    load8<DT>(a, 8 * v, xa);
    load8<DT>(b, 8 * v, xb);
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = xa[e] + xb[e];
    store8<DT>(y, 8 * v, r);
  }
  // tail
  const long t = nv * 8 + (long)blockIdx.x * 256 + threadIdx.x;
  if (t < n && (long)blockIdx.x * 256 + threadIdx.x < 8)
    Elem<DT>::st(y, t, Elem<DT>::ld(a, t) + Elem<DT>::ld(b, t));
}

// gu rows in the gate/up product's 8-column blocks: columns 16 v .. 16 v + 7
// are gate columns 8 v .. 8 v + 7, the next 8 the matching up columns.
template <int DT>
__global__ __launch_bounds__(256) void k_silu_mul(const void* __restrict__ gu,
                                                  void* __restrict__ y, int F) {
  const long row = blockIdx.y;
  const int vecs = F / 8;
  for (int v = blockIdx.x * 256 + threadIdx.x; v < vecs; v += gridDim.x * 256) {
    float g[8], u[8], r[8];
    load8<DT>(gu, row * 2 * F + 16 * v, g);
    load8<DT>(gu, row * 2 * F + 16 * v + 8, u);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float s = g[e] / (1.0f + exp_fixed(-g[e]));
      r[e] = s * u[e];
    }
    store8<DT>(y, row * F + 8 * v, r);
  }
}

// Log-softmax: one 1024-thread workgroup per row whatever the number of rows.
// Thread t takes elements t, t + 1024, ... in ascending order: first their
// maximum m (entries that are NaN never win), then a serial fp32 sum of
// exp(x - m); the 64 sums of a wave meet in an xor butterfly (masks 32 .. 1)
// and the 16 wave sums are added in wave order.  y = (x - m) - log(sum)
// (all -inf when no entry is above -inf).  y may alias x.
__global__ __launch_bounds__(1024) void k_log_softmax(const float* x, float* y, int V) {
  const long row = blockIdx.x;
  const float* xr = x + row * V;
  float* yr = y + row * V;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  __shared__ float red[16];
  // each loop takes U of the thread's elements per trip: the loads go out
  // together, then the elements are used in ascending order
  constexpr int U = 8;
  float m = -__builtin_inff();
  for (int i0 = t; i0 < V; i0 += 1024 * U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = xr[min(i0 + 1024 * u, V - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u) m = (i0 + 1024 * u < V && v[u] > m) ? v[u] : m;
  }
  for (int off = 32; off >= 1; off >>= 1) {
    const float o = __shfl_xor(m, off);
    m = o > m ? o : m;
  }
  if (lane == 0) red[w] = m;
  __syncthreads();
  m = red[0];
  for (int k = 1; k < 16; ++k) m = red[k] > m ? red[k] : m;
  __syncthreads();   // red is reused for the sums
  float a = 0.0f;
  for (int i0 = t; i0 < V; i0 += 1024 * U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = xr[min(i0 + 1024 * u, V - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i0 + 1024 * u < V) a = a + exp_fixed(v[u] - m);
  }
  for (int off = 32; off >= 1; off >>= 1) a = a + __shfl_xor(a, off);
  if (lane == 0) red[w] = a;
  __syncthreads();
  float sum = red[0];
  for (int k = 1; k < 16; ++k) sum = sum + red[k];
  const bool none = m == -__builtin_inff();
  const float ls = log_fixed(sum);
  for (int i0 = t; i0 < V; i0 += 1024 * U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = xr[min(i0 + 1024 * u, V - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i0 + 1024 * u < V) yr[i0 + 1024 * u] = none ? -__builtin_inff() : (v[u] - m) - ls;
  }
}

__device__ __forceinline__ void argbest(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

// One 1024-thread workgroup per row; four independent candidates per
// thread over float4 loads, then a tree.  The (largest value, lowest index)
// pair is the same in any combination order.
__global__ __launch_bounds__(1024) void k_argmax(const float* __restrict__ x,
                                                 int32_t* __restrict__ idx, int V) {
  const long row = blockIdx.x;
  const float* xr = x + row * V;
  float bv[4];
  int bi_[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) { bv[j] = -__builtin_inff(); bi_[j] = 0x7fffffff; }
  const bool vec = ((V & 3) == 0) && ((reinterpret_cast<uintptr_t>(xr) & 15) == 0);
  if (vec) {
    const float4* x4 = reinterpret_cast<const float4*>(xr);
    const int n4 = V >> 2;
    for (int i = threadIdx.x; i < n4; i += 1024) {
      const float4 t = x4[i];
      argbest(bv[0], bi_[0], t.x, 4 * i);
      argbest(bv[1], bi_[1], t.y, 4 * i + 1);
      argbest(bv[2], bi_[2], t.z, 4 * i + 2);
      argbest(bv[3], bi_[3], t.w, 4 * i + 3);
    }
  } else {
    for (int i = threadIdx.x; i < V; i += 1024) argbest(bv[i & 3], bi_[i & 3], xr[i], i);
  }
#pragma unroll
  for (int j = 1; j < 4; ++j) argbest(bv[0], bi_[0], bv[j], bi_[j]);
  float v = bv[0];
  int ix = bi_[0];
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(v, off);
    const int oi = __shfl_xor(ix, off);
    argbest(v, ix, ov, oi);
  }
  __shared__ float sv[16];
  __shared__ int si[16];
  if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = v; si[threadIdx.x >> 6] = ix; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 16; ++w) argbest(v, ix, sv[w], si[w]);
    idx[row] = ix == 0x7fffffff ? 0 : ix;
  }
}

static unsigned grid_for(long work, long per_block, unsigned cap) {
  long g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  return (unsigned)(g > cap ? cap : g);
}

}  // namespace bi

using namespace bi;

extern "C" bi_status bi_embed(const void* table, const int32_t* ids, void* out, int M, int d,
                              int dtype, bi_stream stream) {
  BI_REQUIRE(M >= 0 && d >= 8 && d % 8 == 0, BI_ERR_INVALID,
             "bi_embed: need M >= 0 and d a positive multiple of 8 (M=%d d=%d)", M, d);
  BI_REQUIRE(dtype == BI_F32 || dtype == BI_BF16, BI_ERR_UNSUPPORTED, "bi_embed: dtype %d", dtype);
  if (M == 0) return BI_OK;
  BI_REQUIRE(table && ids && out && aligned16(table) && aligned16(out), BI_ERR_INVALID,
             "bi_embed: null or misaligned pointer");
  BI_REQUIRE(M <= 65535, BI_ERR_INVALID, "bi_embed: M=%d too large", M);
  const dim3 grid(grid_for(d / 8, 256, 64), M);
  if (dtype == BI_BF16) hipLaunchKernelGGL(k_embed<1>, grid, dim3(256), 0, as_stream(stream), table, ids, out, d);
  else hipLaunchKernelGGL(k_embed<0>, grid, dim3(256), 0, as_stream(stream), table, ids, out, d);
  return launched("bi_embed");
}

extern "C" bi_status bi_rope_kv_append(const void* qkv, int M, int h, int h_kv, int d_h,
                                       const int32_t* pos, const float* cos_t,
                                       const float* sin_t, const int32_t* slot_mapping,
                                       int page_size, void* q_out, void* k_pool, void* v_pool,
                                       int dtype, bi_stream stream) {
  BI_REQUIRE(M >= 0 && h >= 1 && h_kv >= 1 && d_h >= 2 && d_h % 2 == 0 && page_size >= 1,
             BI_ERR_INVALID, "bi_rope_kv_append: bad sizes");
  BI_REQUIRE(dtype == BI_F32 || dtype == BI_BF16, BI_ERR_UNSUPPORTED,
             "bi_rope_kv_append: dtype %d", dtype);
  BI_REQUIRE((cos_t == nullptr) == (sin_t == nullptr), BI_ERR_INVALID,
             "bi_rope_kv_append: cos_t and sin_t must both be given or both be NULL");
  if (M == 0) return BI_OK;
  BI_REQUIRE(qkv && slot_mapping && q_out && k_pool && v_pool && (pos || !cos_t),
             BI_ERR_INVALID, "bi_rope_kv_append: null pointer");
  const long work = (long)M * (h + 2 * h_kv) * (d_h / 2);
  BI_REQUIRE(work < (1L << 40), BI_ERR_INVALID, "bi_rope_kv_append: too large");
  const unsigned grid = (unsigned)((work + 255) / 256);
  if (dtype == BI_BF16)
    hipLaunchKernelGGL(k_rope_kv_append<1>, dim3(grid), dim3(256), 0, as_stream(stream), qkv, M,
                       h, h_kv, d_h, pos, cos_t, sin_t, slot_mapping, page_size, q_out, k_pool,
                       v_pool);
  else
    hipLaunchKernelGGL(k_rope_kv_append<0>, dim3(grid), dim3(256), 0, as_stream(stream), qkv, M,
                       h, h_kv, d_h, pos, cos_t, sin_t, slot_mapping, page_size, q_out, k_pool,
                       v_pool);
  return launched("bi_rope_kv_append");
}

extern "C" bi_status bi_add(const void* a, const void* b, void* y, long n, int dtype,
                            bi_stream stream) {
  BI_REQUIRE(n >= 0, BI_ERR_INVALID, "bi_add: n=%ld", n);
  BI_REQUIRE(dtype == BI_F32 || dtype == BI_BF16, BI_ERR_UNSUPPORTED, "bi_add: dtype %d", dtype);
  if (n == 0) return BI_OK;
  BI_REQUIRE(a && b && y && aligned16(a) && aligned16(b) && aligned16(y), BI_ERR_INVALID,
             "bi_add: null or misaligned pointer");
  const unsigned grid = grid_for((n + 7) / 8, 256, 4096);
  if (dtype == BI_BF16) hipLaunchKernelGGL(k_add<1>, dim3(grid), dim3(256), 0, as_stream(stream), a, b, y, n);
  else hipLaunchKernelGGL(k_add<0>, dim3(grid), dim3(256), 0, as_stream(stream), a, b, y, n);
  return launched("bi_add");
}

extern "C" bi_status bi_silu_mul(const void* gu, void* y, int M, int F, int dtype,
                                 bi_stream stream) {
  BI_REQUIRE(M >= 0 && F >= 8 && F % 8 == 0, BI_ERR_INVALID,
             "bi_silu_mul: need F a positive multiple of 8 (F=%d)", F);
  BI_REQUIRE(dtype == BI_F32 || dtype == BI_BF16, BI_ERR_UNSUPPORTED, "bi_silu_mul: dtype %d",
             dtype);
  if (M == 0) return BI_OK;
  BI_REQUIRE(gu && y && aligned16(gu) && aligned16(y), BI_ERR_INVALID,
             "bi_silu_mul: null or misaligned pointer");
  BI_REQUIRE(M <= 65535, BI_ERR_INVALID, "bi_silu_mul: M=%d too large", M);
  const dim3 grid(grid_for(F / 8, 256, 64), M);
  if (dtype == BI_BF16) hipLaunchKernelGGL(k_silu_mul<1>, grid, dim3(256), 0, as_stream(stream), gu, y, F);
  else hipLaunchKernelGGL(k_silu_mul<0>, grid, dim3(256), 0, as_stream(stream), gu, y, F);
  return launched("bi_silu_mul");
}

// ---- seeded sampling ------------------------------------------------------
// MurmurHash3_x86_32 (Appleby's public-domain definition) of the 8-byte key
// (pos, col) as two little-endian 32-bit words, under a 32-bit seed.
__device__ __forceinline__ uint32_t rotl32(uint32_t x, int r) { return (x << r) | (x >> (32 - r)); }
__device__ __forceinline__ uint32_t murmur3_pos_col(uint32_t seed, uint32_t pos, uint32_t col) {
  uint32_t h = seed;
  uint32_t k = pos * 0xcc9e2d51u;
  k = rotl32(k, 15) * 0x1b873593u;
  h = rotl32(h ^ k, 13) * 5u + 0xe6546b64u;
  k = col * 0xcc9e2d51u;
  k = rotl32(k, 15) * 0x1b873593u;
  h = rotl32(h ^ k, 13) * 5u + 0xe6546b64u;
  h ^= 8u;
  h ^= h >> 16;
  h *= 0x85ebca6bu;
  h ^= h >> 13;
  h *= 0xc2b2ae35u;
  h ^= h >> 16;
  return h;
}

// Binary64 log fixed for the sampler, the binary32 log's method carried to
// double: x = 2^e m, m in [sqrt(1/2), sqrt(2)], log m = 2 atanh(s) by its odd
// series to s^23 (first omitted term below 2^-60 relative), then e ln 2 with
// ln 2 split into a head whose last 21 mantissa bits are zero (e * head is
// exact) and the binary64 tail.  Positive normal x only.
__device__ __forceinline__ double log_fixed64(double x) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(x);
  int e = (int)((b >> 52) & 0x7ffull) - 1023;
  double m = __longlong_as_double((long long)((b & 0xfffffffffffffull) | 0x3ff0000000000000ull));
  const bool big = m > 1.4142135623730951;
  m = big ? 0.5 * m : m;
  e = big ? e + 1 : e;
  const double s = (m - 1.0) / (m + 1.0);
  const double z = s * s;
  double q = 1.0 / 23.0;
  q = __builtin_fma(q, z, 1.0 / 21.0);
  q = __builtin_fma(q, z, 1.0 / 19.0);
  q = __builtin_fma(q, z, 1.0 / 17.0);
  q = __builtin_fma(q, z, 1.0 / 15.0);
  q = __builtin_fma(q, z, 1.0 / 13.0);
  q = __builtin_fma(q, z, 1.0 / 11.0);
  q = __builtin_fma(q, z, 1.0 / 9.0);
  q = __builtin_fma(q, z, 1.0 / 7.0);
  q = __builtin_fma(q, z, 1.0 / 5.0);
  q = __builtin_fma(q, z, 1.0 / 3.0);
  q = __builtin_fma(q, z, 1.0);
  const double lm = (s + s) * q;
  const double fe = (double)e;
  return __builtin_fma(fe, 6.93147180369123816490e-01, __builtin_fma(fe, 1.90821492927058770002e-10, lm));
}

__device__ __forceinline__ void argbest64(double& v, int& i, double v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

// Gumbel-max sampling per row: token = argmax_j (x_j * (1 / T) + g_j) in
// binary64, g_j = -log(-log(u_j)), u_j = (h_j + 1/2) 2^-32 with h_j the hash
// of (pos, j) under the row's seed; lowest index on ties; T <= 0: argmax of x.
// A row's draw depends on its own logits, seed and position only.
__global__ __launch_bounds__(1024) void k_sample_gumbel(const float* __restrict__ x,
                                                        const uint32_t* __restrict__ seed,
                                                        const int32_t* __restrict__ pos,
                                                        const float* __restrict__ temp,
                                                        int32_t* __restrict__ out, int V) {
  const long row = blockIdx.x;
  const float* xr = x + row * V;
  const float T = temp[row];
  const bool noise = T > 0.0f;
  const double invT = noise ? 1.0 / (double)T : 1.0;
  const uint32_t sd = seed[row], ps = (uint32_t)pos[row];
  double bv = -__builtin_inf();
  int bix = 0x7fffffff;
  for (int j = threadIdx.x; j < V; j += 1024) {
    double sc = (double)xr[j] * invT;
    if (noise) {
      const double u = ((double)murmur3_pos_col(sd, ps, (uint32_t)j) + 0.5) * 0x1p-32;
      sc = sc + -log_fixed64(-log_fixed64(u));
    }
    argbest64(bv, bix, sc, j);
  }
  for (int off = 32; off >= 1; off >>= 1) {
    const double ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bix, off);
    argbest64(bv, bix, ov, oi);
  }
  __shared__ double sv[16];
  __shared__ int si[16];
  if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = bv; si[threadIdx.x >> 6] = bix; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 16; ++w) argbest64(bv, bix, sv[w], si[w]);
    out[row] = bix == 0x7fffffff ? 0 : bix;
  }
}

extern "C" bi_status bi_sample(const float* x, const uint32_t* seed, const int32_t* pos,
                               const float* temperature, int32_t* out, int M, int V,
                               bi_stream stream) {
  BI_REQUIRE(M >= 0 && V >= 1, BI_ERR_INVALID, "bi_sample: bad sizes M=%d V=%d", M, V);
  if (M == 0) return BI_OK;
  BI_REQUIRE(x && seed && pos && temperature && out, BI_ERR_INVALID, "bi_sample: null pointer");
  hipLaunchKernelGGL(k_sample_gumbel, dim3(M), dim3(1024), 0, as_stream(stream), x, seed, pos,
                     temperature, out, V);
  return launched("bi_sample");
}

extern "C" bi_status bi_log_softmax(const float* x, float* y, int M, int V, bi_stream stream) {
  BI_REQUIRE(M >= 0 && V >= 1, BI_ERR_INVALID, "bi_log_softmax: bad sizes M=%d V=%d", M, V);
  if (M == 0) return BI_OK;
  BI_REQUIRE(x && y, BI_ERR_INVALID, "bi_log_softmax: null pointer");
  BI_REQUIRE(y == x || y + (long)M * V <= x || x + (long)M * V <= y, BI_ERR_INVALID,
             "bi_log_softmax: y must be x or not overlap it");
  hipLaunchKernelGGL(k_log_softmax, dim3(M), dim3(1024), 0, as_stream(stream), x, y, V);
  return launched("bi_log_softmax");
}

extern "C" bi_status bi_argmax(const float* x, int32_t* idx, int M, int V, bi_stream stream) {
  BI_REQUIRE(M >= 0 && V >= 1, BI_ERR_INVALID, "bi_argmax: bad sizes M=%d V=%d", M, V);
  if (M == 0) return BI_OK;
  BI_REQUIRE(x && idx, BI_ERR_INVALID, "bi_argmax: null pointer");
  hipLaunchKernelGGL(k_argmax, dim3(M), dim3(1024), 0, as_stream(stream), x, idx, V);
  return launched("bi_argmax");
}
