// Device helpers shared by the kernels of libbi.so (gfx950 only).
//
// Numeric contract of the whole library: IEEE binary32 arithmetic with
// round-to-nearest-even, fma only where __builtin_fmaf is written (the
// library is built with -ffp-contract=off and without fast-math), division
// and sqrt correctly rounded (HIP's default lowering), fp32 denormals kept.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bi {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---- bfloat16 <-> binary32 ---------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// binary32 -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u)
    return (u & 0x007fffffu) ? ((u | 0x00400000u) >> 16) : (u >> 16);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// ---- element access by dtype (0 = f32, 1 = bf16) -------------------------
template <int DT> struct Elem;
template <> struct Elem<0> {
  typedef float T;
  static constexpr int bytes = 4;
  __device__ static __forceinline__ float ld(const void* p, long i) {
    return static_cast<const float*>(p)[i];
  }
  __device__ static __forceinline__ void st(void* p, long i, float v) {
    static_cast<float*>(p)[i] = v;
  }
};
template <> struct Elem<1> {
  typedef uint16_t T;
  static constexpr int bytes = 2;
  __device__ static __forceinline__ float ld(const void* p, long i) {
    return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
  }
  __device__ static __forceinline__ void st(void* p, long i, float v) {
    static_cast<uint16_t*>(p)[i] = (uint16_t)f32_to_bf16_bits(v);
  }
};

// Load 8 consecutive elements starting at element index i (16-byte aligned
// for bf16, 32-byte for f32) as floats.
template <int DT> __device__ __forceinline__ void load8(const void* p, long i, float* o);
template <> __device__ __forceinline__ void load8<1>(const void* p, long i, float* o) {
  uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + i);
  o[0] = bf16_lo(w.x); o[1] = bf16_hi(w.x); o[2] = bf16_lo(w.y); o[3] = bf16_hi(w.y);
  o[4] = bf16_lo(w.z); o[5] = bf16_hi(w.z); o[6] = bf16_lo(w.w); o[7] = bf16_hi(w.w);
}
template <> __device__ __forceinline__ void load8<0>(const void* p, long i, float* o) {
  const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
  float4 a = q[0], b = q[1];
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
template <int DT> __device__ __forceinline__ void store8(void* p, long i, const float* v);
template <> __device__ __forceinline__ void store8<1>(void* p, long i, const float* v) {
  uint4 w;
  w.x = pack_bf16x2(v[0], v[1]); w.y = pack_bf16x2(v[2], v[3]);
  w.z = pack_bf16x2(v[4], v[5]); w.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p) + i) = w;
}
template <> __device__ __forceinline__ void store8<0>(void* p, long i, const float* v) {
  float4* q = reinterpret_cast<float4*>(static_cast<float*>(p) + i);
  q[0] = make_float4(v[0], v[1], v[2], v[3]);
  q[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// K cache page layout.  A (page, kv head) block of K holds page_size tokens
// of d_h elements as 16-byte units stored unit-major: unit u (elements
// 16/es * u .. 16/es * u + 16/es - 1) of token t sits at byte
// (u * page_size + t) * 16 of the block.  One matrix-core operand of K (16
// tokens x 32 bf16 dims: units 4s .. 4s + 3 of each token) is then 1 KiB of
// contiguous memory, read in whole 128-byte lines.  V keeps token-major rows.
// Element offset, within its block, of element e of token t:
__device__ __forceinline__ long k_block_elem(int t, int e, int page_size, int es) {
  const int per = 16 / es;
  return ((long)(e / per) * page_size + t) * per + e % per;
}

// ---- the library's exp ----------------------------------------------------
// One fixed binary32 exp for softmax and SiLU, so a result never depends on
// which hardware approximation a compiler picks: Cody & Waite range
// reduction ("Software Manual for the Elementary Functions", 1980) with
// ln 2 split into a 15-bit head and an fp32 tail, then the degree-7 Taylor
// polynomial of e^r in Horner form with fma, then scaling by 2^n in two
// exact-power steps.  Below -104 the result is +0, above 88.75 +inf.
__device__ __forceinline__ float exp_fixed(float x) {
  // branch-free: the polynomial runs on x clamped into range, the special
  // cases are selected at the end (same values as testing them first)
  const float xc = __builtin_fminf(__builtin_fmaxf(x, -104.0f), 88.75f);
  const float n = __builtin_rintf(xc * 1.44269502162933349609375f);
  float r = __builtin_fmaf(-n, 0.693145751953125f, xc);
  r = __builtin_fmaf(-n, 1.428606765330187045037746429443359375e-06f, r);
  float p = 1.0f / 5040.0f;
  p = __builtin_fmaf(p, r, 1.0f / 720.0f);
  p = __builtin_fmaf(p, r, 1.0f / 120.0f);
  p = __builtin_fmaf(p, r, 1.0f / 24.0f);
  p = __builtin_fmaf(p, r, 1.0f / 6.0f);
  p = __builtin_fmaf(p, r, 0.5f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  const int ni = (int)n;
  const int n1 = ni / 2;
  const int n2 = ni - n1;
  p = p * __uint_as_float((uint32_t)(n1 + 127) << 23);
  p = p * __uint_as_float((uint32_t)(n2 + 127) << 23);
  p = x < -104.0f ? 0.0f : p;
  p = x > 88.75f ? __builtin_inff() : p;
  return x != x ? x : p;
}

// ---- the library's log ----------------------------------------------------
// One fixed binary32 log for the log-softmax, for the same reason: x = 2^e m
// with m in [sqrt(1/2), sqrt(2)] (exponent and mantissa taken from the bits),
// log m = 2 atanh(s) with s = (m - 1) / (m + 1), |s| <= 0.172, by the odd
// series 2 s (1 + z/3 + z^2/5 + ... + z^6/13), z = s^2, in Horner form with
// fma (the first omitted term is below 2^-39 relative), then e ln 2 added with
// ln 2 split into the exp's head and tail.  For positive normal x; +inf and
// NaN pass through.
__device__ __forceinline__ float log_fixed(float x) {
  const uint32_t b = __float_as_uint(x);
  int e = (int)((b >> 23) & 0xff) - 127;
  float m = __uint_as_float((b & 0x7fffffu) | 0x3f800000u);        // [1, 2)
  const bool big = m > 1.41421353816986083984375f;                  // fp32(sqrt 2)
  m = big ? 0.5f * m : m;
  e = big ? e + 1 : e;
  const float s = (m - 1.0f) / (m + 1.0f);
  const float z = s * s;
  float q = 1.0f / 13.0f;
  q = __builtin_fmaf(q, z, 1.0f / 11.0f);
  q = __builtin_fmaf(q, z, 1.0f / 9.0f);
  q = __builtin_fmaf(q, z, 1.0f / 7.0f);
  q = __builtin_fmaf(q, z, 1.0f / 5.0f);
  q = __builtin_fmaf(q, z, 1.0f / 3.0f);
  q = __builtin_fmaf(q, z, 1.0f);
  const float lm = (s + s) * q;
  const float fe = (float)e;
  const float r = __builtin_fmaf(fe, 0.693145751953125f,
                                 __builtin_fmaf(fe, 1.428606765330187045037746429443359375e-06f, lm));
  return (x != x || x == __builtin_inff()) ? x : r;
}

// Maximum over the 16 lanes of each row of the wave (DPP row rotations;
// max is exact, so the order of the steps does not matter).
__device__ __forceinline__ float row16_max(float v) {
  v = __builtin_fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(
                             0, __float_as_int(v), 0x128, 0xf, 0xf, false)));  // row_ror:8
  v = __builtin_fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(
                             0, __float_as_int(v), 0x124, 0xf, 0xf, false)));  // row_ror:4
  v = __builtin_fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(
                             0, __float_as_int(v), 0x122, 0xf, 0xf, false)));  // row_ror:2
  v = __builtin_fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(
                             0, __float_as_int(v), 0x121, 0xf, 0xf, false)));  // row_ror:1
  return v;
}

// ---- direct global -> LDS copies -----------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;

// One wave copies 64 x 16 bytes: lane l reads 16 bytes at `src` (its own
// address) and the hardware writes them to LDS at lds_base + 16 * l.
// lds_base must be wave-uniform.
__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)lds_base, 16, 0, 0);
}

// The same copy marked non-temporal (cache policy NT), for data that is read
// once (the weights of a skinny GEMM, KV pages): the L2 then keeps its room for
// the operands that other workgroups re-read.
__device__ __forceinline__ void dma16_nt(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)lds_base, 16, 0, 2);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// ---- explicit LDS reads --------------------------------------------------
// The compiler cannot tell LDS reads apart from LDS written by in-flight
// direct copies and would wait for every outstanding copy before each read,
// which serialises a copy ring.  Reads of ring slots therefore go through
// these helpers: one asm statement issues a batch of ds_read_b128 and waits
// for them (s_waitcnt lgkmcnt(0)) before it ends, so the compiler never sees
// a register whose load is still in flight.  Ring-slot reuse is ordered by
// explicit vmcnt waits and s_barrier.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// a[i] = LDS[ba + 1024 i], b[i] = LDS[bb + 1024 i], i = 0..7 (16 bytes each).
__device__ __forceinline__ void lds_read_8x2_stride1k(u32x4_t (&a)[8], u32x4_t (&b)[8],
                                                      uint32_t ba, uint32_t bb) {
  asm volatile(
      "ds_read_b128 %0, %16\n\tds_read_b128 %1, %16 offset:1024\n\t"
      "ds_read_b128 %2, %16 offset:2048\n\tds_read_b128 %3, %16 offset:3072\n\t"
      "ds_read_b128 %4, %16 offset:4096\n\tds_read_b128 %5, %16 offset:5120\n\t"
      "ds_read_b128 %6, %16 offset:6144\n\tds_read_b128 %7, %16 offset:7168\n\t"
      "ds_read_b128 %8, %17\n\tds_read_b128 %9, %17 offset:1024\n\t"
      "ds_read_b128 %10, %17 offset:2048\n\tds_read_b128 %11, %17 offset:3072\n\t"
      "ds_read_b128 %12, %17 offset:4096\n\tds_read_b128 %13, %17 offset:5120\n\t"
      "ds_read_b128 %14, %17 offset:6144\n\tds_read_b128 %15, %17 offset:7168\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5]),
        "=&v"(a[6]), "=&v"(a[7]), "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]), "=&v"(b[3]),
        "=&v"(b[4]), "=&v"(b[5]), "=&v"(b[6]), "=&v"(b[7])
      : "v"(ba), "v"(bb)
      : "memory");
}

// a[i] = LDS[ba + 1024 i], i = 0..7.
__device__ __forceinline__ void lds_read_8_stride1k(u32x4_t (&a)[8], uint32_t ba) {
  asm volatile(
      "ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:1024\n\t"
      "ds_read_b128 %2, %8 offset:2048\n\tds_read_b128 %3, %8 offset:3072\n\t"
      "ds_read_b128 %4, %8 offset:4096\n\tds_read_b128 %5, %8 offset:5120\n\t"
      "ds_read_b128 %6, %8 offset:6144\n\tds_read_b128 %7, %8 offset:7168\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5]),
        "=&v"(a[6]), "=&v"(a[7])
      : "v"(ba)
      : "memory");
}

// a[i] = LDS[ba + 2048 i], i = 0..7.
__device__ __forceinline__ void lds_read_8_stride2k(u32x4_t (&a)[8], uint32_t ba) {
  asm volatile(
      "ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:2048\n\t"
      "ds_read_b128 %2, %8 offset:4096\n\tds_read_b128 %3, %8 offset:6144\n\t"
      "ds_read_b128 %4, %8 offset:8192\n\tds_read_b128 %5, %8 offset:10240\n\t"
      "ds_read_b128 %6, %8 offset:12288\n\tds_read_b128 %7, %8 offset:14336\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5]),
        "=&v"(a[6]), "=&v"(a[7])
      : "v"(ba)
      : "memory");
}

// a[i] = LDS[ba + 2048 i], i = 0..3.
__device__ __forceinline__ void lds_read_4_stride2k(u32x4_t (&a)[4], uint32_t ba) {
  asm volatile(
      "ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:2048\n\t"
      "ds_read_b128 %2, %4 offset:4096\n\tds_read_b128 %3, %4 offset:6144\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
      : "v"(ba)
      : "memory");
}

// a[i] = LDS[ba + 1024 i], i = 0..3.
__device__ __forceinline__ void lds_read_4_stride1k(u32x4_t (&a)[4], uint32_t ba) {
  asm volatile(
      "ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:1024\n\t"
      "ds_read_b128 %2, %4 offset:2048\n\tds_read_b128 %3, %4 offset:3072\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
      : "v"(ba)
      : "memory");
}

// a[i] = LDS[ba + 2048 i], b[i] = LDS[bb + 2048 i], i = 0..3.
__device__ __forceinline__ void lds_read_4x2_stride2k(u32x4_t (&a)[4], u32x4_t (&b)[4],
                                                      uint32_t ba, uint32_t bb) {
  asm volatile(
      "ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:2048\n\t"
      "ds_read_b128 %2, %8 offset:4096\n\tds_read_b128 %3, %8 offset:6144\n\t"
      "ds_read_b128 %4, %9\n\tds_read_b128 %5, %9 offset:2048\n\t"
      "ds_read_b128 %6, %9 offset:4096\n\tds_read_b128 %7, %9 offset:6144\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(b[0]), "=&v"(b[1]),
        "=&v"(b[2]), "=&v"(b[3])
      : "v"(ba), "v"(bb)
      : "memory");
}

// ---- matrix cores -----------------------------------------------------------
// v_mfma_f32_16x16x32_bf16.  Operand layout: lane l holds 8 bf16 of A row
// (l & 15) and of B column (l & 15), both for k = 8 (l >> 4) .. 8 (l >> 4) + 7;
// the 16 x 16 fp32 result gives lane l column (l & 15), rows 4 (l >> 4) + j,
// j = 0..3.  A result row depends only on its own A row and B.
__device__ __forceinline__ f32x4_t mfma16(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i = 4e + c gives the address of 4 consecutive 16-bit elements; lane
// j = 4c + d receives element d of the segments of lanes c, c + 4, c + 8 and
// c + 12, in that order (returned as two packed dwords).
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(3))) char lds_char_t;
__device__ __forceinline__ uint2 lds_read_tr16(const void* lds_base, uint32_t byte_off) {
  const v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16_t*)((lds_char_t*)lds_base + byte_off));
  return __builtin_bit_cast(uint2, r);
}

// Wait until at most n vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt encoding; lgkm and exp counters left alone).
#define BI_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | ((((n) >> 4) & 3) << 14) | (7 << 4) | (15 << 8))

}  // namespace bi
