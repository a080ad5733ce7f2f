// Split-KV attention over a paged KV cache with request-derived split points.
//
// "Lockstep", "The fix": attention split points come from the request, not
// the batch.  "Batch invariance and reproducible inference", "1 . Split-K
// and segmented attention reductions": the split count is ceil(seq_len /
// split tile) whatever else is in the batch, and "From batch size to
// reduction tree": the fp32 partials of the splits are added by a merge.
//
// Chunk c of a request covers absolute positions [c*C, min((c+1)*C, s)).
// One workgroup of C/64 waves computes one (chunk, kv head) partial for the
// R query heads of that kv head:
//   QK  lane-per-key: lane u of wave w owns key 64w+u; its K row sits in LDS
//       (copied there by direct global->LDS copies, 16-byte columns XOR-
//       swizzled by the key index so lanes reading the same column hit
//       different banks); S = fl(dot) * scale with the dot one fma chain
//       over d ascending, q broadcast from LDS as fp32.
//   max over the chunk (exact, any order), +0 for -0; p = exp_fixed(S - m).
//   PV  lane-per-dim: lane l owns dims [DPL*l, DPL*l+DPL) and keeps the V of
//       its wave's 64 keys in registers; within the wave (= a block of 64
//       keys) l and acc are serial sums over keys ascending (acc by fma).
//   blocks are added in wave order: ((B0 + B1) + B2) + B3.
// That is the fp32 (VALU) path.  bf16 KV runs on matrix cores (see
// "bf16 KV: the chunk on matrix cores" below), with the same structure:
// fixed chunks at absolute positions, one partial per chunk, a serial merge.
// Prefill evaluates each query row with the decode chunk's per-element
// arithmetic and merges the chunks on the fly with the merge kernel's
// formula, so prefill row t equals a decode of kv_len = t + 1 bit for bit.
#include <cmath>
#include <mutex>

#include "api.h"
#include "common.h"

namespace bi {

// Softmax weight on the matrix-core paths: p = exp(x) with x = s - m <= 0,
// or -inf for a masked key.  For every such x the value is exp_fixed's (NaN
// stays NaN): the overflow case cannot arise; exp_fixed's two exact-power
// steps 2^(n/2) 2^(n - n/2) are one ldexp -- the exact product p 2^n is
// rounded once either way (the first step is exact, its result being at
// least 2^-76); and below -104 no select is needed, since at the clamp
// (n = -150, p(r) = 0.97...) the product is under half the least subnormal
// and rounds to +0.
__device__ __forceinline__ float exp_p(float x) {
  const float xc = __builtin_fmaxf(x, -104.0f);
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
  p = __builtin_amdgcn_ldexpf(p, (int)n);
  return x != x ? x : p;
}

// Two softmax weights as packed bf16 (lo in bits 0..15): the hardware
// conversion, round to nearest even (the rule of f32_to_bf16_bits for every
// finite value).
__device__ __forceinline__ uint32_t p_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
  typedef float f32x2_v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_v{lo, hi}, bf16x2_v));
}

template <int DT, int DH>
struct AttnShape {
  static constexpr int ES = Elem<DT>::bytes;
  static constexpr int RB = DH * ES;          // bytes per K/V row
  static constexpr int SLOTS = RB / 16;       // 16-byte columns per row
  static constexpr int EPS = 16 / ES;         // elements per column
  static constexpr int SW = SLOTS < 16 ? SLOTS : 16;  // swizzle width
  static constexpr int KPI = 1024 / RB;       // keys per 1 KiB wave copy
  static constexpr int DPL = DH / 64;         // V elements per lane
  static constexpr int VW = (DPL * ES + 3) / 4;  // 32-bit registers per key for V
  static_assert(RB % 16 == 0 && 1024 % RB == 0, "row size");
};

// byte offset of (key u, column c) in the swizzled K block
template <int DT, int DH>
__device__ __forceinline__ int kswz(int u, int c) {
  typedef AttnShape<DT, DH> S;
  return u * S::RB + 16 * (c ^ (u & (S::SW - 1)));
}

// LDS layout of one attention workgroup
template <int DT, int DH, int R, int NW, bool KLDS = true>
struct AttnLds {
  static constexpr int KEYS = 64 * NW;
  static constexpr int K_BYTES = KLDS ? KEYS * AttnShape<DT, DH>::RB : 0;
  static constexpr int Q_OFF = K_BYTES;                        // fp32 q [R][DH]
  static constexpr int P_OFF = Q_OFF + R * DH * 4;             // fp32 p [KEYS][R]
  static constexpr int MX_OFF = P_OFF + KEYS * R * 4;          // fp32 [NW][R]
  static constexpr int CB_OFF = MX_OFF + NW * R * 4;           // fp32 [NW][R][DH+1]
  static constexpr int BYTES = CB_OFF + NW * R * (DH + 1) * 4;
};

// Per-thread result of a chunk: thread tid (< R*DH/DPL... see owner map)
// holds, for the (head, dim) pairs it owns after the block combine, the
// chunk's m, l and acc.  Owner map: pair index q = tid + 64*NW*k covers
// head q / (DH/DPL... ) -- implemented as: head = q / DH_LANES, lane-dims.
template <int R, int NW, int DPL>
struct ChunkOut {
  static constexpr int NT = 64 * NW;
  static constexpr int SLOTS_PER_HEAD = 64;            // DPL dims per slot
  static constexpr int ITEMS = (R * 64 + NT - 1) / NT; // (head, lane) items per thread
  float m[ITEMS], l[ITEMS], acc[ITEMS][DPL];
};

// Computes the partial of keys [j0, j0 + n) (1 <= n <= 64*NW) of kv head g
// for the R query heads whose q vectors are already in LDS (fp32).  The K
// block must be fully copied (this wave's part) before the call; vregs holds
// this lane's V dims for the wave's 64 keys.  All threads of the workgroup
// call it.  Result: item k of thread tid is (head, lane) = divmod(tid + NT*k,
// 64), lane owning dims [DPL*lane, DPL*lane + DPL).
// V element e of this lane's packed V registers for one key
template <int DT, int DH>
__device__ __forceinline__ float v_elem(const uint32_t* v, int e) {
  if (DT == 1) return (AttnShape<DT, DH>::DPL == 2 && e == 1) ? bf16_hi(v[0]) : bf16_lo(v[0]);
  return __uint_as_float(v[e]);
}

struct NoHook {
  __device__ __forceinline__ void operator()() const {}
};

// KSrc(c) returns this lane's 16-byte column c of its key's K row (from the
// LDS block, or from registers in the pipelined kernel).  after_qk runs once
// every K read of the chunk is done, after_pv once every V register is
// consumed: the pipelined kernel issues the next chunk's loads there.
// QG: q is read from global memory (bf16, qg = this kv head's first query
// head, wave-uniform) instead of the fp32 copy in LDS; same values.
template <int DT, int DH, int R, int NW, bool KLDS = true, bool FINAL_SYNC = true,
          bool QG = false, class KSrc, class H1 = NoHook, class H2 = NoHook>
__device__ __forceinline__ void chunk_partial_k(char* lds, int n, float scale, const KSrc& ksrc,
                                                const uint32_t (&vreg)[64][AttnShape<DT, DH>::VW],
                                                ChunkOut<R, NW, AttnShape<DT, DH>::DPL>& out,
                                                const H1& after_qk = H1(),
                                                const H2& after_pv = H2(),
                                                int q_off = AttnLds<DT, DH, R, NW, KLDS>::Q_OFF,
                                                const uint16_t* __restrict__ qg = nullptr) {
  static_assert(!QG || DT == 1, "global q path is for bf16");
  typedef AttnShape<DT, DH> S;
  typedef AttnLds<DT, DH, R, NW, KLDS> L;
  constexpr int DPL = S::DPL;
  constexpr int NT = 64 * NW;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int u = tid;  // this lane's key within the chunk
  const float* qs = reinterpret_cast<const float*>(lds + q_off);
  float* ps = reinterpret_cast<float*>(lds + L::P_OFF);
  float* mx = reinterpret_cast<float*>(lds + L::MX_OFF);
  float* cb = reinterpret_cast<float*>(lds + L::CB_OFF);

  // ---- QK, lane per key
  float sc[R];
#pragma unroll
  for (int i = 0; i < R; ++i) sc[i] = 0.0f;
  const bool valid = u < n;
  if (valid) {
#pragma unroll
    for (int c = 0; c < S::SLOTS; ++c) {
      const uint4 w = ksrc(c);
      float kv[S::EPS];
      if (DT == 1) {
        kv[0] = bf16_lo(w.x); kv[1] = bf16_hi(w.x); kv[2] = bf16_lo(w.y); kv[3] = bf16_hi(w.y);
        kv[4] = bf16_lo(w.z); kv[5] = bf16_hi(w.z); kv[6] = bf16_lo(w.w); kv[7] = bf16_hi(w.w);
      } else {
        kv[0] = __uint_as_float(w.x); kv[1] = __uint_as_float(w.y);
        kv[2] = __uint_as_float(w.z); kv[3] = __uint_as_float(w.w);
      }
#pragma unroll
      for (int i = 0; i < R; ++i) {
        float qv[S::EPS];
        if constexpr (QG) {
          // q straight from global memory at a wave-uniform address: scalar
          // loads into SGPRs (bf16 widened by shifts), no LDS traffic
          const uint4 w4 = *reinterpret_cast<const uint4*>(qg + i * DH + c * S::EPS);
          qv[0] = bf16_lo(w4.x); qv[1] = bf16_hi(w4.x); qv[2] = bf16_lo(w4.y);
          qv[3] = bf16_hi(w4.y); qv[4] = bf16_lo(w4.z); qv[5] = bf16_hi(w4.z);
          qv[6] = bf16_lo(w4.w); qv[7] = bf16_hi(w4.w);
        } else {
          const float4* q4p = reinterpret_cast<const float4*>(qs + i * DH + c * S::EPS);
#pragma unroll
          for (int e4 = 0; e4 < S::EPS / 4; ++e4) {
            const float4 q4 = q4p[e4];
            qv[4 * e4] = q4.x; qv[4 * e4 + 1] = q4.y; qv[4 * e4 + 2] = q4.z; qv[4 * e4 + 3] = q4.w;
          }
        }
#pragma unroll
        for (int e = 0; e < S::EPS; ++e) sc[i] = __builtin_fmaf(qv[e], kv[e], sc[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < R; ++i) sc[i] = sc[i] * scale;
  }
  after_qk();
  // ---- chunk max (exact in any order)
  float m[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    float v = valid ? sc[i] : -__builtin_inff();
    v = fmaxf(v, __shfl_xor(v, 32));
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 8));
    v = fmaxf(v, __shfl_xor(v, 4));
    v = fmaxf(v, __shfl_xor(v, 2));
    v = fmaxf(v, __shfl_xor(v, 1));
    m[i] = v;
  }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < R; ++i) mx[wave * R + i] = m[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < R; ++i) {
    float v = mx[i];
#pragma unroll
    for (int w = 1; w < NW; ++w) v = fmaxf(v, mx[w * R + i]);
    m[i] = v + 0.0f;
  }
  // ---- p = exp(S - m), published for the wave's PV loop
  if (valid) {
#pragma unroll
    for (int i = 0; i < R; ++i) ps[u * R + i] = exp_fixed(sc[i] - m[i]);
  }
  // the PV loop of a wave reads only its own keys' p: wave-local order suffices
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // ---- PV, lane per dim, serial over this wave's keys
  const int nk = min(64, n - 64 * wave);  // keys of this block (may be <= 0)
  float lsum[R], acc[R][DPL];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    lsum[i] = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[i][e] = 0.0f;
  }
#pragma unroll
  for (int k = 0; k < 64; ++k) {
    if (k < nk) {
      const float* pk = ps + (64 * wave + k) * R;
      float pv[R];
      if (R % 4 == 0) {
#pragma unroll
        for (int i4 = 0; i4 < R / 4; ++i4) {
          const float4 t = reinterpret_cast<const float4*>(pk)[i4];
          pv[4 * i4] = t.x; pv[4 * i4 + 1] = t.y; pv[4 * i4 + 2] = t.z; pv[4 * i4 + 3] = t.w;
        }
      } else {
#pragma unroll
        for (int i = 0; i < R; ++i) pv[i] = pk[i];
      }
#pragma unroll
      for (int i = 0; i < R; ++i) {
        lsum[i] = lsum[i] + pv[i];
#pragma unroll
        for (int e = 0; e < DPL; ++e)
          acc[i][e] = __builtin_fmaf(pv[i], v_elem<DT, DH>(vreg[k], e), acc[i][e]);
      }
    }
  }
  after_pv();
  // ---- publish block partials, combine blocks in wave order
  constexpr int CBS = DH + 1;  // floats per (wave, head)
  if (nk > 0) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      float* dst = cb + (wave * R + i) * CBS;
#pragma unroll
      for (int e = 0; e < DPL; ++e) dst[DPL * lane + e] = acc[i][e];
      if (lane == 0) dst[DH] = lsum[i];
    }
  }
  __syncthreads();
  const int nb = (n + 63) >> 6;
  typedef ChunkOut<R, NW, DPL> CO;
#pragma unroll
  for (int k = 0; k < CO::ITEMS; ++k) {
    const int item = tid + NT * k;
    if (item < R * 64) {
      const int hi = item >> 6, ln = item & 63;
      float l = cb[hi * CBS + DH];
      float a[DPL];
#pragma unroll
      for (int e = 0; e < DPL; ++e) a[e] = cb[hi * CBS + DPL * ln + e];
      for (int b = 1; b < nb; ++b) {
        const float* src = cb + (b * R + hi) * CBS;
        l = l + src[DH];
#pragma unroll
        for (int e = 0; e < DPL; ++e) a[e] = a[e] + src[DPL * ln + e];
      }
      out.m[k] = m[hi];
      out.l[k] = l;
#pragma unroll
      for (int e = 0; e < DPL; ++e) out.acc[k][e] = a[e];
    }
  }
  if (FINAL_SYNC) __syncthreads();  // LDS (p, block partials, K) may be reused by the caller
}

template <int DT, int DH, int R, int NW>
__device__ __forceinline__ void chunk_partial(char* lds, int n, float scale,
                                              const uint32_t (&vreg)[64][AttnShape<DT, DH>::VW],
                                              ChunkOut<R, NW, AttnShape<DT, DH>::DPL>& out) {
  const int u = threadIdx.x;
  auto kl = [&](int c) { return *reinterpret_cast<const uint4*>(lds + kswz<DT, DH>(u, c)); };
  chunk_partial_k<DT, DH, R, NW, true>(lds, n, scale, kl, vreg, out);
}

// Pages hold kPage tokens (the only page size the kernels are built for).
constexpr int kPage = 16;

// Stage this wave's 64 keys of the chunk (keys [j0, j0+n)) of kv head g:
// K rows into the swizzled LDS block by direct copies, and this lane's V
// dims into registers.  Keys >= n read key j0 instead (valid memory, never
// used).  j0 and the wave's first key are multiples of the page size, so
// each copy instruction (<= 16 keys) and each key's page are wave-uniform
// and come from scalar loads of the block table.
template <int DT, int DH, int NW>
__device__ __forceinline__ void stage_chunk(char* lds, const void* k_pool, const void* v_pool,
                                            const int32_t* bt, int j0, int n, int g, int h_kv,
                                            uint32_t (&vreg)[64][AttnShape<DT, DH>::VW]) {
  typedef AttnShape<DT, DH> S;
  static_assert(kPage % S::KPI == 0 && 64 % kPage == 0, "page geometry");
  constexpr int NP = 64 / kPage;                 // pages per wave
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wk0 = 64 * wave;                     // first key of this wave in the chunk
  const int nk = min(64, n - wk0);               // keys of this wave (may be <= 0)
  const long hstride = (long)kPage * S::RB;      // bytes per (page, head) block
  const long pstride = hstride * h_kv;           // bytes per page
  const char* kp = static_cast<const char*>(k_pool) + g * hstride;
  const char* vp = static_cast<const char*>(v_pool) + g * hstride;
  const int pfall = bt[j0 / kPage];              // stands in for pages past the end
  int page[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) page[p] = (p * kPage < nk) ? bt[(j0 + wk0) / kPage + p] : pfall;
  // K: one 1 KiB copy covers KPI consecutive keys of one page (unit c of
  // token `slot` sits at (c * kPage + slot) * 16 in the unit-major block)
#pragma unroll
  for (int inst = 0; inst < 64 / S::KPI; ++inst) {
    const int k0 = inst * S::KPI;
    const int kk = k0 + lane / S::SLOTS;         // key of this lane within the wave
    const int slot = (k0 < nk) ? (kk % kPage) : 0;
    const int c = (lane % S::SLOTS) ^ ((wk0 + kk) & (S::SW - 1));
    dma16(kp + page[k0 / kPage] * pstride + (c * kPage + slot) * 16, lds + (wk0 + k0) * S::RB);
  }
  // V: lane-per-dim, one row per key of this wave, kept packed
  const long lane_off = (long)lane * S::DPL * S::ES;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const char* pb = vp + page[p] * pstride + lane_off;
#pragma unroll
    for (int s = 0; s < kPage; ++s) {
      const int k = p * kPage + s;
      const char* src = pb + ((k < nk) ? s : 0) * S::RB;
      if (S::DPL * S::ES == 2) {
        vreg[k][0] = *reinterpret_cast<const uint16_t*>(src);
      } else {
#pragma unroll
        for (int e = 0; e < S::VW; ++e) vreg[k][e] = reinterpret_cast<const uint32_t*>(src)[e];
      }
    }
  }
}

// q vectors of the R heads of group g of one row -> LDS as fp32
template <int DT, int DH, int R, int NW>
__device__ __forceinline__ void stage_q(char* lds, const void* q, long qrow_elem) {
  typedef AttnLds<DT, DH, R, NW> L;
  float* qs = reinterpret_cast<float*>(lds + L::Q_OFF);
  for (int i = threadIdx.x; i < R * DH; i += 64 * NW) qs[i] = Elem<DT>::ld(q, qrow_elem + i);
}

// ---------------------------------------------------------------------------
// decode partials: grid (total_chunks, h_kv)
// ---------------------------------------------------------------------------
template <int DT, int DH, int R, int NW>
__global__ __launch_bounds__(64 * NW) void k_decode_partials(
    const void* __restrict__ q, const void* __restrict__ k_pool, const void* __restrict__ v_pool,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ kv_len,
    const int32_t* __restrict__ chunk_off, int B, int h, int h_kv, int page_size, int max_pages,
    float scale, float* __restrict__ part_ml, float* __restrict__ part_acc) {
  typedef AttnShape<DT, DH> S;
  typedef ChunkOut<R, NW, S::DPL> CO;
  constexpr int C = 64 * NW;
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int crow = blockIdx.x, g = blockIdx.y;
  // request owning this chunk row: largest r with chunk_off[r] <= crow
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (chunk_off[mid] <= crow) lo = mid; else hi = mid - 1;
  }
  const int r = lo;
  const int c = crow - chunk_off[r];
  const int j0 = c * C;
  const int n = min(C, kv_len[r] - j0);
  const int32_t* bt = block_table + (long)r * max_pages;

  uint32_t vreg[64][S::VW];
  stage_chunk<DT, DH, NW>(lds, k_pool, v_pool, bt, j0, n, g, h_kv, vreg);
  stage_q<DT, DH, R, NW>(lds, q, ((long)r * h + g * R) * DH);
  __syncthreads();
  CO out;
  chunk_partial<DT, DH, R, NW>(lds, n, scale, vreg, out);
#pragma unroll
  for (int k = 0; k < CO::ITEMS; ++k) {
    const int item = threadIdx.x + 64 * NW * k;
    if (item < R * 64) {
      const int hi2 = item >> 6, ln = item & 63;
      const long prow = (long)crow * h + g * R + hi2;
      if (ln == 0) {
        part_ml[2 * prow] = out.m[k];
        part_ml[2 * prow + 1] = out.l[k];
      }
#pragma unroll
      for (int e = 0; e < S::DPL; ++e) part_acc[prow * DH + S::DPL * ln + e] = out.acc[k][e];
    }
  }
}

// ---------------------------------------------------------------------------
// serial merge: one wave per (request, head); lane owns DH/64 dims
// ---------------------------------------------------------------------------
// REV (twin only): chunks combined from the last to the first.  The
// partials of request r start at row chunk_off[r] (chunk_off == nullptr:
// at row r * fixed_stride, with n_r from the twin's split policy).
__device__ __forceinline__ int free_splits(int s, int chunk2, int* len) {
  if (s <= 0) {
    *len = 0;
    return 0;
  }
  int n = max((s + 255) / 256, (s + chunk2 - 1) / chunk2);
  int l = (s + n - 1) / n;
  l = (l + 15) & ~15;
  *len = l;
  return (s + l - 1) / l;
}

template <int DH, int OUT_DT, bool REV = false>
__global__ __launch_bounds__(256) void k_merge(const float* __restrict__ part_ml,
                                               const float* __restrict__ part_acc,
                                               const int32_t* __restrict__ chunk_off, int B,
                                               int h, void* __restrict__ out,
                                               const int32_t* __restrict__ kv_len = nullptr,
                                               int chunk2 = 0, int stride = 0) {
  constexpr int DPL = DH / 64;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wid >= B * h) return;
  const int r = wid / h, hi = wid % h;
  int c0, n;
  if (chunk_off != nullptr) {
    c0 = chunk_off[r];
    n = chunk_off[r + 1] - c0;
  } else {
    int len;
    c0 = r * stride;
    n = min(free_splits(kv_len[r], chunk2, &len), stride);
  }
  const long o = ((long)r * h + hi) * DH + DPL * lane;
  if (n <= 0) {  // no keys: the output is defined as zero
#pragma unroll
    for (int e = 0; e < DPL; ++e) Elem<OUT_DT>::st(out, o + e, 0.f);
    return;
  }
  // partial row of the c-th chunk in merge order
  auto prow = [&](int c) { return (long)(REV ? c0 + n - 1 - c : c0 + c) * h + hi; };
  long row = prow(0);
  float M = part_ml[2 * row], L = part_ml[2 * row + 1];
  float A[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) A[e] = part_acc[row * DH + DPL * lane + e];
  // the merge is serial, but its loads are not: G chunks are loaded at a time
  // (indices clamped to the last chunk), then merged one by one in order
  constexpr int G = 8;
  for (int cg = 1; cg < n; cg += G) {
    float mc[G], lc[G], ac[G][DPL];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const long rw = prow(min(cg + i, n - 1));
      mc[i] = part_ml[2 * rw];
      lc[i] = part_ml[2 * rw + 1];
#pragma unroll
      for (int e = 0; e < DPL; ++e) ac[i][e] = part_acc[rw * DH + DPL * lane + e];
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if (cg + i < n) {
        const float Mn = M > mc[i] ? M : mc[i];
        const float a = exp_fixed(M - Mn), b = exp_fixed(mc[i] - Mn);
        L = __builtin_fmaf(lc[i], b, L * a);
#pragma unroll
        for (int e = 0; e < DPL; ++e) A[e] = __builtin_fmaf(ac[i][e], b, A[e] * a);
        M = Mn;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e) Elem<OUT_DT>::st(out, o + e, A[e] / L);
}

// ---------------------------------------------------------------------------
// decode twin: split length per request from the occupancy policy
// (free_splits: at least ceil(s/256) splits, more when the batch leaves cores
// idle), so the split points of a request move with the batch.  Same chunk
// arithmetic as the invariant kernel; partial rows at r * stride + c.
// ---------------------------------------------------------------------------
template <int DT, int DH, int R>
__global__ __launch_bounds__(256) void k_decode_free(
    const void* __restrict__ q, const void* __restrict__ k_pool, const void* __restrict__ v_pool,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ kv_len, int h, int h_kv,
    int max_pages, float scale, int chunk2, int stride, float* __restrict__ part_ml,
    float* __restrict__ part_acc) {
  typedef AttnShape<DT, DH> S;
  typedef ChunkOut<R, 4, S::DPL> CO;
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int r = blockIdx.x / stride, c = blockIdx.x % stride, g = blockIdx.y;
  int len;
  const int s = kv_len[r];
  const int n_r = free_splits(s, chunk2, &len);
  if (c >= n_r) return;  // c < stride by the grid, so rows stay inside the workspace
  const int j0 = c * len;
  const int n = min(len, s - j0);
  const int32_t* bt = block_table + (long)r * max_pages;
  uint32_t vreg[64][S::VW];
  stage_chunk<DT, DH, 4>(lds, k_pool, v_pool, bt, j0, n, g, h_kv, vreg);
  stage_q<DT, DH, R, 4>(lds, q, ((long)r * h + g * R) * DH);
  __syncthreads();
  CO out;
  chunk_partial<DT, DH, R, 4>(lds, n, scale, vreg, out);
#pragma unroll
  for (int k = 0; k < CO::ITEMS; ++k) {
    const int item = threadIdx.x + 256 * k;
    if (item < R * 64) {
      const int hi2 = item >> 6, ln = item & 63;
      const long prow = ((long)r * stride + c) * h + g * R + hi2;
      if (ln == 0) {
        part_ml[2 * prow] = out.m[k];
        part_ml[2 * prow + 1] = out.l[k];
      }
#pragma unroll
      for (int e = 0; e < S::DPL; ++e) part_acc[prow * DH + S::DPL * ln + e] = out.acc[k][e];
    }
  }
}

// ---------------------------------------------------------------------------
// prefill: grid (ceil(T / QB), h_kv).  A workgroup takes QB consecutive
// rows of one request (a block never straddles requests: rows are assigned
// per request in blocks of QB), stages each chunk once and runs every row's
// partial, merging serially into per-row running state.
// ---------------------------------------------------------------------------
template <int DT, int DH, int R, int NW, int QB, bool REL = false>
__global__ __launch_bounds__(64 * NW) void k_prefill(
    const void* __restrict__ q, const int32_t* __restrict__ q_start,
    const int32_t* __restrict__ q_pos0, int Rq,
    const void* __restrict__ k_pool, const void* __restrict__ v_pool,
    const int32_t* __restrict__ block_table, int h, int h_kv, int page_size, int max_pages,
    float scale, void* __restrict__ out) {
  typedef AttnShape<DT, DH> S;
  typedef ChunkOut<R, NW, S::DPL> CO;
  constexpr int C = 64 * NW;
  constexpr int DPL = S::DPL;
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int blk = blockIdx.x, g = blockIdx.y;
  // request of this block: rows are cut into blocks of QB per request, in
  // request order; the grid is an upper bound and surplus blocks exit
  int r = -1, first = 0;
  for (int i = 0; i < Rq; ++i) {
    const int nb = (q_start[i + 1] - q_start[i] + QB - 1) / QB;
    if (blk < first + nb) { r = i; break; }
    first += nb;
  }
  if (r < 0) return;
  const int t0 = q_start[r] + (blk - first) * QB;
  const int t1 = min(t0 + QB, q_start[r + 1]);
  if (t0 >= t1) return;
  const int pos0 = q_pos0[r] + (t0 - q_start[r]);
  const int pos_last = pos0 + (t1 - t0) - 1;
  const int32_t* bt = block_table + (long)r * max_pages;

  float Mr[QB][CO::ITEMS], Lr[QB][CO::ITEMS], Ar[QB][CO::ITEMS][DPL];
  // Chunk boundaries: absolute multiples of C (REL = false, the invariant
  // path); the twin (REL = true) starts them at the prefill chunk's first
  // position (rounded down to a page), so they move with the prompt's cuts.
  const int shift = REL ? ((q_pos0[r] % C) & ~(kPage - 1)) : 0;
  auto jstart = [&](int c) { return shift == 0 ? c * C : (c == 0 ? 0 : shift + (c - 1) * C); };
  const int nch = shift == 0 ? pos_last / C + 1
                             : (pos_last < shift ? 1 : (pos_last - shift) / C + 2);
  for (int c = 0; c < nch; ++c) {
    const int j0 = jstart(c);
    const int jend = jstart(c + 1);
    const int nmax = min(jend, pos_last + 1) - j0;
    uint32_t vreg[64][S::VW];
    stage_chunk<DT, DH, NW>(lds, k_pool, v_pool, bt, j0, nmax, g, h_kv, vreg);
#pragma unroll
    for (int qi = 0; qi < QB; ++qi) {
      const int t = t0 + qi;
      if (t < t1) {
        const int pos = pos0 + qi;
        const int n = min(jend, pos + 1) - j0;  // keys of this chunk visible to row t
        if (n > 0) {                             // uniform across the workgroup
          stage_q<DT, DH, R, NW>(lds, q, ((long)t * h + g * R) * DH);
          __syncthreads();
          CO co;
          chunk_partial<DT, DH, R, NW>(lds, min(n, C), scale, vreg, co);
#pragma unroll
          for (int k = 0; k < CO::ITEMS; ++k) {
            if (c == 0) {
              Mr[qi][k] = co.m[k];
              Lr[qi][k] = co.l[k];
#pragma unroll
              for (int e = 0; e < DPL; ++e) Ar[qi][k][e] = co.acc[k][e];
            } else {
              const float M = Mr[qi][k], mc = co.m[k];
              const float Mn = M > mc ? M : mc;
              const float a = exp_fixed(M - Mn), b = exp_fixed(mc - Mn);
              Lr[qi][k] = __builtin_fmaf(co.l[k], b, Lr[qi][k] * a);
#pragma unroll
              for (int e = 0; e < DPL; ++e)
                Ar[qi][k][e] = __builtin_fmaf(co.acc[k][e], b, Ar[qi][k][e] * a);
              Mr[qi][k] = Mn;
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int qi = 0; qi < QB; ++qi) {
    const int t = t0 + qi;
    if (t < t1) {
#pragma unroll
      for (int k = 0; k < CO::ITEMS; ++k) {
        const int item = threadIdx.x + 64 * NW * k;
        if (item < R * 64) {
          const int hi2 = item >> 6, ln = item & 63;
          const long o = ((long)t * h + g * R + hi2) * DH + DPL * ln;
#pragma unroll
          for (int e = 0; e < DPL; ++e) Elem<DT>::st(out, o + e, Ar[qi][k][e] / Lr[qi][k]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 KV: the chunk on matrix cores.
//
// Per chunk (keys j0 .. j0 + n - 1, n <= C) of one kv head, for a tile of up
// to 16 rows, each a (query row, query head) pair:
//   S = q K^T by v_mfma_f32_16x16x32_bf16, one accumulation chain over the
//       d_h in steps of 32 (ascending); s = S * scale;
//   m = max of s over the row's visible keys, plus 0;
//   p = exp(s - m) for visible keys, 0 otherwise; P = bf16(p);
//   l = P . 1 and acc = P V, each one MFMA chain over the chunk's keys in
//       steps of 32 (ascending).
// Every step depends only on the row's own q and the chunk's keys: a row's
// results do not depend on the other rows of its tile (decode and prefill
// rows give the same bits), on the batch, or on physical pages.
//
// Layout: wave w computes S for the chunk's keys 64w .. 64w + 63 (four key
// tiles of 16); its K fragments come straight from global memory (a tile is
// one 16-token page).  V of the whole chunk is copied to LDS (rows of d_h
// bf16, 16-byte pieces XOR-swizzled by the key) and read back as MFMA B
// fragments by transposing reads; P goes through LDS as bf16 [row][key]
// (8-key blocks swizzled by the row).  Wave w then owns d_h / 16 / NW
// 16-dim tiles of the output.  Keys past n read valid memory and are masked;
// their V rows are zeroed so that no stale value can reach the sum.
// ---------------------------------------------------------------------------
template <int DH, int C, int MT, int VH = 1, int PR = 16>
struct MfmaLds {
  static constexpr int NW = C / 64;
  static constexpr int RB = DH * 2;                       // bytes per V row
  static constexpr int V_OFF = 0;                         // bf16 V [C / VH][DH]
  static constexpr int P_OFF = C / VH * RB;               // bf16 P [MT * PR][C]
  static constexpr int MX_OFF = P_OFF + MT * PR * C * 2;  // fp32 [NW][MT * 16]
  static constexpr int BYTES = MX_OFF + NW * MT * 16 * 4;
  static constexpr int PM = (C / 8 < 16 ? C / 8 : 16) - 1;  // P block swizzle mask
};

// V rows in LDS: the 16-byte pieces of row `key` are XOR-swizzled by an even
// mask, so pairs of pieces (the 32 bytes one transposing read takes from a
// row) stay together, and the four rows of a 16-lane group and the rows of
// two neighbouring groups (keys 8 apart) fall on distinct banks.
template <int DH>
__device__ __forceinline__ int vswz_mask(int key) {
  constexpr int PAIRS = DH * 2 / 32;
  return 2 * (((key & 3) | (((key >> 3) & 1) << 2)) & (PAIRS - 1));
}

template <int DH>
__device__ __forceinline__ uint32_t vswz(int key, int piece) {
  return (uint32_t)(key * DH * 2 + 16 * (piece ^ vswz_mask<DH>(key)));
}

// Copies V rows of this wave's 64 keys (absolute keys j0 + 64w + k) into the
// chunk's LDS block, one 1 KiB copy per instruction, page ids per 16 keys.
template <int DH>
__device__ __forceinline__ void mfma_stage_v(char* lds, const char* vbase, long pstride,
                                             const int (&pg)[4], int wave) {
  constexpr int RB = DH * 2, SLOTS = RB / 16, KPI = 1024 / RB;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int inst = 0; inst < 64 / KPI; ++inst) {
    const int k = inst * KPI + lane / SLOTS;       // key within the wave
    const int slot = lane % SLOTS;
    const int key = 64 * wave + k;                 // key within the chunk
    const int page = pg[k / kPage];
    const char* src = vbase + page * pstride + (k % kPage) * RB + 16 * (slot ^ vswz_mask<DH>(key));
    dma16_nt(src, lds + (64 * wave + inst * KPI) * RB);
  }
}

// K fragments (B operand of QK) of this wave's four key tiles; tiles at or
// past `ntiles` (wholly past the chunk's end, masked) are not read.
template <int DH>
__device__ __forceinline__ void mfma_load_k(u32x4_t (&kf)[4][DH / 32], const char* kbase,
                                            long pstride, const int (&pg)[4], int ntiles) {
  const int lane = threadIdx.x & 63;
  // lane l takes token l % 16, dims 32 s + 8 (l / 16) .. + 7: unit 4 s + l / 16
  // of the unit-major block, at (unit * kPage + token) * 16 = 1024 s + 16 l --
  // each operand is one contiguous KiB
  static_assert(kPage == 16, "one 16-token page per operand");
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const char* blk = kbase + pg[t] * pstride + 16 * lane;
#pragma unroll
    for (int s = 0; s < DH / 32; ++s)   // read once: non-temporal
      kf[t][s] = t < ntiles
                     ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(blk + 1024 * s))
                     : u32x4_t{0u, 0u, 0u, 0u};
  }
}

// Key tiles of wave `wave` (keys 64 wave + 16 t ..) that hold a key below n.
__device__ __forceinline__ int live_tiles(int n, int wave) {
  return min(4, max(0, (n - 64 * wave + 15) / 16));
}

// Zero V rows n .. of this wave's keys (keys past the chunk's end).
template <int DH>
__device__ __forceinline__ void mfma_zero_v_tail(char* lds, int n, int wave) {
  constexpr int RB = DH * 2, SLOTS = RB / 16;
  const int lane = threadIdx.x & 63;
  const int k0 = max(n, 64 * wave), k1 = 64 * wave + 64;
  for (int i = lane; i < (k1 - k0) * SLOTS; i += 64)
    *reinterpret_cast<uint4*>(lds + (k0 + i / SLOTS) * RB + 16 * (i % SLOTS)) =
        make_uint4(0u, 0u, 0u, 0u);
}

// V in two halves through one buffer of C / 2 rows: wave w copies keys
// C / 2 * half + 32 w .. + 31 of the chunk (page ids vpg, one per 16 keys) to
// rows 32 w .. 32 w + 31.
template <int DH, int C>
__device__ __forceinline__ void mfma_stage_v_half(char* lds, const char* vbase, long pstride,
                                                  const int (&vpg)[2], int wave) {
  constexpr int RB = DH * 2, SLOTS = RB / 16, KPI = 1024 / RB, KW = C / 2 / (C / 64);
  static_assert(KW == 32, "32 keys per wave and half");
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int inst = 0; inst < KW / KPI; ++inst) {
    const int k = inst * KPI + lane / SLOTS;       // key within the wave's 32
    const int slot = lane % SLOTS;
    const int row = KW * wave + k;                 // row of the half buffer
    const char* src = vbase + vpg[k / kPage] * pstride + (k % kPage) * RB +
                      16 * (slot ^ vswz_mask<DH>(row));
    dma16_nt(src, lds + (KW * wave + inst * KPI) * RB);
  }
}

// Zero the rows of this wave's 32 keys of the half that lie at or past n.
template <int DH, int C>
__device__ __forceinline__ void mfma_zero_v_half_tail(char* lds, int n, int half, int wave) {
  constexpr int RB = DH * 2, SLOTS = RB / 16, KW = 32;
  const int lane = threadIdx.x & 63;
  const int first = max(n - C / 2 * half, KW * wave), end = KW * wave + KW;   // rows
  for (int i = lane; i < (end - first) * SLOTS; i += 64)
    *reinterpret_cast<uint4*>(lds + (first + i / SLOTS) * RB + 16 * (i % SLOTS)) =
        make_uint4(0u, 0u, 0u, 0u);
}

// The chunk for MT row tiles.  qf: A fragments of q; kf: this wave's K
// fragments; key abs position of (wave, tile t, lane) = j0 + 64w + 16t +
// (l & 15); lastpos[mt][j]: last visible absolute key of row 4 (l >> 4) + j
// of tile mt (-1 for rows that are not used).  Only rows with j < RJ may be
// used (decode puts its query heads on rows 0, 4, 8, 12 and passes RJ = 1;
// P then keeps those four rows only and the other rows enter P V as zeros).
// V must be staged (and the tail zeroed) by every wave before the call; with
// VH = 2 the buffer holds the first C / 2 keys and next_v_half() refills it
// with the rest once P V reaches them.  Outputs for this lane's rows and this
// wave's dim tiles; m = -inf marks a row with no visible key.
template <int DH, int C, int MT, int RJ = 4, int VH = 1, class H1 = NoHook, class H2 = NoHook>
__device__ __forceinline__ void mfma_chunk(char* lds, const u32x4_t (&qf)[MT][DH / 32],
                                           const u32x4_t (&kf)[4][DH / 32], int j0,
                                           const int (&lastpos)[MT][4], float scale,
                                           float (&m_out)[MT][4], float (&l_out)[MT][4],
                                           f32x4_t (&acc)[MT][DH / 16 / (C / 64)],
                                           const H1& after_qk = H1(),
                                           const H2& next_v_half = H2()) {
  // RJ = 1 keeps only P rows 4 i (the others are zero): 4 rows per tile
  constexpr int PR = RJ == 1 ? 4 : 16;
  typedef MfmaLds<DH, C, MT, VH, PR> L;
  static_assert(VH == 1 || VH == 2, "V resident whole or in two halves");
  static_assert(RJ == 1 || RJ == 4, "all rows of a tile, or rows 4 i");
  constexpr int NW = L::NW, KS = DH / 32, DPW = DH / 16 / NW;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g4 = lane >> 4, col = lane & 15;
  float* mx = reinterpret_cast<float*>(lds + L::MX_OFF);
  char* pl = lds + L::P_OFF;

  // ---- S = q K^T, scaled and masked
  float sv[MT][4][4];  // [row tile][key tile][j]
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f32x4_t c = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) c = mfma16(qf[mt][s], kf[t][s], c);
      const int key = j0 + 64 * wave + 16 * t + col;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sv[mt][t][j] = (j < RJ && key <= lastpos[mt][j]) ? c[j] * scale : -__builtin_inff();
    }
  }
  after_qk();  // the K fragments are free
  // ---- row maxima: in lane over the key tiles, over the 16 lanes of the
  // row group, then over the waves
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int j = 0; j < RJ; ++j) {
      float v = fmaxf(fmaxf(sv[mt][0][j], sv[mt][1][j]), fmaxf(sv[mt][2][j], sv[mt][3][j]));
      v = row16_max(v);
      if (col == 0) mx[wave * MT * 16 + mt * 16 + 4 * g4 + j] = v;
    }
  }
  __syncthreads();
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int j = 0; j < RJ; ++j) {
      float v = mx[mt * 16 + 4 * g4 + j];
#pragma unroll
      for (int w = 1; w < NW; ++w) v = fmaxf(v, mx[w * MT * 16 + mt * 16 + 4 * g4 + j]);
      m_out[mt][j] = v + 0.0f;
    }
  }
  // ---- P = bf16(exp(s - m)) into LDS [row][key]
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int key = 64 * wave + 16 * t + col;  // within the chunk
#pragma unroll
      for (int j = 0; j < RJ; ++j) {
        const int row = 4 * g4 + j;
        const float mm = m_out[mt][j];
        // a masked key: exp(-inf) = 0 (a row with no visible key subtracts 0)
        const float p = exp_p(sv[mt][t][j] - (mm == -__builtin_inff() ? 0.0f : mm));
        const int prow = PR == 16 ? row : row >> 2;   // row 4 g4 when PR = 4
        const uint32_t off = (uint32_t)((mt * PR + prow) * C * 2 +
                                        16 * ((key >> 3) ^ (row & L::PM)) + 2 * (key & 7));
        *reinterpret_cast<uint16_t*>(pl + off) = (uint16_t)p_bf16x2(p, 0.0f);
      }
    }
  }
  __syncthreads();
  // ---- l = P . 1 and acc = P V over the chunk's keys, 32 at a time
  const u32x4_t ones = u32x4_t{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  f32x4_t lacc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    lacc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int d = 0; d < DPW; ++d) acc[mt][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const int e = col >> 2, c4 = col & 3;  // this lane as a transposing-read source
#pragma unroll
  for (int ks = 0; ks < C / 32; ++ks) {
    // second half of the keys: the caller refills the V buffer
    if (VH == 2 && ks == C / 64) next_v_half();
    const int vrow0 = (VH == 2 && ks >= C / 64) ? C / 2 : 0;   // first key in the buffer
    u32x4_t a[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = col;
      if (PR == 16) {
        const uint32_t off = (uint32_t)((mt * 16 + row) * C * 2 +
                                        16 * ((4 * ks + g4) ^ (row & L::PM)));
        a[mt] = *reinterpret_cast<const u32x4_t*>(pl + off);
      } else {   // rows 4 i from LDS, zeros for the rest
        const uint32_t off = (uint32_t)((mt * PR + (row >> 2)) * C * 2 +
                                        16 * ((4 * ks + g4) ^ (row & L::PM)));
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(pl + off);
        a[mt] = (row & 3) == 0 ? v : u32x4_t{0u, 0u, 0u, 0u};
      }
      lacc[mt] = mfma16(a[mt], ones, lacc[mt]);
    }
#pragma unroll
    for (int d = 0; d < DPW; ++d) {
      const int dt = wave * DPW + d;                       // 16-dim tile
      const int piece = 2 * dt + (c4 >> 1);
      const int k0 = 32 * ks + 8 * g4 + e - vrow0;
      const uint2 lo = lds_read_tr16(lds, vswz<DH>(k0, piece) + 8 * (c4 & 1));
      const uint2 hi = lds_read_tr16(lds, vswz<DH>(k0 + 4, piece) + 8 * (c4 & 1));
      const u32x4_t b = u32x4_t{lo.x, lo.y, hi.x, hi.y};
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt][d] = mfma16(a[mt], b, acc[mt][d]);
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) l_out[mt][j] = lacc[mt][j];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = RJ; j < 4; ++j) m_out[mt][j] = -__builtin_inff();
}

// Decode partials on matrix cores, C / 64 waves.  One workgroup per (row,
// kv head), kv head fastest: blockIdx.x = row * h_kv + g, so the h_kv
// workgroups that read the same pages run side by side.  FREE = false: rows
// are chunk rows, chunks of C keys at absolute multiples of C.  FREE = true
// (the twin): B * stride rows, request r's split c of the length the
// occupancy policy gives it (free_splits), partial row r * stride + c.
template <int DH, int R, int C, bool FREE = false>
__global__ __launch_bounds__(C) void k_decode_mfma(
    const void* __restrict__ q, const void* __restrict__ k_pool, const void* __restrict__ v_pool,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ kv_len,
    const int32_t* __restrict__ chunk_off, int B, int h, int h_kv, int max_pages, float scale,
    float* __restrict__ part_ml, float* __restrict__ part_acc, int chunk2 = 0, int stride = 0) {
  typedef MfmaLds<DH, C, 1, 2, 4> L;   // V through LDS in two halves, P rows 4 i
  constexpr int KS = DH / 32, DPW = DH / 16 / L::NW;
  static_assert(R <= 4, "one row group holds the query heads of a kv head");
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = blockIdx.x % h_kv, row = blockIdx.x / h_kv;
  int r, j0, n, len;
  long crow;
  if (FREE) {
    r = row / stride;
    const int c = row % stride;
    len = kv_len[r];
    int slen;
    const int nr = free_splits(len, chunk2, &slen);
    if (c >= nr) return;
    j0 = c * slen;
    n = min(slen, len - j0);
    crow = (long)r * stride + c;
  } else {
    crow = row;
    // request owning this chunk row: the number of r >= 1 with chunk_off[r]
    // <= crow, counted 64 requests per vector load.  chunk_off ascends
    // strictly, so the lanes that pass form a prefix and the last of them
    // holds chunk_off[r] (chunk_off[0] = 0).
    r = 0;
    int base = 0;
    for (int b0 = 1; b0 < B; b0 += 64) {
      const int i = b0 + lane;
      const int v = i < B ? chunk_off[i] : 0x7fffffff;
      const int cnt = __builtin_popcountll(__ballot(v <= (int)crow));
      r += cnt;
      if (cnt > 0) base = __builtin_amdgcn_readlane(v, cnt - 1);
      if (cnt < 64) break;
    }
    r = __builtin_amdgcn_readfirstlane(r);
    base = __builtin_amdgcn_readfirstlane(base);
    j0 = ((int)crow - base) * C;
  }
  // page ids: loaded with clamped indices before kv_len (so the loads go out
  // together), then every page past the chunk's last key replaced by its
  // first (a valid page)
  const int32_t* bt = block_table + (long)r * max_pages;
  int pg[4];
  const int first = bt[j0 / kPage];
  int ids[4], vids[2][2];
#pragma unroll
  for (int p = 0; p < 4; ++p)
    ids[p] = bt[min((j0 + 64 * wave + kPage * p) / kPage, max_pages - 1)];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int p = 0; p < 2; ++p)
      vids[hf][p] = bt[min((j0 + C / 2 * hf + 32 * wave + kPage * p) / kPage, max_pages - 1)];
  if (!FREE) {
    len = kv_len[r];
    n = min(C, len - j0);
  }
  int vpg[2][2];   // V pages of this wave's 32 keys of each half
#pragma unroll
  for (int p = 0; p < 4; ++p) pg[p] = 64 * wave + kPage * p < n ? ids[p] : first;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int p = 0; p < 2; ++p)
      vpg[hf][p] = C / 2 * hf + 32 * wave + kPage * p < n ? vids[hf][p] : first;
  const long hstride = (long)kPage * DH * 2, pstride = hstride * h_kv;
  const char* kbase = static_cast<const char*>(k_pool) + g * hstride;
  const char* vbase = static_cast<const char*>(v_pool) + g * hstride;
  u32x4_t kf[4][KS];
  mfma_load_k<DH>(kf, kbase, pstride, pg, live_tiles(n, wave));
  mfma_stage_v_half<DH, C>(lds, vbase, pstride, vpg[0], wave);
  // query head hd sits on A row 4 hd, so each row group of the score tile
  // (lanes 16 G .. 16 G + 15, j = 0) holds one head: every lane has a real
  // score per key tile
  u32x4_t qf[1][KS];
  const int col = lane & 15, g4 = lane >> 4;
  const bool qreal = (col & 3) == 0 && (col >> 2) < R;
  const uint16_t* qrow =
      static_cast<const uint16_t*>(q) + ((long)r * h + g * R + (qreal ? col >> 2 : 0)) * DH;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(qrow + 8 * g4 + 32 * s);
    qf[0][s] = qreal ? v : u32x4_t{0u, 0u, 0u, 0u};
  }
  BI_WAIT_VMCNT(0);
  if (n < C / 2) mfma_zero_v_half_tail<DH, C>(lds, n, 0, wave);
  int lastpos[1][4];
  lastpos[0][0] = g4 < R ? j0 + n - 1 : -1;
  lastpos[0][1] = lastpos[0][2] = lastpos[0][3] = -1;
  float m[1][4], l[1][4];
  f32x4_t acc[1][DPW];
  // between the halves of P V: every wave is done with the first half of V;
  // copy the second (keys past n only zeroed) and wait for all of it
  auto v_second_half = [&]() {
    __syncthreads();
    if (n > C / 2) mfma_stage_v_half<DH, C>(lds, vbase, pstride, vpg[1], wave);
    BI_WAIT_VMCNT(0);
    if (n < C) mfma_zero_v_half_tail<DH, C>(lds, n, 1, wave);
    __syncthreads();
  };
  mfma_chunk<DH, C, 1, 1, 2>(lds, qf, kf, j0, lastpos, scale, m, l, acc, NoHook(),
                             v_second_half);
  if (g4 < R) {  // row 4 g4 = query head g4, in every lane of row group g4
    const long prow = crow * h + g * R + g4;
    if (col == 0 && wave == 0) {
      part_ml[2 * prow] = m[0][0];
      part_ml[2 * prow + 1] = l[0][0];
    }
#pragma unroll
    for (int d = 0; d < DPW; ++d) part_acc[prow * DH + 16 * (wave * DPW + d) + col] = acc[0][d][0];
  }
}

// Prefill on matrix cores: grid (blocks of QB = 16 MT / R query rows of one
// request, h_kv), C / 64 waves.  Each chunk of keys is staged once for the
// block's rows; each row merges the chunks' partials in chunk order with the
// rule of the decode merge, so row t equals the decode of kv_len = t + 1.
// REL (twin): chunk boundaries start at the prompt cut (rounded down to a
// page) instead of at absolute multiples of C.
template <int DH, int R, int C, int MT, bool REL = false>
__global__ __launch_bounds__(C) void k_prefill_mfma(
    const void* __restrict__ q, const int32_t* __restrict__ q_start,
    const int32_t* __restrict__ q_pos0, int Rq, const void* __restrict__ k_pool,
    const void* __restrict__ v_pool, const int32_t* __restrict__ block_table, int h, int h_kv,
    int max_pages, float scale, void* __restrict__ out) {
  typedef MfmaLds<DH, C, MT, 2> L;   // V through LDS in two halves
  constexpr int KS = DH / 32, DPW = DH / 16 / L::NW, QB = MT * 16 / R;
  static_assert((MT * 16) % R == 0, "row tiles hold whole query rows");
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, g4 = lane >> 4;
  // the last row blocks see the most chunks: launch them first
  const int blk = gridDim.x - 1 - blockIdx.x, g = blockIdx.y;
  int r = -1, firstb = 0;  // request of this block: blocks of QB rows, request by request
  for (int i = 0; i < Rq; ++i) {
    const int nb = (q_start[i + 1] - q_start[i] + QB - 1) / QB;
    if (blk < firstb + nb) { r = i; break; }
    firstb += nb;
  }
  if (r < 0) return;
  const int t0 = q_start[r] + (blk - firstb) * QB;
  const int t1 = min(t0 + QB, q_start[r + 1]);
  if (t0 >= t1) return;
  const int nrows = t1 - t0;
  const int pos0 = q_pos0[r] + (t0 - q_start[r]);
  const int pos_last = pos0 + nrows - 1;
  const int32_t* bt = block_table + (long)r * max_pages;
  const long hstride = (long)kPage * DH * 2, pstride = hstride * h_kv;
  const char* kbase = static_cast<const char*>(k_pool) + g * hstride;
  const char* vbase = static_cast<const char*>(v_pool) + g * hstride;

  // q fragments: A row mt * 16 + col is query row (that / R), head (that % R)
  u32x4_t qf[MT][KS];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int rr = mt * 16 + col, rho = rr / R, hd = rr % R;
    const bool real = rho < nrows;
    const uint16_t* qrow =
        static_cast<const uint16_t*>(q) + ((long)(t0 + (real ? rho : 0)) * h + g * R + hd) * DH;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(qrow + 8 * g4 + 32 * s);
      qf[mt][s] = real ? v : u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  int rowpos[MT][4];  // this lane's rows: absolute position, or -1
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rho = (mt * 16 + 4 * g4 + j) / R;
      rowpos[mt][j] = rho < nrows ? pos0 + rho : -1;
    }

  const int shift = REL ? ((q_pos0[r] % C) & ~(kPage - 1)) : 0;
  auto jstart = [&](int c) { return shift == 0 ? c * C : (c == 0 ? 0 : shift + (c - 1) * C); };
  const int nch = shift == 0 ? pos_last / C + 1
                             : (pos_last < shift ? 1 : (pos_last - shift) / C + 2);
  float M[MT][4], Lr[MT][4];
  f32x4_t A[MT][DPW];
  for (int c = 0; c < nch; ++c) {
    const int j0 = jstart(c);
    const int n = min(jstart(c + 1), pos_last + 1) - j0;
    int pg[4], vpg[2][2];   // K pages of this wave's 64 keys; V pages of its 32 keys per half
    const int first = bt[j0 / kPage];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int k0 = 64 * wave + kPage * p;
      pg[p] = k0 < n ? bt[(j0 + k0) / kPage] : first;
    }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int k0 = C / 2 * hf + 32 * wave + kPage * p;
        vpg[hf][p] = k0 < n ? bt[(j0 + k0) / kPage] : first;
      }
    if (c > 0) __syncthreads();  // the previous chunk's V and P are no longer read
    u32x4_t kf[4][KS];
    mfma_load_k<DH>(kf, kbase, pstride, pg, live_tiles(n, wave));
    mfma_stage_v_half<DH, C>(lds, vbase, pstride, vpg[0], wave);
    BI_WAIT_VMCNT(0);
    if (n < C / 2) mfma_zero_v_half_tail<DH, C>(lds, n, 0, wave);
    int lastpos[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) lastpos[mt][j] = min(rowpos[mt][j], j0 + n - 1);
    float m[MT][4], l[MT][4];
    f32x4_t acc[MT][DPW];
    // between the halves of P V: every wave is done with the first half of
    // V; copy the second (keys past n only zeroed) and wait for all of it
    auto v_second_half = [&]() {
      __syncthreads();
      if (n > C / 2) mfma_stage_v_half<DH, C>(lds, vbase, pstride, vpg[1], wave);
      BI_WAIT_VMCNT(0);
      if (n < C) mfma_zero_v_half_tail<DH, C>(lds, n, 1, wave);
      __syncthreads();
    };
    mfma_chunk<DH, C, MT, 4, 2>(lds, qf, kf, j0, lastpos, scale, m, l, acc, NoHook(),
                                v_second_half);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (c == 0) {
          M[mt][j] = m[mt][j];
          Lr[mt][j] = l[mt][j];
#pragma unroll
          for (int d = 0; d < DPW; ++d) A[mt][d][j] = acc[mt][d][j];
        } else if (m[mt][j] != -__builtin_inff()) {  // the row sees keys of this chunk
          const float Mo = M[mt][j], mc = m[mt][j];
          const float Mn = Mo > mc ? Mo : mc;
          const float a = exp_fixed(Mo - Mn), b = exp_fixed(mc - Mn);
          Lr[mt][j] = __builtin_fmaf(l[mt][j], b, Lr[mt][j] * a);
#pragma unroll
          for (int d = 0; d < DPW; ++d)
            A[mt][d][j] = __builtin_fmaf(acc[mt][d][j], b, A[mt][d][j] * a);
          M[mt][j] = Mn;
        }
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rr = mt * 16 + 4 * g4 + j, rho = rr / R, hd = rr % R;
      if (rho < nrows) {
        const long o = ((long)(t0 + rho) * h + g * R + hd) * DH;
#pragma unroll
        for (int d = 0; d < DPW; ++d)
          Elem<1>::st(out, o + 16 * (wave * DPW + d) + col, A[mt][d][j] / Lr[mt][j]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 KV, 256-key chunks at absolute positions: prefill with each chunk
// staged once per workgroup for 128 TPW (row, head) pairs.
//
// Eight waves; wave w owns TPW tiles of 16 pairs: pair p = 16 (TPW w + tt) +
// i is query row p / R of the block at query head p % R of the kv head.  Per
// chunk, K of all 256 keys (page blocks as in the pool, unit-major) and V
// (rows of d_h, 16-byte pieces XOR-swizzled by the key) are copied to LDS
// once; each wave then takes its own rows through the whole chunk:
//   pass 1: S = q K^T key tile by key tile; the row maxima, m = max + 0;
//   pass 2: per 32 keys, S again (the same MFMA chains: the same bits),
//           p = bf16(exp(s - m)) into the wave's LDS scratch as P^T
//           [key][row], read back as A operands by transposing reads;
//           l = P . 1 and acc = P V, one MFMA chain each over the chunk's
//           keys in steps of 32.
// Every per-element chain -- a score's chain over d_h, the key chains of l
// and acc, the mask, the exp and the rounding of p -- is the decode chunk's,
// with the same operand layouts, so each row's chunk partial is the decode
// partial bit for bit.  Steps past the wave's last visible key are skipped:
// their P is zero in every row of the wave, and a step of zero products
// leaves each accumulator (never a negative zero) as it is.  Each row merges
// its chunk partials in chunk order with the decode merge rule.
// ---------------------------------------------------------------------------
template <int DH, int TPW>
struct RowsLds {
  static constexpr int C = 256, NWV = 8, RB = DH * 2;
  static constexpr int K_OFF = 0;                 // bf16 K page blocks [C / 16][unit][16]
  static constexpr int V_OFF = C * RB;            // bf16 V [C][DH], swizzled pieces
  static constexpr int P_OFF = 2 * C * RB;        // per wave: bf16 P^T [TPW][32][16]
  static constexpr int PW = TPW * 16 * 64;
  static constexpr int BYTES = P_OFF + NWV * PW;
};

// One chunk for one wave's TPW row tiles: the maxima (pass 1), then P, l and
// acc 32 keys at a time (pass 2).  K and V are staged in LDS; pscr is the
// wave's P scratch, bf16 P^T [32 keys][16 rows] per tile, read back as A
// operands by transposing reads.  MASK = false: every row sees all nkt * 16
// keys.  A masked score gives p = exp(-inf) = 0; a row that sees no key of
// the chunk (m = -inf) subtracts 0 instead of m, so that p is 0, not NaN.
template <int DH, int TPW, bool MASK>
__device__ __forceinline__ void rows_chunk(char* lds, char* pscr,
                                           const u32x4_t (&qf)[TPW][DH / 32],
                                           const int (&rowpos)[TPW][4], int j0, int nkt, int nks,
                                           float scale, float (&m)[TPW][4],
                                           f32x4_t (&lacc)[TPW], f32x4_t (&acc)[TPW][DH / 16]) {
  typedef RowsLds<DH, TPW> L;
  constexpr int KS = DH / 32, DT = DH / 16, RB = L::RB;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, g4 = lane >> 4;
  const int e = col >> 2, c4 = col & 3;  // this lane as a transposing-read source
  const char* kl = lds + L::K_OFF + 16 * lane;
  // ---- pass 1: row maxima
  float mx[TPW][4];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
    for (int j = 0; j < 4; ++j) mx[tt][j] = -__builtin_inff();
  // two key tiles per step, their chains interleaved (a tile at or past nkt
  // lies past every row's last key: masked)
#pragma unroll 2
  for (int kt = 0; kt < nkt; kt += 2) {
    u32x4_t kf[2][KS];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int s = 0; s < KS; ++s)
        kf[h2][s] = *reinterpret_cast<const u32x4_t*>(kl + (kt + h2) * kPage * RB + 1024 * s);
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      f32x4_t cc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) cc[h2] = mfma16(qf[tt][s], kf[h2][s], cc[h2]);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int key = j0 + 16 * (kt + h2) + col;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          mx[tt][j] = fmaxf(mx[tt][j], (!MASK || key <= rowpos[tt][j]) ? cc[h2][j] * scale
                                                                     : -__builtin_inff());
      }
    }
  }
  float msub[TPW][4];  // subtracted before the exp
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m[tt][j] = row16_max(mx[tt][j]) + 0.0f;
      msub[tt][j] = (MASK && m[tt][j] == -__builtin_inff()) ? 0.0f : m[tt][j];
    }
  // ---- pass 2
  const u32x4_t ones = u32x4_t{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    lacc[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int d = 0; d < DT; ++d) acc[tt][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // per-lane LDS addresses of step 0; step ks adds ks 32 rows of V and
  // ks 2 pages of K (the V swizzle mask of a key depends on key % 4 and
  // key / 8 % 2 only, the same at every step, and the high half of a
  // transposing read lies 4 rows on)
  uint32_t vofs[DT];  // from lds
#pragma unroll
  for (int d = 0; d < DT; ++d)
    vofs[d] = L::V_OFF + vswz<DH>(8 * g4 + e, 2 * d + (c4 >> 1)) + 8 * (c4 & 1);
  const uint32_t pw0 = (uint32_t)(col * 32 + 8 * (g4 ^ (col >> 3)));  // key col of half 0
  const uint32_t pw1 = (uint32_t)((16 + col) * 32 + 8 * (g4 ^ (2 + (col >> 3))));
  const uint32_t pr = (uint32_t)((8 * g4 + e) * 32 + 8 * (c4 ^ g4));
  for (int ks = 0; ks < nks; ++ks) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the last step's P reads are done
    u32x4_t kf[2][KS];
    const char* kstep = kl + ks * 2 * kPage * RB;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int s = 0; s < KS; ++s)
        kf[h2][s] = *reinterpret_cast<const u32x4_t*>(kstep + h2 * kPage * RB + 1024 * s);
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      f32x4_t cc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) cc[h2] = mfma16(qf[tt][s], kf[h2][s], cc[h2]);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int key = j0 + 16 * (2 * ks + h2) + col;
        float pv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float sv =
              (!MASK || key <= rowpos[tt][j]) ? cc[h2][j] * scale : -__builtin_inff();
          pv[j] = exp_p(sv - msub[tt][j]);
        }
        // rows 4 g4 .. 4 g4 + 3 of key 16 h2 + col: 8 bytes of P^T, in slot
        // g4 ^ (key / 8) of the key's 32 (lanes col and col + 8 on
        // different banks)
        *reinterpret_cast<uint2*>(pscr + tt * 1024 + (h2 ? pw1 : pw0)) =
            make_uint2(p_bf16x2(pv[0], pv[1]), p_bf16x2(pv[2], pv[3]));
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // P written
    u32x4_t a[TPW];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      // A row col, keys 8 g4 .. 8 g4 + 7 of the 32 (key / 8 = g4)
      const uint2 lo = lds_read_tr16(pscr, tt * 1024 + pr);
      const uint2 hi = lds_read_tr16(pscr, tt * 1024 + pr + 4 * 32);
      a[tt] = u32x4_t{lo.x, lo.y, hi.x, hi.y};
      lacc[tt] = mfma16(a[tt], ones, lacc[tt]);
    }
#pragma unroll
    for (int d = 0; d < DT; ++d) {
      const uint32_t o = vofs[d] + ks * 32 * RB;
      const uint2 lo = lds_read_tr16(lds, o);
      const uint2 hi = lds_read_tr16(lds, o + 4 * RB);
      const u32x4_t b = u32x4_t{lo.x, lo.y, hi.x, hi.y};
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) acc[tt][d] = mfma16(a[tt], b, acc[tt][d]);
    }
  }
}

template <int DH, int R, int TPW>
__global__ __launch_bounds__(512) void k_prefill_rows(
    const void* __restrict__ q, const int32_t* __restrict__ q_start,
    const int32_t* __restrict__ q_pos0, int Rq, const void* __restrict__ k_pool,
    const void* __restrict__ v_pool, const int32_t* __restrict__ block_table, int h, int h_kv,
    int max_pages, float scale, void* __restrict__ out) {
  typedef RowsLds<DH, TPW> L;
  constexpr int C = L::C, KS = DH / 32, DT = DH / 16, RB = L::RB;
  constexpr int PAIRS = 16 * TPW * L::NWV, QB = PAIRS / R;
  constexpr int KI = kPage * RB / 1024;                  // 1 KiB copies per K page block
  constexpr int SLOTS = RB / 16, KPI = 1024 / RB;        // V: pieces per row, rows per copy
  static_assert(PAIRS % R == 0, "a block holds whole query rows");
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, g4 = lane >> 4;
  // one-dimensional grid, kv head fastest: the row blocks that see the most
  // chunks start first on every head, and (with the workgroups dealt to the
  // XCDs in turn) the blocks of one kv head share one XCD's L2 when h_kv is
  // a multiple of the XCD count
  const int g = blockIdx.x % h_kv, blk = gridDim.x / h_kv - 1 - blockIdx.x / h_kv;
  int r = -1, firstb = 0;  // request of this block: blocks of QB rows, request by request
  for (int i = 0; i < Rq; ++i) {
    const int nb = (q_start[i + 1] - q_start[i] + QB - 1) / QB;
    if (blk < firstb + nb) { r = i; break; }
    firstb += nb;
  }
  if (r < 0) return;
  const int t0 = q_start[r] + (blk - firstb) * QB;
  const int t1 = min(t0 + QB, q_start[r + 1]);
  if (t0 >= t1) return;
  const int nrows = t1 - t0;
  const int pos0 = q_pos0[r] + (t0 - q_start[r]);
  const int pos_last = pos0 + nrows - 1;
  const int32_t* bt = block_table + (long)r * max_pages;
  const long hstride = (long)kPage * DH * 2, pstride = hstride * h_kv;
  const char* kbase = static_cast<const char*>(k_pool) + g * hstride;
  const char* vbase = static_cast<const char*>(v_pool) + g * hstride;

  // q fragments: A row i of tile tt is pair 16 (TPW wave + tt) + i
  u32x4_t qf[TPW][KS];
  int rowpos[TPW][4];  // this lane's result rows: absolute position, or -1
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int rr = 16 * (TPW * wave + tt) + col, rho = rr / R, hd = rr % R;
    const bool real = rho < nrows;
    const uint16_t* qrow =
        static_cast<const uint16_t*>(q) + ((long)(t0 + (real ? rho : 0)) * h + g * R + hd) * DH;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(qrow + 8 * g4 + 32 * s);
      qf[tt][s] = real ? v : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rj = (16 * (TPW * wave + tt) + 4 * g4 + j) / R;
      rowpos[tt][j] = rj < nrows ? pos0 + rj : -1;
    }
  }
  // last position among the wave's rows (-1: the wave has none)
  const int rho_first = 16 * TPW * wave / R;
  const int wlast = rho_first < nrows ? pos0 + min((16 * TPW * (wave + 1) - 1) / R, nrows - 1)
                                      : -1;
  char* pscr = lds + L::P_OFF + wave * L::PW;
  float M[TPW][4], Lr[TPW][4];
  f32x4_t A[TPW][DT];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) M[tt][j] = Lr[tt][j] = 0.0f;
#pragma unroll
    for (int d = 0; d < DT; ++d) A[tt][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const int nch = pos_last / C + 1;
  for (int c = 0; c < nch; ++c) {
    const int j0 = c * C;
    const int n = min(C, pos_last + 1 - j0);
    // this wave copies pages 2 w, 2 w + 1 of the chunk (keys 32 w .. + 31);
    // pages past the chunk's end read its first page and their V is zeroed
    const int first = bt[j0 / kPage];
    int pid[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int k0 = 32 * wave + kPage * p;
      pid[p] = k0 < n ? bt[(j0 + k0) / kPage] : first;
    }
    if (c > 0) __syncthreads();  // every wave is done with the previous chunk
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int kb = 32 * wave + kPage * p;  // first key of the page in the chunk
      const char* ksrc = kbase + pid[p] * pstride + 16 * lane;
#pragma unroll
      for (int i = 0; i < KI; ++i) dma16_nt(ksrc + 1024 * i, lds + L::K_OFF + kb * RB + 1024 * i);
      const char* vsrc = vbase + pid[p] * pstride;
#pragma unroll
      for (int inst = 0; inst < kPage / KPI; ++inst) {
        const int k = inst * KPI + lane / SLOTS, slot = lane % SLOTS;
        dma16_nt(vsrc + k * RB + 16 * (slot ^ vswz_mask<DH>(kb + k)),
                 lds + L::V_OFF + (kb + inst * KPI) * RB);
      }
    }
    BI_WAIT_VMCNT(0);
    if (n < 32 * wave + 32) {  // zero V rows of this wave's keys at or past n
      const int k0 = max(n, 32 * wave);
      for (int i = lane; i < (32 * wave + 32 - k0) * SLOTS; i += 64)
        *reinterpret_cast<uint4*>(lds + L::V_OFF + (k0 + i / SLOTS) * RB + 16 * (i % SLOTS)) =
            make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();
    if (wlast < j0) continue;  // no row of this wave sees a key of the chunk
    const int vis = min(n, wlast + 1 - j0);  // keys the wave's rows may see
    const int nkt = (vis + 15) / 16, nks = (vis + 31) / 32;

    float m[TPW][4];
    f32x4_t lacc[TPW], acc[TPW][DT];
    // every row of the wave sees every key of the chunk: no mask
    if (n == C && pos0 + rho_first >= j0 + C - 1)
      rows_chunk<DH, TPW, false>(lds, pscr, qf, rowpos, j0, C / 16, C / 32, scale, m, lacc, acc);
    else
      rows_chunk<DH, TPW, true>(lds, pscr, qf, rowpos, j0, nkt, nks, scale, m, lacc, acc);
    // ---- merge the chunk partial into each row's running result
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (c == 0) {
          M[tt][j] = m[tt][j];
          Lr[tt][j] = lacc[tt][j];
#pragma unroll
          for (int d = 0; d < DT; ++d) A[tt][d][j] = acc[tt][d][j];
        } else if (m[tt][j] != -__builtin_inff()) {  // the row sees keys of this chunk
          // the decode merge's weights exp(Mo - Mn) and exp(mc - Mn): one of
          // them is exp(0) = 1
          const float Mo = M[tt][j], mc = m[tt][j];
          const bool old_max = Mo > mc;
          const float Mn = old_max ? Mo : mc;
          const float ex = exp_p(old_max ? mc - Mo : Mo - mc);
          const float ea = old_max ? 1.0f : ex, eb = old_max ? ex : 1.0f;
          Lr[tt][j] = __builtin_fmaf(lacc[tt][j], eb, Lr[tt][j] * ea);
#pragma unroll
          for (int d = 0; d < DT; ++d)
            A[tt][d][j] = __builtin_fmaf(acc[tt][d][j], eb, A[tt][d][j] * ea);
          M[tt][j] = Mn;
        }
      }
    }
  }
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rr = 16 * (TPW * wave + tt) + 4 * g4 + j, rho = rr / R, hd = rr % R;
      if (rho < nrows) {
        const long o = ((long)(t0 + rho) * h + g * R + hd) * DH;
#pragma unroll
        for (int d = 0; d < DT; ++d) Elem<1>::st(out, o + 16 * d + col, A[tt][d][j] / Lr[tt][j]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct AttnArgsCheck {
  static bi_status common(const char* who, int h, int h_kv, int d_h, int page_size,
                          int kv_chunk, int dtype) {
    BI_REQUIRE(h >= 1 && h_kv >= 1 && h % h_kv == 0, BI_ERR_INVALID,
               "%s: h=%d must be a positive multiple of h_kv=%d", who, h, h_kv);
    const int R = h / h_kv;
    BI_REQUIRE(R == 2 || R == 4, BI_ERR_UNSUPPORTED, "%s: query group size %d not in {2,4}",
               who, R);
    BI_REQUIRE(d_h == 64 || d_h == 128, BI_ERR_UNSUPPORTED, "%s: d_h=%d not in {64,128}", who,
               d_h);
    BI_REQUIRE(dtype == BI_F32 || dtype == BI_BF16, BI_ERR_UNSUPPORTED, "%s: dtype %d", who,
               dtype);
    BI_REQUIRE(kv_chunk == 64 || kv_chunk == 256, BI_ERR_UNSUPPORTED,
               "%s: kv_chunk=%d not in {64,256}", who, kv_chunk);
    BI_REQUIRE(page_size == kPage, BI_ERR_UNSUPPORTED, "%s: page_size=%d (kernels are built "
               "for %d-token pages)", who, page_size, kPage);
    return BI_OK;
  }
};

template <int DT, int DH, int R, int NW>
static void launch_decode(const void* q, const void* kp, const void* vp, const int32_t* bt,
                          const int32_t* kvl, const int32_t* off, int B, int tot, int h,
                          int h_kv, int ps, int mp, float scale, float* ml, float* acc,
                          hipStream_t s) {
  constexpr int lds = AttnLds<DT, DH, R, NW>::BYTES;
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)k_decode_partials<DT, DH, R, NW>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    attr = true;
  }
  hipLaunchKernelGGL((k_decode_partials<DT, DH, R, NW>), dim3(tot, h_kv), dim3(64 * NW), lds, s,
                     q, kp, vp, bt, kvl, off, B, h, h_kv, ps, mp, scale, ml, acc);
}

// bf16 KV: matrix-core kernels, chunk length C = 64 nw.
template <int DH, int R, int C, bool FREE = false>
static void launch_decode_mfma(dim3 grid, const void* q, const void* kp, const void* vp,
                               const int32_t* bt, const int32_t* kvl, const int32_t* off, int B,
                               int h, int h_kv, int mp, float scale, float* ml, float* acc,
                               hipStream_t s, int chunk2 = 0, int stride = 0) {
  constexpr int lds = MfmaLds<DH, C, 1, 2, 4>::BYTES;
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)k_decode_mfma<DH, R, C, FREE>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    attr = true;
  }
  hipLaunchKernelGGL((k_decode_mfma<DH, R, C, FREE>), grid, dim3(C), lds, s, q, kp, vp, bt, kvl,
                     off, B, h, h_kv, mp, scale, ml, acc, chunk2, stride);
}

// Row tiles per workgroup of k_prefill_mfma (the twin's kernel, and the
// invariant path's at 64-key chunks): two at 256-key chunks (a 2048-token
// prompt measured 260 us against 300 with one and 414 with four, where the
// registers leave one workgroup per CU), one at 64 (more would spill).
template <int C>
constexpr int prefill_tiles() { return C == 256 ? 2 : 1; }

template <int DH, int R, int C, bool REL>
static void launch_prefill_mfma(const void* q, const int32_t* qs, const int32_t* qp, int Rq,
                                int T, const void* kp, const void* vp, const int32_t* bt, int h,
                                int h_kv, int mp, float scale, void* out, hipStream_t s) {
  constexpr int MT = prefill_tiles<C>();
  constexpr int lds = MfmaLds<DH, C, MT, 2>::BYTES, QB = 16 * MT / R;
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)k_prefill_mfma<DH, R, C, MT, REL>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    attr = true;
  }
  const int blocks = (T + QB - 1) / QB + Rq;
  hipLaunchKernelGGL((k_prefill_mfma<DH, R, C, MT, REL>), dim3(blocks, h_kv), dim3(C), lds, s,
                     q, qs, qp, Rq, kp, vp, bt, h, h_kv, mp, scale, out);
}

template <int DT, int DH, int R>
static void decode_nw(int nw, const void* q, const void* kp, const void* vp, const int32_t* bt,
                      const int32_t* kvl, const int32_t* off, int B, int tot, int h, int h_kv,
                      int ps, int mp, float scale, float* ml, float* acc, hipStream_t s) {
  if constexpr (DT == 1) {
    const dim3 grid((unsigned)tot * h_kv);
    if (nw == 1) launch_decode_mfma<DH, R, 64>(grid, q, kp, vp, bt, kvl, off, B, h, h_kv, mp, scale, ml, acc, s);
    else launch_decode_mfma<DH, R, 256>(grid, q, kp, vp, bt, kvl, off, B, h, h_kv, mp, scale, ml, acc, s);
  } else {
    if (nw == 1) launch_decode<DT, DH, R, 1>(q, kp, vp, bt, kvl, off, B, tot, h, h_kv, ps, mp, scale, ml, acc, s);
    else launch_decode<DT, DH, R, 4>(q, kp, vp, bt, kvl, off, B, tot, h, h_kv, ps, mp, scale, ml, acc, s);
  }
}

template <int DT, int DH>
static void decode_r(int R, int nw, const void* q, const void* kp, const void* vp,
                     const int32_t* bt, const int32_t* kvl, const int32_t* off, int B, int tot,
                     int h, int h_kv, int ps, int mp, float scale, float* ml, float* acc,
                     hipStream_t s) {
  if (R == 2) decode_nw<DT, DH, 2>(nw, q, kp, vp, bt, kvl, off, B, tot, h, h_kv, ps, mp, scale, ml, acc, s);
  else decode_nw<DT, DH, 4>(nw, q, kp, vp, bt, kvl, off, B, tot, h, h_kv, ps, mp, scale, ml, acc, s);
}

constexpr int kPrefillQB = 8;

template <int DT, int DH, int R, int NW, bool REL = false>
static void launch_prefill(const void* q, const int32_t* qs, const int32_t* qp, int Rq, int T,
                           const void* kp, const void* vp, const int32_t* bt, int h, int h_kv,
                           int ps, int mp, float scale, void* out, hipStream_t s) {
  constexpr int lds = AttnLds<DT, DH, R, NW>::BYTES;
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)k_prefill<DT, DH, R, NW, kPrefillQB, REL>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    attr = true;
  }
  const int blocks = (T + kPrefillQB - 1) / kPrefillQB + Rq;
  hipLaunchKernelGGL((k_prefill<DT, DH, R, NW, kPrefillQB, REL>), dim3(blocks, h_kv),
                     dim3(64 * NW), lds, s, q, qs, qp, Rq, kp, vp, bt, h, h_kv, ps, mp, scale, out);
}

template <int DH, int R, int TPW = 1>
static void launch_prefill_rows(const void* q, const int32_t* qs, const int32_t* qp, int Rq,
                                int T, const void* kp, const void* vp, const int32_t* bt, int h,
                                int h_kv, int mp, float scale, void* out, hipStream_t s) {
  constexpr int lds = RowsLds<DH, TPW>::BYTES, QR = 128 * TPW / R;
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)k_prefill_rows<DH, R, TPW>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    attr = true;
  }
  const int blocks = (T + QR - 1) / QR + Rq;
  hipLaunchKernelGGL((k_prefill_rows<DH, R, TPW>), dim3(blocks * h_kv), dim3(512), lds, s, q, qs,
                     qp, Rq, kp, vp, bt, h, h_kv, mp, scale, out);
}

template <int DT, int DH, int R, bool REL = false>
static void prefill_nw(int nw, const void* q, const int32_t* qs, const int32_t* qp, int Rq, int T,
                       const void* kp, const void* vp, const int32_t* bt, int h, int h_kv, int ps,
                       int mp, float scale, void* out, hipStream_t s) {
  if constexpr (DT == 1) {
    if (nw == 1) launch_prefill_mfma<DH, R, 64, REL>(q, qs, qp, Rq, T, kp, vp, bt, h, h_kv, mp, scale, out, s);
    else if (!REL) launch_prefill_rows<DH, R>(q, qs, qp, Rq, T, kp, vp, bt, h, h_kv, mp, scale, out, s);
    else launch_prefill_mfma<DH, R, 256, REL>(q, qs, qp, Rq, T, kp, vp, bt, h, h_kv, mp, scale, out, s);
  } else {
    if (nw == 1) launch_prefill<DT, DH, R, 1, REL>(q, qs, qp, Rq, T, kp, vp, bt, h, h_kv, ps, mp, scale, out, s);
    else launch_prefill<DT, DH, R, 4, REL>(q, qs, qp, Rq, T, kp, vp, bt, h, h_kv, ps, mp, scale, out, s);
  }
}

template <int DT, int DH, bool REL = false>
static void prefill_r(int R, int nw, const void* q, const int32_t* qs, const int32_t* qp, int Rq,
                      int T, const void* kp, const void* vp, const int32_t* bt, int h, int h_kv,
                      int ps, int mp, float scale, void* out, hipStream_t s) {
  if (R == 2) prefill_nw<DT, DH, 2, REL>(nw, q, qs, qp, Rq, T, kp, vp, bt, h, h_kv, ps, mp, scale, out, s);
  else prefill_nw<DT, DH, 4, REL>(nw, q, qs, qp, Rq, T, kp, vp, bt, h, h_kv, ps, mp, scale, out, s);
}

// ---- twin host plumbing --------------------------------------------------
// Occupancy policy of the decode twin, on the host: the batch and the longest
// sequence set a second chunk length from the device's compute units; a
// request then gets max(ceil(s/256), ceil(s/chunk2)) splits.
struct FreePolicy {
  int chunk2, stride;
};
static FreePolicy free_policy(int B, int h, int h_kv, int max_kv_len) {
  constexpr int kCUs = 256, kMaxSplits = 64;
  const double ext_seq = max_kv_len / 64.0;
  const int ext_cores = (int)(kCUs * (std::log2(ext_seq) > 1.0 ? std::log2(ext_seq) : 1.0));
  const int group = h / h_kv;
  const int block_h = group < 16 ? group : 16;
  const int token_grid = B * ((h + block_h - 1) / block_h);
  int ms2 = (ext_cores + token_grid - 1) / token_grid;
  ms2 = ms2 < kMaxSplits ? ms2 : kMaxSplits;
  ms2 = ms2 > 1 ? ms2 : 1;
  FreePolicy p;
  p.chunk2 = (max_kv_len + ms2 - 1) / ms2;
  // max(ceil(s/256), ceil(s/chunk2)) grows with s and bounds the split
  // count free_splits gives a request of length s, so its value at the
  // longest request bounds every request's count.  Partial rows of request
  // r start at r * stride.
  const int a = (max_kv_len + 255) / 256, b = (max_kv_len + p.chunk2 - 1) / p.chunk2;
  p.stride = a > b ? a : b;
  return p;
}

template <int DT, int DH, int R>
static void launch_decode_free(const void* q, const void* kp, const void* vp, const int32_t* bt,
                               const int32_t* kvl, int B, int h, int h_kv, int mp, float scale,
                               FreePolicy pol, float* ml, float* acc, hipStream_t s) {
  if constexpr (DT == 1) {
    launch_decode_mfma<DH, R, 256, true>(dim3((unsigned)B * pol.stride * h_kv), q, kp, vp, bt, kvl, nullptr,
                                         B, h, h_kv, mp, scale, ml, acc, s, pol.chunk2,
                                         pol.stride);
  } else {
    constexpr int lds = AttnLds<DT, DH, R, 4>::BYTES;
    static bool attr = false;
    if (!attr) {
      (void)hipFuncSetAttribute((const void*)k_decode_free<DT, DH, R>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      attr = true;
    }
    hipLaunchKernelGGL((k_decode_free<DT, DH, R>), dim3(B * pol.stride, h_kv), dim3(256), lds, s,
                       q, kp, vp, bt, kvl, h, h_kv, mp, scale, pol.chunk2, pol.stride, ml, acc);
  }
}

// The softmax weights alone: p[i] = exp_p(x[i]) and its bf16 bits.
__global__ __launch_bounds__(256) void k_softmax_weights(const float* __restrict__ x,
                                                         float* __restrict__ p,
                                                         uint16_t* __restrict__ pb, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float v = exp_p(x[i]);
  p[i] = v;
  if (pb != nullptr) pb[i] = (uint16_t)(p_bf16x2(v, 0.0f) & 0xffffu);
}

}  // namespace bi

extern "C" bi_status bi_softmax_weights(const float* x, float* p, uint16_t* p_bf16, int n,
                                        bi_stream stream) {
  using namespace bi;
  BI_REQUIRE(n >= 0, BI_ERR_INVALID, "bi_softmax_weights: bad size n=%d", n);
  if (n == 0) return BI_OK;
  BI_REQUIRE(x && p, BI_ERR_INVALID, "bi_softmax_weights: null pointer");
  hipLaunchKernelGGL(k_softmax_weights, dim3((n + 255) / 256), dim3(256), 0, as_stream(stream),
                     x, p, p_bf16, n);
  return launched("bi_softmax_weights");
}

extern "C" bi_status bi_prefill_attn(const void* q, const int32_t* q_start,
                                     const int32_t* q_pos0, int R, int T, const void* k_pool,
                                     const void* v_pool, const int32_t* block_table, int h,
                                     int h_kv, int d_h, int page_size, int max_pages,
                                     int kv_chunk, float scale, int dtype, void* out,
                                     bi_stream stream) {
  using namespace bi;
  bi_status st = AttnArgsCheck::common("bi_prefill_attn", h, h_kv, d_h, page_size, kv_chunk,
                                       dtype);
  if (st != BI_OK) return st;
  BI_REQUIRE(R >= 0 && T >= 0 && max_pages >= 1, BI_ERR_INVALID,
             "bi_prefill_attn: bad sizes R=%d T=%d max_pages=%d", R, T, max_pages);
  BI_REQUIRE(kv_chunk % page_size == 0, BI_ERR_UNSUPPORTED,
             "bi_prefill_attn: page_size %d must divide kv_chunk %d", page_size, kv_chunk);
  if (R == 0 || T == 0) return BI_OK;
  BI_REQUIRE(q && q_start && q_pos0 && k_pool && v_pool && block_table && out, BI_ERR_INVALID,
             "bi_prefill_attn: null pointer");
  BI_REQUIRE(aligned16(q) && aligned16(k_pool) && aligned16(v_pool) && aligned16(out),
             BI_ERR_INVALID, "bi_prefill_attn: pointers must be 16-byte aligned");
  // grids: (T / 8 + R, h_kv) for fp32; (T / 32 + R) x h_kv in one dimension
  // for the bf16 row-block kernel (32 or more rows per block)
  BI_REQUIRE((long)T / kPrefillQB + R < 0x7fffffffL && h_kv <= 65535 &&
                 ((long)T / 32 + R + 1) * h_kv < 0x7fffffffL,
             BI_ERR_INVALID, "bi_prefill_attn: grid too large");
  const int Rg = h / h_kv, nw = kv_chunk / 64;
  hipStream_t s = as_stream(stream);
  if (dtype == BI_BF16) {
    if (d_h == 128) prefill_r<1, 128>(Rg, nw, q, q_start, q_pos0, R, T, k_pool, v_pool, block_table, h, h_kv, page_size, max_pages, scale, out, s);
    else prefill_r<1, 64>(Rg, nw, q, q_start, q_pos0, R, T, k_pool, v_pool, block_table, h, h_kv, page_size, max_pages, scale, out, s);
  } else {
    if (d_h == 128) prefill_r<0, 128>(Rg, nw, q, q_start, q_pos0, R, T, k_pool, v_pool, block_table, h, h_kv, page_size, max_pages, scale, out, s);
    else prefill_r<0, 64>(Rg, nw, q, q_start, q_pos0, R, T, k_pool, v_pool, block_table, h, h_kv, page_size, max_pages, scale, out, s);
  }
  return launched("bi_prefill_attn");
}

extern "C" bi_status bi_decode_attn(const void* q, const void* k_pool, const void* v_pool,
                                    const int32_t* block_table, const int32_t* kv_len,
                                    const int32_t* chunk_off, int B, int total_chunks, int h,
                                    int h_kv, int d_h, int page_size, int max_pages,
                                    int kv_chunk, float scale, int dtype, float* part_ml,
                                    float* part_acc, bi_stream stream) {
  using namespace bi;
  bi_status st = AttnArgsCheck::common("bi_decode_attn", h, h_kv, d_h, page_size, kv_chunk,
                                       dtype);
  if (st != BI_OK) return st;
  BI_REQUIRE(B >= 0 && total_chunks >= 0 && max_pages >= 1, BI_ERR_INVALID,
             "bi_decode_attn: bad sizes B=%d total_chunks=%d max_pages=%d", B, total_chunks,
             max_pages);
  BI_REQUIRE(kv_chunk % page_size == 0, BI_ERR_UNSUPPORTED,
             "bi_decode_attn: page_size %d must divide kv_chunk %d", page_size, kv_chunk);
  if (B == 0 || total_chunks == 0) return BI_OK;
  BI_REQUIRE(total_chunks <= 0x7fffffff / h && h_kv <= 65535, BI_ERR_INVALID,
             "bi_decode_attn: grid too large");
  BI_REQUIRE(q && k_pool && v_pool && block_table && kv_len && chunk_off && part_ml && part_acc,
             BI_ERR_INVALID, "bi_decode_attn: null pointer");
  BI_REQUIRE(aligned16(q) && aligned16(k_pool) && aligned16(v_pool) && aligned16(part_acc),
             BI_ERR_INVALID, "bi_decode_attn: pointers must be 16-byte aligned");
  const int R = h / h_kv, nw = kv_chunk / 64;
  hipStream_t s = as_stream(stream);
  if (dtype == BI_BF16) {
    if (d_h == 128) decode_r<1, 128>(R, nw, q, k_pool, v_pool, block_table, kv_len, chunk_off, B, total_chunks, h, h_kv, page_size, max_pages, scale, part_ml, part_acc, s);
    else decode_r<1, 64>(R, nw, q, k_pool, v_pool, block_table, kv_len, chunk_off, B, total_chunks, h, h_kv, page_size, max_pages, scale, part_ml, part_acc, s);
  } else {
    if (d_h == 128) decode_r<0, 128>(R, nw, q, k_pool, v_pool, block_table, kv_len, chunk_off, B, total_chunks, h, h_kv, page_size, max_pages, scale, part_ml, part_acc, s);
    else decode_r<0, 64>(R, nw, q, k_pool, v_pool, block_table, kv_len, chunk_off, B, total_chunks, h, h_kv, page_size, max_pages, scale, part_ml, part_acc, s);
  }
  return launched("bi_decode_attn");
}

extern "C" bi_status bi_merge_partials(const float* part_ml, const float* part_acc,
                                       const int32_t* chunk_off, int B, int h, int d_h,
                                       void* out, int out_dtype, bi_stream stream) {
  using namespace bi;
  BI_REQUIRE(B >= 0 && h >= 1, BI_ERR_INVALID, "bi_merge_partials: bad sizes B=%d h=%d", B, h);
  BI_REQUIRE(d_h == 64 || d_h == 128, BI_ERR_UNSUPPORTED, "bi_merge_partials: d_h=%d", d_h);
  BI_REQUIRE(out_dtype == BI_F32 || out_dtype == BI_BF16, BI_ERR_UNSUPPORTED,
             "bi_merge_partials: dtype %d", out_dtype);
  if (B == 0) return BI_OK;
  BI_REQUIRE(part_ml && part_acc && chunk_off && out, BI_ERR_INVALID,
             "bi_merge_partials: null pointer");
  BI_REQUIRE((long)B * h <= 0x7fffffffL, BI_ERR_INVALID, "bi_merge_partials: too large");
  hipStream_t s = as_stream(stream);
  const dim3 grid((unsigned)(((long)B * h + 3) / 4));
  if (d_h == 128) {
    if (out_dtype == BI_BF16) hipLaunchKernelGGL((k_merge<128, 1>), grid, dim3(256), 0, s, part_ml, part_acc, chunk_off, B, h, out);
    else hipLaunchKernelGGL((k_merge<128, 0>), grid, dim3(256), 0, s, part_ml, part_acc, chunk_off, B, h, out);
  } else {
    if (out_dtype == BI_BF16) hipLaunchKernelGGL((k_merge<64, 1>), grid, dim3(256), 0, s, part_ml, part_acc, chunk_off, B, h, out);
    else hipLaunchKernelGGL((k_merge<64, 0>), grid, dim3(256), 0, s, part_ml, part_acc, chunk_off, B, h, out);
  }
  return launched("bi_merge_partials");
}

// ---------------------------------------------------------------------------
// decode attention that allocates nothing: partials in a static device buffer
// ---------------------------------------------------------------------------

namespace bi {
namespace {

// Scratch of bi_decode_attn_noalloc: the fp32 partials (m, l) then acc.  One
// copy per GPU, held from the library's load on that GPU to the end of the
// process; every call on a GPU reuses it.  In host code `scratch` is only a
// stand-in for the device symbol: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) unsigned char scratch[BI_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up on first use there).
bi_status scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(BI_ERR_HIP, "bi_decode_attn_noalloc: hipGetDevice: %s",
                                   hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(BI_ERR_UNSUPPORTED, "bi_decode_attn_noalloc: device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(BI_ERR_HIP, "bi_decode_attn_noalloc: hipGetSymbolAddress: %s",
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BI_OK;
}

}  // namespace
}  // namespace bi

extern "C" bi_status bi_decode_attn_noalloc(const void* q, const void* k_pool,
                                            const void* v_pool, const int32_t* block_table,
                                            const int32_t* kv_len, const int32_t* chunk_off,
                                            int B, int total_chunks, int h, int h_kv, int d_h,
                                            int page_size, int max_pages, int kv_chunk,
                                            float scale, int dtype, void* out, int out_dtype,
                                            bi_stream stream) {
  using namespace bi;
  bi_status st = AttnArgsCheck::common("bi_decode_attn_noalloc", h, h_kv, d_h, page_size,
                                       kv_chunk, dtype);
  if (st != BI_OK) return st;
  BI_REQUIRE(out_dtype == BI_F32 || out_dtype == BI_BF16, BI_ERR_UNSUPPORTED,
             "bi_decode_attn_noalloc: out dtype %d", out_dtype);
  BI_REQUIRE(B >= 0 && total_chunks >= 0, BI_ERR_INVALID,
             "bi_decode_attn_noalloc: bad sizes B=%d total_chunks=%d", B, total_chunks);
  if (B == 0 || total_chunks == 0) return BI_OK;
  const size_t ml_bytes = (size_t)total_chunks * h * 2 * sizeof(float);
  const size_t acc_off = (ml_bytes + 255) & ~(size_t)255;
  const size_t need = acc_off + (size_t)total_chunks * h * d_h * sizeof(float);
  BI_REQUIRE(need <= (size_t)BI_NOALLOC_SCRATCH_BYTES, BI_ERR_WORKSPACE,
             "bi_decode_attn_noalloc: %zu bytes of partials exceed the %d-byte static buffer "
             "(total_chunks=%d h=%d d_h=%d)", need, (int)BI_NOALLOC_SCRATCH_BYTES,
             total_chunks, h, d_h);
  BI_REQUIRE(out != nullptr, BI_ERR_INVALID, "bi_decode_attn_noalloc: null pointer");
  void* base = nullptr;
  st = scratch_on_current_device(&base);
  if (st != BI_OK) return st;
  float* part_ml = static_cast<float*>(base);
  float* part_acc = reinterpret_cast<float*>(static_cast<unsigned char*>(base) + acc_off);
  st = bi_decode_attn(q, k_pool, v_pool, block_table, kv_len, chunk_off, B, total_chunks, h,
                      h_kv, d_h, page_size, max_pages, kv_chunk, scale, dtype, part_ml,
                      part_acc, stream);
  if (st != BI_OK) return st;
  return bi_merge_partials(part_ml, part_acc, chunk_off, B, h, d_h, out, out_dtype, stream);
}

// ---------------------------------------------------------------------------
// batch-adaptive twins
// ---------------------------------------------------------------------------

extern "C" size_t bi_decode_attn_free_workspace_bytes(int B, int h, int d_h, int max_kv_len) {
  if (B < 0 || h <= 0 || d_h <= 0 || max_kv_len <= 0) return 0;
  const int a = (max_kv_len + 255) / 256;
  const long stride = a > 64 ? a : 64;
  return (size_t)B * stride * h * ((size_t)d_h + 2) * sizeof(float);
}

extern "C" bi_status bi_decode_attn_free(const void* q, const void* k_pool, const void* v_pool,
                                         const int32_t* block_table, const int32_t* kv_len, int B,
                                         int max_kv_len, int h, int h_kv, int d_h, int page_size,
                                         int max_pages, float scale, int dtype, void* workspace,
                                         size_t workspace_bytes, void* out, bi_stream stream) {
  using namespace bi;
  bi_status st = AttnArgsCheck::common("bi_decode_attn_free", h, h_kv, d_h, page_size, 256,
                                       dtype);
  if (st != BI_OK) return st;
  BI_REQUIRE(B >= 0 && max_kv_len >= 1 && max_pages >= 1, BI_ERR_INVALID,
             "bi_decode_attn_free: bad sizes");
  if (B == 0) return BI_OK;
  BI_REQUIRE(q && k_pool && v_pool && block_table && kv_len && workspace && out, BI_ERR_INVALID,
             "bi_decode_attn_free: null pointer");
  const size_t need = bi_decode_attn_free_workspace_bytes(B, h, d_h, max_kv_len);
  BI_REQUIRE(workspace_bytes >= need, BI_ERR_WORKSPACE,
             "bi_decode_attn_free: workspace %zu < %zu bytes", workspace_bytes, need);
  const FreePolicy pol = free_policy(B, h, h_kv, max_kv_len);
  BI_REQUIRE((long)B * pol.stride <= 0x7fffffffL, BI_ERR_INVALID, "bi_decode_attn_free: grid");
  // the workspace query's bound (ceil(max/256) or 64 splits) covers pol.stride
  BI_REQUIRE(pol.stride <= ((max_kv_len + 255) / 256 > 64 ? (max_kv_len + 255) / 256 : 64),
             BI_ERR_INVALID, "bi_decode_attn_free: split policy exceeds its bound");
  float* ml = static_cast<float*>(workspace);
  float* acc = ml + (size_t)B * pol.stride * h * 2;
  hipStream_t s = as_stream(stream);
  const int R = h / h_kv;
#define BI_DF(dt, dh)                                                                         \
  do {                                                                                        \
    if (R == 2) launch_decode_free<dt, dh, 2>(q, k_pool, v_pool, block_table, kv_len, B, h,  \
                                              h_kv, max_pages, scale, pol, ml, acc, s);      \
    else launch_decode_free<dt, dh, 4>(q, k_pool, v_pool, block_table, kv_len, B, h, h_kv,   \
                                       max_pages, scale, pol, ml, acc, s);                   \
  } while (0)
  if (dtype == BI_BF16) { if (d_h == 128) BI_DF(1, 128); else BI_DF(1, 64); }
  else { if (d_h == 128) BI_DF(0, 128); else BI_DF(0, 64); }
#undef BI_DF
  st = launched("bi_decode_attn_free");
  if (st != BI_OK) return st;
  const dim3 grid((unsigned)(((long)B * h + 3) / 4));
#define BI_MF(dh, od)                                                                          \
  hipLaunchKernelGGL((k_merge<dh, od, true>), grid, dim3(256), 0, s, ml, acc, nullptr, B, h,  \
                     out, kv_len, pol.chunk2, pol.stride)
  if (d_h == 128) { if (dtype == BI_BF16) BI_MF(128, 1); else BI_MF(128, 0); }
  else { if (dtype == BI_BF16) BI_MF(64, 1); else BI_MF(64, 0); }
#undef BI_MF
  return launched("bi_decode_attn_free");
}

extern "C" bi_status bi_merge_partials_free(const float* part_ml, const float* part_acc,
                                            const int32_t* chunk_off, int B, int h, int d_h,
                                            void* out, int out_dtype, bi_stream stream) {
  using namespace bi;
  BI_REQUIRE(B >= 0 && h >= 1, BI_ERR_INVALID, "bi_merge_partials_free: bad sizes");
  BI_REQUIRE(d_h == 64 || d_h == 128, BI_ERR_UNSUPPORTED, "bi_merge_partials_free: d_h=%d", d_h);
  BI_REQUIRE(out_dtype == BI_F32 || out_dtype == BI_BF16, BI_ERR_UNSUPPORTED,
             "bi_merge_partials_free: dtype %d", out_dtype);
  if (B == 0) return BI_OK;
  BI_REQUIRE(part_ml && part_acc && chunk_off && out, BI_ERR_INVALID,
             "bi_merge_partials_free: null pointer");
  hipStream_t s = as_stream(stream);
  const dim3 grid((unsigned)(((long)B * h + 3) / 4));
  if (d_h == 128) {
    if (out_dtype == BI_BF16) hipLaunchKernelGGL((k_merge<128, 1, true>), grid, dim3(256), 0, s, part_ml, part_acc, chunk_off, B, h, out, nullptr, 0, 0);
    else hipLaunchKernelGGL((k_merge<128, 0, true>), grid, dim3(256), 0, s, part_ml, part_acc, chunk_off, B, h, out, nullptr, 0, 0);
  } else {
    if (out_dtype == BI_BF16) hipLaunchKernelGGL((k_merge<64, 1, true>), grid, dim3(256), 0, s, part_ml, part_acc, chunk_off, B, h, out, nullptr, 0, 0);
    else hipLaunchKernelGGL((k_merge<64, 0, true>), grid, dim3(256), 0, s, part_ml, part_acc, chunk_off, B, h, out, nullptr, 0, 0);
  }
  return launched("bi_merge_partials_free");
}

extern "C" bi_status bi_prefill_attn_free(const void* q, const int32_t* q_start,
                                          const int32_t* q_pos0, int R, int T, const void* k_pool,
                                          const void* v_pool, const int32_t* block_table, int h,
                                          int h_kv, int d_h, int page_size, int max_pages,
                                          float scale, int dtype, void* out, bi_stream stream) {
  using namespace bi;
  // chunk length from the amount of work: short chunks when the grid is small
  const long wgs = ((long)T / kPrefillQB + R) * h_kv;
  const int chunk = wgs < 256 ? 64 : 256;
  bi_status st = AttnArgsCheck::common("bi_prefill_attn_free", h, h_kv, d_h, page_size, chunk,
                                       dtype);
  if (st != BI_OK) return st;
  BI_REQUIRE(R >= 0 && T >= 0 && max_pages >= 1, BI_ERR_INVALID,
             "bi_prefill_attn_free: bad sizes");
  if (R == 0 || T == 0) return BI_OK;
  BI_REQUIRE(q && q_start && q_pos0 && k_pool && v_pool && block_table && out, BI_ERR_INVALID,
             "bi_prefill_attn_free: null pointer");
  const int Rg = h / h_kv, nw = chunk / 64;
  hipStream_t s = as_stream(stream);
  if (dtype == BI_BF16) {
    if (d_h == 128) prefill_r<1, 128, true>(Rg, nw, q, q_start, q_pos0, R, T, k_pool, v_pool, block_table, h, h_kv, page_size, max_pages, scale, out, s);
    else prefill_r<1, 64, true>(Rg, nw, q, q_start, q_pos0, R, T, k_pool, v_pool, block_table, h, h_kv, page_size, max_pages, scale, out, s);
  } else {
    if (d_h == 128) prefill_r<0, 128, true>(Rg, nw, q, q_start, q_pos0, R, T, k_pool, v_pool, block_table, h, h_kv, page_size, max_pages, scale, out, s);
    else prefill_r<0, 64, true>(Rg, nw, q, q_start, q_pos0, R, T, k_pool, v_pool, block_table, h, h_kv, page_size, max_pages, scale, out, s);
  }
  return launched("bi_prefill_attn_free");
}
