// bi_gemm: C = A W^T with one fixed K chain per output element.
//
// "Batch invariance and reproducible inference", "2 . Cross-block
// accumulation": split-K leaves the order to whichever block lands first,
// and the replacement matmul accumulates its K loop in one fixed order per
// output tile; "3 . Kernel selection changing with shape": a tile choice
// that follows M changes the tree.  Here every bf16 output element is the
// chain  acc = 0; for kt = 0 .. ceil(K/32)-1: acc = mfma16x16x32(A_kt, W_kt,
// acc)  with A in the MFMA A operand and W in the B operand and the same
// k -> lane assignment, in every kernel.  The kernels differ only in how
// they tile M and N (chosen from M and N), which moves no rounding: an
// MFMA output row does not depend on the other rows of its tile.
//
// Operand "fragments": 64 lanes x 16 bytes; lane l holds 8 consecutive k of
// row (l % 16) at offset 8 * (l / 16) inside the 32-wide K-tile -- exactly
// the operand layout of v_mfma_f32_16x16x32_bf16, so a fragment copied to
// LDS by one direct global->LDS instruction is read back by the same lane
// with one conflict-free ds_read_b128.
#include "api.h"
#include "common.h"

namespace bi {

constexpr int kFrag = 1024;  // bytes per operand fragment

__device__ __forceinline__ f32x4_t mfma(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return mfma16(a, b, c);
}

// OUTF32: 0 = bf16 store, 1 = fp32 store, 2 = fp32 atomic add (split-K twin)
template <int OUTF32>
__device__ __forceinline__ void store_tile(void* C, const f32x4_t& acc, int row0, int col0, int M,
                                           int N, int lane) {
  const int col = col0 + (lane & 15);
  if (col >= N) return;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = row0 + 4 * (lane >> 4) + j;
    if (row < M) {
      const long idx = (long)row * N + col;
      if (OUTF32 == 2)
        atomicAdd(static_cast<float*>(C) + idx, acc[j]);
      else if (OUTF32 == 1)
        static_cast<float*>(C)[idx] = acc[j];
      else
        static_cast<uint16_t*>(C)[idx] = (uint16_t)f32_to_bf16_bits(acc[j]);
    }
  }
}

// The small-M kernels split roles across waves.  Copy waves only issue
// direct global->LDS copies of the operand the whole workgroup shares, into
// an NS-slot ring; compute waves only issue register loads of their private
// operand and run the MFMAs.  A wave's memory counter then tracks one kind of
// operation, so copy waves can keep many stages in flight while compute waves
// wait exactly for their own loads.  Copy and compute waves run separate
// loops with the same barrier sequence (one s_barrier per stage): after the
// barrier of stage st, stage st is in LDS and the slot of stage st-1 is free.
// With K known at compile time the loops unroll into straight-line code.
constexpr int kCopyWaves = 4;

// ---------------------------------------------------------------------------
// wide kernel (M <= 64, large N): 4 compute waves, each owning one 16-column
// strip of W (64 columns per workgroup) and all MT row tiles; W streams into
// a ring of RING stages of registers.  A (shared) goes through the LDS ring.
// ---------------------------------------------------------------------------
template <int MT, int OUTF32, int NSTC>
__global__ __launch_bounds__(512) void k_gemm_wide(const uint16_t* __restrict__ A,
                                                   const uint16_t* __restrict__ W, void* C,
                                                   int M, int N, int Ktot, int kslice) {
  // K slice of this workgroup (one slice covering all of K on the invariant
  // path; the split-K twin launches several along y).  Rows keep stride Ktot.
  const int kbeg = blockIdx.y * kslice;
  const int K = min(kslice, Ktot - kbeg);
  const long ld = Ktot;
  A += kbeg;
  W += kbeg;
  constexpr int KTS = 4, NS = 4, RING = 4;
  constexpr int SLOT = 16 * kFrag;           // room for MT * KTS <= 16 fragments
  constexpr int QA = MT * KTS / kCopyWaves;  // copies per copy wave per stage
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int lrow = lane & 15, lk = (lane >> 4) * 8;
  const int KT = (K + 31) >> 5;
  const int NST = NSTC > 0 ? NSTC : (KT + KTS - 1) / KTS;

  if (wave >= 4) {
    // ---- copy waves: A stages into the ring
    const int cw = wave - 4;
    auto issue_a = [&](int st) {
      char* slot = smem + (st % NS) * SLOT;
#pragma unroll
      for (int i = 0; i < QA; ++i) {
        const int f = cw + kCopyWaves * i;  // fragment (mt, kt) = divmod(f, KTS)
        int kk = (st * KTS + f % KTS) * 32 + lk;
        if (NSTC == 0) kk = kk < K ? kk : 0;
        dma16(A + (long)min((f / KTS) * 16 + lrow, M - 1) * ld + kk, slot + f * kFrag);
      }
    };
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
      if (s < NST) issue_a(s);
    auto step = [&](int st, bool steady) {
      if (steady) BI_WAIT_VMCNT((NS - 2) * QA); else BI_WAIT_VMCNT(0);
      __builtin_amdgcn_s_barrier();
      if (st + NS - 1 < NST) issue_a(st + NS - 1);
    };
    if constexpr (NSTC > 0) {
#pragma unroll
      for (int st = 0; st < NSTC; ++st) step(st, st + NS - 1 <= NSTC);
    } else {
      for (int st = 0; st < NST; ++st) step(st, st + NS - 1 <= NST);
    }
    return;
  }

  // ---- compute waves
  const int ntile = blockIdx.x * 4 + wave;
  const uint16_t* wrow = W + (long)min(ntile * 16 + lrow, N - 1) * ld;
  auto load_w = [&](int st, u32x4_t (&dst)[KTS]) {
    const int stc = st < NST ? st : NST - 1;
#pragma unroll
    for (int kt = 0; kt < KTS; ++kt) {
      int kk = (stc * KTS + kt) * 32 + lk;
      if (NSTC == 0) kk = kk < K ? kk : 0;
      dst[kt] = *reinterpret_cast<const u32x4_t*>(wrow + kk);
    }
  };
  u32x4_t wreg[RING][KTS];
  f32x4_t acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < RING; ++r) load_w(r, wreg[r]);
  const uint32_t lds0 = lds_addr(smem) + lane * 16;
  auto step = [&](int st, int j, bool guarded, bool refill) {
    __builtin_amdgcn_s_barrier();
    const uint32_t slot = lds0 + (st % NS) * SLOT;
    u32x4_t a0[8], a1[8];
    lds_read_8x2_stride1k(a0, a1, slot, slot + 8 * kFrag);
#pragma unroll
    for (int kt = 0; kt < KTS; ++kt) {
      const int ktg = st * KTS + kt;
      if (!guarded || ktg < KT) {
        const bool tail = guarded && ktg * 32 + lk >= K;
        const u32x4_t z = u32x4_t{0, 0, 0, 0};
        const u32x4_t b = tail ? z : wreg[j][kt];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const int f = m * KTS + kt;
          const u32x4_t a = tail ? z : (f < 8 ? a0[f & 7] : a1[f & 7]);
          acc[m] = mfma(a, b, acc[m]);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (refill) load_w(st + RING, wreg[j]);
    __builtin_amdgcn_sched_barrier(0);
  };
  if constexpr (NSTC > 0) {
#pragma unroll
    for (int st = 0; st < NSTC; ++st) step(st, st % RING, false, st + RING < NSTC);
  } else {
    const int NMAIN = ((KT / KTS) / RING) * RING;  // full stages, whole ring turns
    for (int st0 = 0; st0 < NMAIN; st0 += RING) {
#pragma unroll
      for (int j = 0; j < RING; ++j) step(st0 + j, j, false, true);
    }
#pragma unroll
    for (int j = 0; j < RING; ++j)
      if (NMAIN + j < NST) step(NMAIN + j, j, true, false);
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) store_tile<OUTF32>(C, acc[m], m * 16, ntile * 16, M, N, lane);
}

// ---------------------------------------------------------------------------
// narrow kernel (M <= 64, N up to a few thousand): one 16-column strip of W
// per workgroup, shared through a deep LDS ring filled by the copy waves;
// compute wave w owns row tile w and streams its A fragments into registers.
// ---------------------------------------------------------------------------
template <int MT, int OUTF32, int NSTC>
__global__ __launch_bounds__((MT + kCopyWaves) * 64) void k_gemm_narrow(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W, void* C, int M, int N,
    int Ktot, int kslice) {
  const int kbeg = blockIdx.y * kslice;
  const int K = min(kslice, Ktot - kbeg);
  const long ld = Ktot;
  A += kbeg;
  W += kbeg;
  constexpr int KTS = 8, NS = 16, RING = 4;
  constexpr int SLOT = KTS * kFrag;
  constexpr int QW = KTS / kCopyWaves;  // copies per copy wave per stage
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n0 = blockIdx.x * 16;
  const int lrow = lane & 15, lk = (lane >> 4) * 8;
  const int KT = (K + 31) >> 5;
  const int NST = NSTC > 0 ? NSTC : (KT + KTS - 1) / KTS;

  if (wave >= MT) {
    // ---- copy waves: W stages into the ring
    const int cw = wave - MT;
    const uint16_t* wrow = W + (long)min(n0 + lrow, N - 1) * ld;
    auto issue_w = [&](int st) {
      char* slot = smem + (st % NS) * SLOT;
#pragma unroll
      for (int i = 0; i < QW; ++i) {
        const int kt = cw + kCopyWaves * i;
        int kk = (st * KTS + kt) * 32 + lk;
        if (NSTC == 0) kk = kk < K ? kk : 0;
        dma16(wrow + kk, slot + kt * kFrag);
      }
    };
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
      if (s < NST) issue_w(s);
    auto step = [&](int st, bool steady) {
      if (steady) BI_WAIT_VMCNT((NS - 2) * QW); else BI_WAIT_VMCNT(0);
      __builtin_amdgcn_s_barrier();
      if (st + NS - 1 < NST) issue_w(st + NS - 1);
    };
    if constexpr (NSTC > 0) {
#pragma unroll
      for (int st = 0; st < NSTC; ++st) step(st, st + NS - 1 <= NSTC);
    } else {
      for (int st = 0; st < NST; ++st) step(st, st + NS - 1 <= NST);
    }
    return;
  }

  // ---- compute waves
  const uint16_t* arow = A + (long)min(wave * 16 + lrow, M - 1) * ld;
  auto load_a = [&](int st, u32x4_t (&dst)[KTS]) {
    const int stc = st < NST ? st : NST - 1;
#pragma unroll
    for (int kt = 0; kt < KTS; ++kt) {
      int kk = (stc * KTS + kt) * 32 + lk;
      if (NSTC == 0) kk = kk < K ? kk : 0;
      dst[kt] = *reinterpret_cast<const u32x4_t*>(arow + kk);
    }
  };
  u32x4_t areg[RING][KTS];
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < RING; ++r) load_a(r, areg[r]);
  const uint32_t lds0 = lds_addr(smem) + lane * 16;
  auto step = [&](int st, int j, bool guarded, bool refill) {
    __builtin_amdgcn_s_barrier();
    u32x4_t b[8];
    lds_read_8_stride1k(b, lds0 + (st % NS) * SLOT);
#pragma unroll
    for (int kt = 0; kt < KTS; ++kt) {
      const int ktg = st * KTS + kt;
      if (!guarded || ktg < KT) {
        const bool tail = guarded && ktg * 32 + lk >= K;
        const u32x4_t z = u32x4_t{0, 0, 0, 0};
        acc = mfma(tail ? z : areg[j][kt], tail ? z : b[kt], acc);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (refill) load_a(st + RING, areg[j]);
    __builtin_amdgcn_sched_barrier(0);
  };
  if constexpr (NSTC > 0) {
#pragma unroll
    for (int st = 0; st < NSTC; ++st) step(st, st % RING, false, st + RING < NSTC);
  } else {
    const int NMAIN = ((KT / KTS) / RING) * RING;
    for (int st0 = 0; st0 < NMAIN; st0 += RING) {
#pragma unroll
      for (int j = 0; j < RING; ++j) step(st0 + j, j, false, true);
    }
#pragma unroll
    for (int j = 0; j < RING; ++j)
      if (NMAIN + j < NST) step(NMAIN + j, j, true, false);
  }
  store_tile<OUTF32>(C, acc, wave * 16, n0, M, N, lane);
}

// ---------------------------------------------------------------------------
// tiled kernel: 128 x 128 output tile per workgroup, 4 waves in 2 x 2, each
// 64 x 64 (4 x 4 MFMA tiles).  Stages of 2 K-tiles through NS LDS slots.
// ---------------------------------------------------------------------------
template <int OUTF32>
__global__ __launch_bounds__(256) void k_gemm_tiled(const uint16_t* __restrict__ A,
                                                    const uint16_t* __restrict__ W, void* C,
                                                    int M, int N, int K, int tiles_n) {
  constexpr int NS = 2;
  constexpr int KTS = 2;
  constexpr int AFR = 8 * KTS, FPS = 16 * KTS;  // A fragments first, then W
  constexpr int PER_WAVE = FPS / 4;
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * 128, n0 = tn * 128;
  const int wm = wave >> 1, wn = wave & 1;
  const int KT = (K + 31) >> 5;
  const int NST = (KT + KTS - 1) / KTS;
  const int lrow = lane & 15, lk = (lane >> 4) * 8;

  auto issue = [&](int st) {
    char* slot = smem + (st % NS) * FPS * kFrag;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int f = wave + 4 * i;
      const int g = f < AFR ? f : f - AFR;
      const int tile = g / KTS, kt = g % KTS;
      int kk = (st * KTS + kt) * 32 + lk;
      kk = kk < K ? kk : 0;
      const uint16_t* src;
      if (f < AFR)
        src = A + (long)min(m0 + tile * 16 + lrow, M - 1) * K + kk;
      else
        src = W + (long)min(n0 + tile * 16 + lrow, N - 1) * K + kk;
      dma16(src, slot + f * kFrag);
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < NST) issue(s);

  const uint32_t lds0 = lds_addr(smem) + lane * 16;
  for (int st = 0; st < NST; ++st) {
    if (st + NS - 1 <= NST)
      BI_WAIT_VMCNT(PER_WAVE * (NS - 2));
    else
      BI_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
    if (st + NS - 1 < NST) issue(st + NS - 1);
    const uint32_t slot = lds0 + (st % NS) * FPS * kFrag;
#pragma unroll
    for (int kt = 0; kt < KTS; ++kt) {
      const int ktg = st * KTS + kt;
      if (ktg < KT) {
        static_assert(KTS == 2, "fragment stride 2 KiB");
        u32x4_t a[4], b[4];
        lds_read_4x2_stride2k(a, b, slot + (4 * wm * KTS + kt) * kFrag,
                              slot + (AFR + 4 * wn * KTS + kt) * kFrag);
        if (ktg * 32 + lk >= K) {
#pragma unroll
          for (int i = 0; i < 4; ++i) a[i] = b[i] = u32x4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma(a[i], b[j], acc[i][j]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      store_tile<OUTF32>(C, acc[i][j], m0 + (4 * wm + i) * 16, n0 + (4 * wn + j) * 16, M, N, lane);
}

// ---------------------------------------------------------------------------
// fp32: one thread per output element, serial fma chain over k ascending.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gemm_f32(const float* __restrict__ A,
                                                  const float* __restrict__ W,
                                                  float* __restrict__ C, int M, int N, int K) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)M * N) return;
  const int i = (int)(idx / N), j = (int)(idx % N);
  const float* a = A + (long)i * K;
  const float* w = W + (long)j * K;
  float acc = 0.0f;
  for (int k = 0; k < K; ++k) acc = __builtin_fmaf(a[k], w[k], acc);
  C[idx] = acc;
}

// ---------------------------------------------------------------------------
// launch plumbing
// ---------------------------------------------------------------------------
template <int MT, int OUTF32, int NSTC>
static void launch_wide_k(const void* A, const void* W, void* C, int M, int N, int K,
                          hipStream_t s, int splits = 1, int kslice = 0) {
  if (splits == 1) kslice = K;
  constexpr int lds = 4 * 16 * kFrag;
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)k_gemm_wide<MT, OUTF32, NSTC>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    attr = true;
  }
  hipLaunchKernelGGL((k_gemm_wide<MT, OUTF32, NSTC>), dim3((N + 63) / 64, splits), dim3(512),
                     lds, s, (const uint16_t*)A, (const uint16_t*)W, C, M, N, K, kslice);
}

// K = 4096 runs a fully unrolled pipeline (4 K-tiles per stage)
template <int MT, int OUTF32>
static void launch_wide(const void* A, const void* W, void* C, int M, int N, int K,
                        hipStream_t s) {
  if (K == 4096) launch_wide_k<MT, OUTF32, 32>(A, W, C, M, N, K, s);
  else launch_wide_k<MT, OUTF32, 0>(A, W, C, M, N, K, s);
}

template <int MT, int OUTF32, int NSTC>
static void launch_narrow_k(const void* A, const void* W, void* C, int M, int N, int K,
                            hipStream_t s, int splits = 1, int kslice = 0) {
  if (splits == 1) kslice = K;
  constexpr int lds = 16 * 8 * kFrag;
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)k_gemm_narrow<MT, OUTF32, NSTC>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    attr = true;
  }
  hipLaunchKernelGGL((k_gemm_narrow<MT, OUTF32, NSTC>), dim3((N + 15) / 16, splits),
                     dim3((MT + kCopyWaves) * 64), lds, s,
                     (const uint16_t*)A, (const uint16_t*)W, C, M, N, K, kslice);
}

// K = 4096 and K = 14336 run fully unrolled pipelines (8 K-tiles per stage)
template <int MT, int OUTF32>
static void launch_narrow(const void* A, const void* W, void* C, int M, int N, int K,
                          hipStream_t s) {
  if (K == 4096) launch_narrow_k<MT, OUTF32, 16>(A, W, C, M, N, K, s);
  else if (K == 14336) launch_narrow_k<MT, OUTF32, 56>(A, W, C, M, N, K, s);
  else launch_narrow_k<MT, OUTF32, 0>(A, W, C, M, N, K, s);
}

// Small M: wide strips (A shared through LDS) when N offers >= 256
// workgroups of 64 columns, else one strip of 16 columns per workgroup.
template <int OUTF32>
static void dispatch_skinny(const void* A, const void* W, void* C, int M, int N, int K,
                            hipStream_t s) {
  const int MT = (M + 15) / 16;
  const bool wide = N >= 64 * 256;
#define BI_SKINNY(mt)                                                   \
  if (MT == mt) {                                                       \
    if (wide) launch_wide<mt, OUTF32>(A, W, C, M, N, K, s);             \
    else launch_narrow<mt, OUTF32>(A, W, C, M, N, K, s);                \
    return;                                                             \
  }
  BI_SKINNY(1) BI_SKINNY(2) BI_SKINNY(3) BI_SKINNY(4)
#undef BI_SKINNY
}

template <int OUTF32>
static void launch_tiled(const void* A, const void* W, void* C, int M, int N, int K,
                         hipStream_t s) {
  constexpr size_t lds = 2 * 32 * kFrag;
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)k_gemm_tiled<OUTF32>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    attr = true;
  }
  const int tiles_m = (M + 127) / 128, tiles_n = (N + 127) / 128;
  hipLaunchKernelGGL((k_gemm_tiled<OUTF32>), dim3(tiles_m * tiles_n), dim3(256), lds, s,
                     (const uint16_t*)A, (const uint16_t*)W, C, M, N, K, tiles_n);
}

// ---------------------------------------------------------------------------
// large tiles for large M (chunked prefill): 256 x 256 output tile per
// workgroup, 8 waves as 2 (M) x 4 (N), each 128 x 64 (8 x 4 MFMA tiles).
// Two K-tiles per stage, two stages of A and W rows in LDS by direct copies
// of whole 128-byte lines.  Same MFMA chain per output element as every
// other path.  Workgroups are mapped so that each XCD (blockIdx % 8) takes a
// contiguous range of tiles in grouped order (4 row-blocks at a time), so
// the tiles resident on one XCD share A rows and W columns in its L2.
// ---------------------------------------------------------------------------
template <int OUTF32>
__global__ __launch_bounds__(512) void k_gemm_big(const uint16_t* __restrict__ A,
                                                  const uint16_t* __restrict__ W, void* C,
                                                  int M, int N, int K, int tiles_m, int tiles_n) {
  // Stage = 2 K-tiles (64 columns of K = one 128-byte line per row).  LDS
  // stage layout is line-major: A rows 0..255 then W rows 0..255, 8 rows
  // (8 lines) per 1 KiB block; the 16-byte unit u of row r sits at slot
  // u ^ (r & 7).  Each direct copy moves 8 whole lines (128-byte requests);
  // a fragment (16 rows x 32 K) is read back with per-lane addresses.
  constexpr int NS = 2, BLK = 64, PER_WAVE = BLK / 8;  // 1 KiB blocks per stage
  constexpr int STAGE = BLK * 1024;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int nt = tiles_m * tiles_n, b = blockIdx.x;
  const int xcd = b % 8, idx = b / 8;
  const int per = nt / 8, rem = nt % 8;
  const int t = xcd * per + (xcd < rem ? xcd : rem) + idx;
  // grouped order inside that range: GM row-blocks at a time, row fastest,
  // so the XCD's resident workgroups form a GM x (32 / GM) block of tiles
  // sharing A rows and W columns in its L2
  constexpr int GM = 4;
  const int grp = t / (GM * tiles_n), first = grp * GM;
  const int gm = min(GM, tiles_m - first);
  const int tm = first + (t % (GM * tiles_n)) % gm, tn = (t % (GM * tiles_n)) / gm;
  const int m0 = tm * 256, n0 = tn * 256;
  const int wm = wave >> 2, wn = wave & 3;
  const int KT = (K + 31) >> 5;
  const int NST = (KT + 1) >> 1;

  // copy lane: row (lane >> 3) of its block, slot (lane & 7) holds unit
  // slot ^ (row & 7) of that row's 128-byte span
  const int crow = lane >> 3, cunit = (lane & 7) ^ crow;
  auto issue = [&](int st) {
    char* slot = smem + (st % NS) * STAGE;
    int kk = st * 64 + cunit * 8;
    kk = kk < K ? kk : 0;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int blk = wave + 8 * i;  // 0..31 A row blocks, 32..63 W row blocks
      const uint16_t* src = blk < 32
          ? A + (long)min(m0 + blk * 8 + crow, M - 1) * K + kk
          : W + (long)min(n0 + (blk - 32) * 8 + crow, N - 1) * K + kk;
      dma16(src, slot + blk * 1024);
    }
  };
  // read lane: row (lane & 15) of a 16-row tile, unit 4 kt + (lane >> 4)
  auto rd_off = [&](int kt) {
    const int r = lane & 15, u = 4 * kt + (lane >> 4);
    return (uint32_t)(((r >> 3) & 1) * 1024 + (r & 7) * 128 + 16 * (u ^ (r & 7)));
  };
  const uint32_t off0 = rd_off(0), off1 = rd_off(1);

  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  issue(0);
  const uint32_t lds0 = lds_addr(smem);
  for (int st = 0; st < NST; ++st) {
    BI_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
    if (st + 1 < NST) issue(st + 1);
    const uint32_t sb = lds0 + (st % NS) * STAGE;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int ktg = 2 * st + kt;
      if (ktg < KT) {
        const uint32_t off = kt ? off1 : off0;
        u32x4_t a[8], bw[4];
        // A row tiles 8 wm .. 8 wm + 7 (tile t at blocks 2t, 2t + 1: stride
        // 2 KiB), W column tiles 4 wn .. 4 wn + 3
        lds_read_8_stride2k(a, sb + (8 * wm) * 2048 + off);
        lds_read_4_stride2k(bw, sb + 32 * 1024 + (4 * wn) * 2048 + off);
        if (ktg * 32 + 8 * (lane >> 4) >= K) {
#pragma unroll
          for (int i = 0; i < 8; ++i) a[i] = u32x4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma(a[i], bw[j], acc[i][j]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      store_tile<OUTF32>(C, acc[i][j], m0 + (8 * wm + i) * 16, n0 + (4 * wn + j) * 16, M, N,
                         lane);
}

template <int OUTF32>
static void launch_big(const void* A, const void* W, void* C, int M, int N, int K,
                       hipStream_t s) {
  constexpr size_t lds = 2 * 64 * 1024;
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)k_gemm_big<OUTF32>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    attr = true;
  }
  const int tiles_m = (M + 255) / 256, tiles_n = (N + 255) / 256;
  hipLaunchKernelGGL((k_gemm_big<OUTF32>), dim3(tiles_m * tiles_n), dim3(512), lds, s,
                     (const uint16_t*)A, (const uint16_t*)W, C, M, N, K, tiles_m, tiles_n);
}

// Split-K over `splits` workgroup slices of kslice (multiple of 32) columns of
// K, fp32 partial sums added atomically into C32 (which the caller zeroed).
// Used only by the batch-adaptive twin.
void gemm_splitk_atomic(const void* A, const void* W, float* C32, int M, int N, int K,
                        int splits, int kslice, hipStream_t s) {
  const int MT = (M + 15) / 16;
  const bool wide = N >= 64 * 256;
#define BI_SPLIT(mt)                                                                   \
  if (MT == mt) {                                                                      \
    if (wide) launch_wide_k<mt, 2, 0>(A, W, C32, M, N, K, s, splits, kslice);          \
    else launch_narrow_k<mt, 2, 0>(A, W, C32, M, N, K, s, splits, kslice);             \
    return;                                                                            \
  }
  BI_SPLIT(1) BI_SPLIT(2) BI_SPLIT(3) BI_SPLIT(4)
#undef BI_SPLIT
}

void gemm_dispatch(const void* A, const void* W, void* C, int M, int N, int K, int out_f32,
                   hipStream_t s) {
  if (M <= 64) {
    if (out_f32) dispatch_skinny<1>(A, W, C, M, N, K, s);
    else dispatch_skinny<0>(A, W, C, M, N, K, s);
  } else if (M >= 1024 && N >= 2048) {
    if (out_f32) launch_big<1>(A, W, C, M, N, K, s);
    else launch_big<0>(A, W, C, M, N, K, s);
  } else {
    if (out_f32) launch_tiled<1>(A, W, C, M, N, K, s);
    else launch_tiled<0>(A, W, C, M, N, K, s);
  }
}

}  // namespace bi

extern "C" bi_status bi_gemm(const void* A, const void* W, void* C, int M, int N, int K,
                             int in_dtype, int out_dtype, bi_stream stream) {
  using namespace bi;
  BI_REQUIRE(M >= 0 && N >= 1 && K >= 1, BI_ERR_INVALID, "bi_gemm: bad shape M=%d N=%d K=%d",
             M, N, K);
  BI_REQUIRE((in_dtype == BI_BF16 && (out_dtype == BI_BF16 || out_dtype == BI_F32)) ||
                 (in_dtype == BI_F32 && out_dtype == BI_F32),
             BI_ERR_UNSUPPORTED, "bi_gemm: dtype pair (%d, %d) not supported", in_dtype,
             out_dtype);
  if (M == 0) return BI_OK;
  BI_REQUIRE(A && W && C, BI_ERR_INVALID, "bi_gemm: null pointer");
  BI_REQUIRE(aligned16(A) && aligned16(W) && aligned16(C), BI_ERR_INVALID,
             "bi_gemm: pointers must be 16-byte aligned");
  BI_REQUIRE((long)M * N < (1L << 40) && (long)N * K < (1L << 40) && (long)M * K < (1L << 40),
             BI_ERR_INVALID, "bi_gemm: tensor too large");
  hipStream_t s = as_stream(stream);
  if (in_dtype == BI_F32) {
    const long total = (long)M * N;
    hipLaunchKernelGGL(k_gemm_f32, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       (const float*)A, (const float*)W, (float*)C, M, N, K);
    return launched("bi_gemm");
  }
  BI_REQUIRE(K % 8 == 0, BI_ERR_UNSUPPORTED, "bi_gemm: bf16 needs K %% 8 == 0 (K=%d)", K);
  gemm_dispatch(A, W, C, M, N, K, out_dtype == BI_F32, s);
  return launched("bi_gemm");
}
