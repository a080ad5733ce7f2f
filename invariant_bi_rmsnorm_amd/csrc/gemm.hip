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
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

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
      if (OUTF32)
        static_cast<float*>(C)[idx] = acc[j];
      else
        static_cast<uint16_t*>(C)[idx] = (uint16_t)f32_to_bf16_bits(acc[j]);
    }
  }
}

// ---------------------------------------------------------------------------
// skinny kernel: M <= 64 (MT row tiles), SB column tiles of 16 per workgroup.
// 4 waves stream stages of 8 K-tiles (256 k) of A and W through a ring of NS
// LDS slots with direct global->LDS copies; each (row tile, column tile)
// pair keeps one accumulator and walks the K-tiles in ascending order.
// ---------------------------------------------------------------------------
template <int MT, int SB, int NS, int OUTF32>
__global__ __launch_bounds__(256) void k_gemm_skinny(const uint16_t* __restrict__ A,
                                                     const uint16_t* __restrict__ W, void* C,
                                                     int M, int N, int K) {
  constexpr int KTS = 8;               // K-tiles per stage
  constexpr int WFR = SB * KTS;        // W fragments per stage
  constexpr int FPS = (SB + MT) * KTS; // fragments per stage
  constexpr int PER_WAVE = FPS / 4;    // copies each wave issues per stage
  constexpr int PAIRS = MT * SB;
  constexpr int PPW = (PAIRS + 3) / 4; // accumulators per wave
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = blockIdx.x * 16 * SB;
  const int KT = (K + 31) >> 5;
  const int NST = (KT + KTS - 1) / KTS;
  const int lrow = lane & 15, lk = (lane >> 4) * 8;

  auto issue = [&](int st) {
    char* slot = smem + (st % NS) * FPS * kFrag;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int f = wave + 4 * i;
      const int kt = (f < WFR ? f : f - WFR) % KTS;
      int kk = (st * KTS + kt) * 32 + lk;
      kk = kk < K ? kk : 0;
      const uint16_t* src;
      if (f < WFR) {
        const int n = min(n0 + (f / KTS) * 16 + lrow, N - 1);
        src = W + (long)n * K + kk;
      } else {
        const int m = min(((f - WFR) / KTS) * 16 + lrow, M - 1);
        src = A + (long)m * K + kk;
      }
      dma16(src, slot + f * kFrag);
    }
  };

  f32x4_t acc[PPW];
#pragma unroll
  for (int p = 0; p < PPW; ++p) acc[p] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // prologue: stages 0 .. NS-2 in flight
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < NST) issue(s);

  const uint32_t lds0 = lds_addr(smem) + lane * 16;
  for (int st = 0; st < NST; ++st) {
    // this wave's copies of stage st have landed (newer stages may still fly)
    if (st + NS - 1 <= NST)
      BI_WAIT_VMCNT(PER_WAVE * (NS - 2));
    else
      BI_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();  // all waves' copies landed; slot (st-1)%NS is free
    if (st + NS - 1 < NST) issue(st + NS - 1);
    const uint32_t slot = lds0 + (st % NS) * FPS * kFrag;
    const int kt_left = KT - st * KTS;  // K-tiles of this stage that exist
#pragma unroll
    for (int p = 0; p < PPW; ++p) {
      const int pair = wave + 4 * p;
      if (pair < PAIRS) {
        const int mt = pair / SB, sb = pair % SB;
        static_assert(KTS == 8, "stage = 8 K-tiles");
        u32x4_t a[KTS], b[KTS];
        lds_read_8x2_stride1k(a, b, slot + (WFR + mt * KTS) * kFrag, slot + sb * KTS * kFrag);
#pragma unroll
        for (int kt = 0; kt < KTS; ++kt) {
          if (kt < kt_left) {
            if ((st * KTS + kt) * 32 + lk >= K) a[kt] = b[kt] = u32x4_t{0, 0, 0, 0};
            acc[p] = mfma(a[kt], b[kt], acc[p]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int p = 0; p < PPW; ++p) {
    const int pair = wave + 4 * p;
    if (pair < PAIRS)
      store_tile<OUTF32>(C, acc[p], (pair / SB) * 16, n0 + (pair % SB) * 16, M, N, lane);
  }
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
template <int MT, int SB, int NS, int OUTF32>
static void launch_skinny(const void* A, const void* W, void* C, int M, int N, int K,
                          hipStream_t s) {
  constexpr size_t lds = (size_t)NS * (SB + MT) * 8 * kFrag;
  static_assert(lds <= 160 * 1024, "LDS budget");
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)k_gemm_skinny<MT, SB, NS, OUTF32>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    attr = true;
  }
  const int grid = (N + 16 * SB - 1) / (16 * SB);
  hipLaunchKernelGGL((k_gemm_skinny<MT, SB, NS, OUTF32>), dim3(grid), dim3(256), lds, s,
                     (const uint16_t*)A, (const uint16_t*)W, C, M, N, K);
}

// ring depth: as many 8-K-tile stages as fit in ~128 KiB, at most 6
constexpr int skinny_ns(int MT, int SB) {
  return (128 / (8 * (SB + MT))) > 6 ? 6 : (128 / (8 * (SB + MT)));
}

template <int OUTF32>
static void dispatch_skinny(const void* A, const void* W, void* C, int M, int N, int K,
                            hipStream_t s) {
  // column tiles per workgroup: widest that still gives >= 256 workgroups
  const int MT = (M + 15) / 16;
  const int sb = (N >= 4 * 16 * 256) ? 4 : (N >= 2 * 16 * 256) ? 2 : 1;
#define BI_SKINNY(mt, sbv)                                                              \
  if (MT == mt && sb == sbv) {                                                         \
    launch_skinny<mt, sbv, skinny_ns(mt, sbv), OUTF32>(A, W, C, M, N, K, s);           \
    return;                                                                            \
  }
  BI_SKINNY(1, 1) BI_SKINNY(1, 2) BI_SKINNY(1, 4)
  BI_SKINNY(2, 1) BI_SKINNY(2, 2) BI_SKINNY(2, 4)
  BI_SKINNY(3, 1) BI_SKINNY(3, 2) BI_SKINNY(3, 4)
  BI_SKINNY(4, 1) BI_SKINNY(4, 2) BI_SKINNY(4, 4)
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
  if (M <= 64) {
    if (out_dtype == BI_F32)
      dispatch_skinny<1>(A, W, C, M, N, K, s);
    else
      dispatch_skinny<0>(A, W, C, M, N, K, s);
  } else {
    if (out_dtype == BI_F32)
      launch_tiled<1>(A, W, C, M, N, K, s);
    else
      launch_tiled<0>(A, W, C, M, N, K, s);
  }
  return launched("bi_gemm");
}
