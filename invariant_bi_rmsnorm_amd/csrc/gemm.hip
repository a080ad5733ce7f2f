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
// the operand layout of v_mfma_f32_16x16x32_bf16.  A 16-byte unit of k that
// lies past K (K % 32 != 0) enters both operands as zeros in every kernel.
// The tiled kernel copies fragments to LDS in that layout (one direct
// global->LDS instruction per fragment, read back by the same lane); the
// small-M and large-tile kernels copy whole 128-byte row lines and read
// fragments back through a swizzled line-major layout.
#include <algorithm>
#include <type_traits>

#include "api.h"
#include "common.h"
#include "rownorm.h"

namespace bi {

constexpr int kFrag = 1024;  // bytes per operand fragment

// Packed weight of the bf16 products (bi_pack_weight): W [N][K] stored as
// [ceil(N/256)][ceil(K/64)][16][16][64], zero-padded; element (n, k) sits at
// wp_off(n, k, ceil(K/64)).  A 16-row x 64-k block is 2 KiB in a row, the 16
// blocks of a 256-row panel at one 64-wide K step are 32 KiB in a row, and a
// panel's K steps follow each other, so a 256 x 256 tile reads one
// contiguous panel and a strip of 16 rows reads 2 KiB runs.
__device__ __forceinline__ long wp_off(int n, int k, int kb) {
  return (((long)(n >> 8) * kb + (k >> 6)) * 16 + ((n >> 4) & 15)) * 1024 + (n & 15) * 64 +
         (k & 63);
}

__device__ __forceinline__ f32x4_t mfma(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return mfma16(a, b, c);
}

// OUTF32: 0 = bf16 store, 1 = fp32 store (2 in the skinny kernel: fp32
// store into the split-K twin's slice blockIdx.y)
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
      if (OUTF32 == 1)
        static_cast<float*>(C)[idx] = acc[j];
      else
        static_cast<uint16_t*>(C)[idx] = (uint16_t)f32_to_bf16_bits(acc[j]);
    }
  }
}

// SwiGLU epilogue of a pair tile: MFMA columns 0..7 are gate columns a0 .. a0
// + 7, columns 8..15 the matching up columns.  Each is rounded to bf16 as the
// GEMM's own output would be, then act = bf16(g / (1 + exp(-g)) * u) with the
// arithmetic of bi_silu_mul, so the pair equals the GEMM followed by it.
__device__ __forceinline__ void store_swiglu(void* act, const f32x4_t& acc, int row0, int a0,
                                             int M, int I, int lane) {
  float up[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) up[j] = __shfl_xor(acc[j], 8);   // lane l + 8 holds the up column
  const int c = lane & 15, col = a0 + c;
  if (c >= 8 || col >= I) return;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = row0 + 4 * (lane >> 4) + j;
    if (row < M) {
      const float g = bf16_bits_to_f32((uint16_t)f32_to_bf16_bits(acc[j]));
      const float u = bf16_bits_to_f32((uint16_t)f32_to_bf16_bits(up[j]));
      const float sg = g / (1.0f + exp_fixed(-g));
      static_cast<uint16_t*>(act)[(long)row * I + col] = (uint16_t)f32_to_bf16_bits(sg * u);
    }
  }
}

// Where the QKV projection's epilogue puts its results: rotary tables (both
// NULL for no rotation), positions, the token -> cache slot map and the
// outputs, laid out as bi_rope_kv_append takes them.
struct RopeArgs {
  const int32_t* pos;
  const float* cos_t;
  const float* sin_t;
  const int32_t* slots;
  void* q_out;
  void* k_pool;
  void* v_pool;
  int page_size, h, h_kv, d_h;
};

// RoPE + KV-append epilogue of a pair tile: MFMA columns 0..7 are dims i0 ..
// i0 + 7 of head hh, columns 8..15 the dims d_h / 2 further on, the two
// halves a rotation mixes.  Each is rounded to bf16 as the GEMM's own output
// would be, then rotated and stored with the arithmetic of bi_rope_kv_append,
// so the tile equals the GEMM followed by it.
// The loads the epilogue of pair tile `tile` needs for this lane's four rows
// (cache slots, and the rotary table entries at the rows' positions; rows
// past M read row M - 1, unused).  They depend on no product, so the kernel
// issues them before its K loop and they arrive while the chain runs.
struct RopePre {
  int32_t sl[4];
  float cs[4], sn[4];
};

__device__ __forceinline__ RopePre rope_prefetch(const RopeArgs& ra, int row0, int tile, int M,
                                                 int N, int lane) {
  RopePre p;
#pragma unroll
  for (int j = 0; j < 4; ++j) p.sl[j] = 0, p.cs[j] = 1.f, p.sn[j] = 0.f;
  if (tile >= N / 16) return p;
  const int per_head = ra.d_h / 16, half = ra.d_h / 2;
  const int hh = tile / per_head, c = lane & 15;
  const int i = (tile - hh * per_head) * 8 + (c & 7);
  const bool rotate = hh < ra.h + ra.h_kv && ra.cos_t != nullptr;
  const int rbase = row0 + 4 * (lane >> 4);
  if (hh >= ra.h) {
#pragma unroll
    for (int j = 0; j < 4; ++j) p.sl[j] = ra.slots[min(rbase + j, M - 1)];
  }
  if (rotate) {   // uniform over the wave: one tile, one head
    int32_t pr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) pr[j] = ra.pos[min(rbase + j, M - 1)];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const long t = (long)pr[j] * half + i;
      p.cs[j] = ra.cos_t[t];
      p.sn[j] = ra.sin_t[t];
    }
  }
  return p;
}

__device__ __forceinline__ void store_rope(const RopeArgs& ra, const f32x4_t& acc,
                                           const RopePre& pre, int row0, int tile, int M, int N,
                                           int lane) {
  float other[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) other[j] = __shfl_xor(acc[j], 8);   // lane l ^ 8: the other half
  if (tile >= N / 16) return;
  const int per_head = ra.d_h / 16, half = ra.d_h / 2;
  const int hh = tile / per_head, c = lane & 15, hi = c >> 3;
  const int i = (tile - hh * per_head) * 8 + (c & 7);
  const bool rotate = hh < ra.h + ra.h_kv && ra.cos_t != nullptr;
  const int rbase = row0 + 4 * (lane >> 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = rbase + j;
    if (row >= M) continue;
    const float own = bf16_bits_to_f32((uint16_t)f32_to_bf16_bits(acc[j]));
    const float oth = bf16_bits_to_f32((uint16_t)f32_to_bf16_bits(other[j]));
    float y = own;
    if (rotate)
      y = hi ? __builtin_fmaf(own, pre.cs[j], oth * pre.sn[j])
             : __builtin_fmaf(own, pre.cs[j], -(oth * pre.sn[j]));
    const int e = i + hi * half;   // element of the head row
    long o;
    void* dst;
    if (hh < ra.h) {
      dst = ra.q_out;
      o = ((long)row * ra.h + hh) * ra.d_h + e;
    } else {
      const int g = hh < ra.h + ra.h_kv ? hh - ra.h : hh - ra.h - ra.h_kv;
      const int page = pre.sl[j] / ra.page_size, in_page = pre.sl[j] - page * ra.page_size;
      const long blk = ((long)page * ra.h_kv + g) * ra.page_size * ra.d_h;
      if (hh < ra.h + ra.h_kv) {   // K: unit-major block (common.h)
        dst = ra.k_pool;
        o = blk + k_block_elem(in_page, e, ra.page_size, 2);
      } else {
        dst = ra.v_pool;
        o = blk + (long)in_page * ra.d_h + e;
      }
    }
    static_cast<uint16_t*>(dst)[o] = (uint16_t)f32_to_bf16_bits(y);
  }
}

// ---------------------------------------------------------------------------
// skinny kernel (every M <= 64, and larger M while it is the cheaper kernel):
// one workgroup per CT 16-column strips of W and one group of 8 MB rows of A
// (blockIdx.z; MB and CT are chosen from M and N so that rows x columns per
// workgroup balance).  Per CU the bytes to move are
// its rows of A plus its strips of W, so both ride the fastest path into a
// CU: direct global->LDS copies of
// whole 128-byte lines (8 rows x 128 bytes per instruction).  One wave
// sustains only a fraction of a CU's copy rate, so eight copy waves issue the
// copies; four compute waves read fragments with ds_read_b128 and run the
// MFMAs.  A stage holds KS K-tiles (LPS = KS / 2 lines of each row, about
// 24 KiB in all, so one barrier covers enough bytes).  A and W have rings of
// their own, each fed by four copy waves: A (re-read by every workgroup)
// stays in L2 and needs only a few stages in flight, while W comes from HBM
// and its ring runs as many stages ahead as LDS allows.  Ring layout per
// stage is line-major, [line][8-row block][row][16-byte unit], with unit u of
// row r at slot u ^ (r & 7), so fragment reads are conflict-free.  A is MB
// 8-row blocks (M <= 8 * MB); a 16-row tile whose second block lies past the
// copied rows reads other data there, which only reaches output rows >= M
// (an MFMA output row depends on its own A row alone) and is never stored.
//
// All waves pass the same s_barrier once per stage: after the barrier of
// stage st, stage st of both rings is in LDS and the slots of stage st - 1
// are free.
// ---------------------------------------------------------------------------
constexpr int kSmallCopyWaves = 8, kSmallComputeWaves = 4, kSmallGroupWaves = 4;
constexpr int kSmallThreads = (kSmallCopyWaves + kSmallComputeWaves) * 64;

// L1 (one block of rows in the skinny kernel): stages of up to 16 K-tiles,
// whose fragments the compute wave reads one K-tile at a time
template <int MB, int CT, bool L1 = false>
struct SmallCfg {
  static constexpr int MT = (MB + 1) / 2;                // 16-row tiles
  static constexpr int BLK = MB + 2 * CT;                // 8-row blocks per line
  // lines of each row per stage: about 24 KiB a stage, but longer stages
  // (fewer barriers and fragment waits per K) for the batch-64 tiles
  static constexpr int LPS0 = MB == 4 && CT == 2   ? 6
                              : MB == 4 && CT == 3 ? 4
                                                   : 24 / BLK;
  static constexpr int LPS_MAX = MB == 1 && !L1 ? 4 : 8;   // MB = 1: registers for two per CU
  static constexpr int LPS = LPS0 < 1 ? 1 : LPS0 > LPS_MAX ? LPS_MAX : LPS0;
  static constexpr int KS = 2 * LPS;                     // K-tiles per stage
  static constexpr int A_ITEMS = MB * LPS, W_ITEMS = 2 * CT * LPS;   // KiB per stage
  static constexpr int QA = (A_ITEMS + kSmallGroupWaves - 1) / kSmallGroupWaves;
  static constexpr int QW = (W_ITEMS + kSmallGroupWaves - 1) / kSmallGroupWaves;
  // A ring: about 96 KiB, but 36 KiB (3 stages, the rest of LDS to the W
  // ring) for tiles of 32 rows and 2 strips, the batch-64 O and down
  // projections: measured O 16.8 -> 15.1 us, down 43.4 -> 41.2 us, while
  // tiles of 1, 3 (with the RoPE epilogue) or 8 strips were slower with it
  static constexpr int AD0 = (MB == 1                              ? 24
                              : MB == 4 && CT == 2                 ? 36
                              : MB == 4 && CT == 3                 ? 48
                                                                   : 96) /
                             A_ITEMS;
  static constexpr int AD1 = AD0 < 3 ? 3 : AD0 > 6 ? 6 : AD0;
  static constexpr int AD = AD1 < 1 + 63 / QA ? AD1 : 1 + 63 / QA;   // A ring slots
  static constexpr int A_RING = AD * A_ITEMS * 1024;
  static constexpr int BUDGET = (MB == 1 ? 80 : 160) * 1024;   // MB = 1: two per CU
  static constexpr int WD0 = (BUDGET - A_RING) / (W_ITEMS * 1024);
  static constexpr int WD1 = WD0 < 16 ? WD0 : 16;
  static constexpr int WD = WD1 < 1 + 63 / QW ? WD1 : 1 + 63 / QW;   // W ring slots
  static constexpr int LDS = A_RING + WD * W_ITEMS * 1024;
  static constexpr int WN = CT % 4 == 0 ? 4 : CT % 3 == 0 ? 3 : CT % 2 == 0 ? 2 : 1;  // along N
  static constexpr int WM = 4 / WN;                      // ... and along M
  static constexpr int IM = (MT + WM - 1) / WM;          // row tiles per wave
  static constexpr int JN = CT / WN;                     // column tiles per wave
  static_assert(AD >= 3 && WD >= 3 && LDS <= BUDGET, "rings");
  static_assert(CT % WN == 0, "tiling");
};

// One group of four copy waves feeding one ring of RD slots: NB 8-row blocks
// (rows row0 + 8 b + 0..7, clamped to rmax) times LPS lines per stage; item
// j = line * NB + b of a stage goes to slot offset j KiB and group wave gw
// takes items gw, gw + 4, ...  Lane: row (lane >> 3) of the block, LDS slot
// (lane & 7) <- 16-byte unit (lane & 7) ^ row.  Before the barrier of stage
// st, the wave waits for its own copies of stage st.
// PAIR 0: block b holds rows row0 + 8 b .. (also the SwiGLU product, whose
// weight comes in 8-row gate/up blocks); PAIR 2 (RoPE): blocks 2p, 2p + 1
// hold the two rotation halves of 16-column pair tile row0 / 16 + p, heads of
// `arg` rows (8 dims of each half per tile).
// `pre` extra barriers, matching the compute waves' own before their first
// stage, follow the first RD - 1 stages' copies.
// WP: base is a packed weight (wp_off) and ld its count of 64-wide K steps;
// otherwise base is row-major with row stride ld (kbeg is then any multiple
// of 8; packed, a multiple of 64).
template <int NB, int LPS, int RD, bool NT, int PAIR = 0, bool WP = false>
__device__ __forceinline__ void small_copy_ring(const uint16_t* __restrict__ base, long ld,
                                                int row0, int rmax, int kbeg, int K, int NST,
                                                char* ring, int gw, int lane, int arg = 0,
                                                int pre = 0) {
  constexpr int NIT = NB * LPS, QB = NIT / kSmallGroupWaves, XR = NIT % kSmallGroupWaves;
  constexpr int QMAX = QB + (XR > 0), KS = 2 * LPS;
  const bool extra = gw < XR;
  const int crow = lane >> 3, koff = ((lane & 7) ^ crow) * 8;
  const uint16_t* src[QMAX];
#pragma unroll
  for (int i = 0; i < QMAX; ++i) {
    const int j = min(gw + kSmallGroupWaves * i, NIT - 1), b = j % NB, line = j / NB;
    int row;
    if constexpr (PAIR == 2) {
      const int per_head = arg / 16, tile = min(row0 / 16 + (b >> 1), rmax / 16);
      const int hh = tile / per_head;
      row = hh * arg + (b & 1) * (arg / 2) + (tile - hh * per_head) * 8 + crow;
    } else {
      row = min(row0 + b * 8 + crow, rmax);
    }
    src[i] = WP ? base + wp_off(row, kbeg + line * 64 + koff, (int)ld)
                : base + (long)row * ld + kbeg + line * 64 + koff;
  }
  // elements from one stage's copy to the next: KS K-tiles of 32
  const long adv = WP ? (long)(KS / 2) * 16 * 1024 : 32 * KS;
  auto issue = [&](int st) {
    char* slot = ring + (st % RD) * (NIT * 1024);
#pragma unroll
    for (int i = 0; i < QMAX; ++i) {
      if (i < QB || extra) {
        const int j = gw + kSmallGroupWaves * i, line = j / NB;
        const int k = st * (32 * KS) + line * 64 + koff;   // this lane's first k
        const uint16_t* p = k < K ? src[i] + st * adv : WP ? base : src[i] - line * 64 - koff;
        if (NT) dma16_nt(p, slot + j * 1024);
        else dma16(p, slot + j * 1024);
      }
    }
  };
#pragma unroll
  for (int s = 0; s < RD - 1; ++s)
    if (s < NST) issue(s);
  for (int i = 0; i < pre; ++i) __builtin_amdgcn_s_barrier();
  for (int st = 0; st < NST; ++st) {
    if (st + RD - 1 > NST) BI_WAIT_VMCNT(0);
    else if (extra) BI_WAIT_VMCNT((RD - 2) * QMAX);
    else BI_WAIT_VMCNT((RD - 2) * QB);
    __builtin_amdgcn_s_barrier();
    if (st + RD - 1 < NST) issue(st + RD - 1);
  }
}

// SwiGLU epilogue on all of the workgroup's waves.  The compute waves leave
// their fp32 tiles in LDS (tile (m, c), 16 x 16 row-major, at (m CT + c)
// KiB); then every thread takes act elements t, t + kSmallThreads, ... of
// the workgroup's `rows` rows x 8 CT act columns (a gate column and its up
// column 8 further in the same tile) with store_swiglu's arithmetic, so the
// bits are those of the GEMM followed by bi_silu_mul.  Spread over 12 waves
// rather than left to the 4 compute waves, whose epilogue of exp and
// division per element ran several microseconds behind the K loop.
template <int CT>
__device__ __forceinline__ void swiglu_from_lds(const float* at, void* act, int m0, int rows,
                                                int a0, int I) {
  const int n = rows * 8 * CT;
  for (int e = threadIdx.x; e < n; e += kSmallThreads) {
    const int r = e / (8 * CT), a = e - r * (8 * CT);
    if (a0 + a >= I) continue;
    const float* t = at + (((r >> 4) * CT + (a >> 3)) * 16 + (r & 15)) * 16 + (a & 7);
    const float g = bf16_bits_to_f32((uint16_t)f32_to_bf16_bits(t[0]));
    const float u = bf16_bits_to_f32((uint16_t)f32_to_bf16_bits(t[8]));
    const float sg = g / (1.0f + exp_fixed(-g));
    static_cast<uint16_t*>(act)[(long)(m0 + r) * I + a0 + a] =
        (uint16_t)f32_to_bf16_bits(sg * u);
  }
}

// RoPE + KV-append epilogue on all of the workgroup's waves, from the fp32
// tiles the compute waves leave in LDS (laid out as for swiglu_from_lds).  A
// work item is one (row, pair tile, half): the 8 dims of a head row that one
// half of a pair tile holds, which are one 16-byte unit of a q row, of a K
// page (unit-major) and of a V page row.  It rounds the 8 own and the 8
// partner values to bf16, rotates with store_rope's arithmetic and writes
// the unit with one 16-byte store, where the compute waves' lanes stored 2
// bytes each.
template <int CT>
__device__ __forceinline__ void rope_from_lds(const float* at, const RopeArgs& ra, int m0,
                                              int rows, int t0, int N) {
  const int per_head = ra.d_h / 16, half = ra.d_h / 2;
  const int n = rows * CT * 2;
  for (int w = threadIdx.x; w < n; w += kSmallThreads) {
    const int r = w / (2 * CT), c = (w >> 1) % CT, hi = w & 1;
    const int tile = t0 + c;
    if (tile >= N / 16) continue;
    const int hh = tile / per_head, i0 = (tile - hh * per_head) * 8;
    const bool rotate = hh < ra.h + ra.h_kv && ra.cos_t != nullptr;
    const int row = m0 + r;
    const float* trow = at + (((r >> 4) * CT + c) * 16 + (r & 15)) * 16;
    float own[8], oth[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      own[j] = bf16_bits_to_f32((uint16_t)f32_to_bf16_bits(trow[8 * hi + j]));
      oth[j] = bf16_bits_to_f32((uint16_t)f32_to_bf16_bits(trow[8 * (hi ^ 1) + j]));
    }
    float y[8];
    if (rotate) {
      const long tb = (long)ra.pos[row] * half + i0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float cs = ra.cos_t[tb + j], sn = ra.sin_t[tb + j];
        y[j] = hi ? __builtin_fmaf(own[j], cs, oth[j] * sn)
                  : __builtin_fmaf(own[j], cs, -(oth[j] * sn));
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = own[j];
    }
    const u32x4_t v = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                       pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
    const int e0 = i0 + hi * half;   // first of the 8 elements of the head row
    long o;
    void* dst;
    if (hh < ra.h) {
      dst = ra.q_out;
      o = ((long)row * ra.h + hh) * ra.d_h + e0;
    } else {
      const int g = hh < ra.h + ra.h_kv ? hh - ra.h : hh - ra.h - ra.h_kv;
      const int sl = ra.slots[row];
      const int page = sl / ra.page_size, in_page = sl - page * ra.page_size;
      const long blk = ((long)page * ra.h_kv + g) * ra.page_size * ra.d_h;
      if (hh < ra.h + ra.h_kv) {   // K: unit-major block (common.h)
        dst = ra.k_pool;
        o = blk + k_block_elem(in_page, e0, ra.page_size, 2);
      } else {
        dst = ra.v_pool;
        o = blk + (long)in_page * ra.d_h + e0;
      }
    }
    *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(dst) + o) = v;
  }
}

// (one block of rows: two workgroups share a CU, 24 waves, so at most 80
// VGPRs)
template <int MB, int CT, int OUTF32>
__global__ __launch_bounds__(kSmallThreads) __attribute__((amdgpu_waves_per_eu(MB == 1 ? 6 : 1)))
void k_gemm_small(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W, void* C, int M, int N,
    int Ktot, int kslice, RopeArgs ra) {
  using G = SmallCfg<MB, CT, MB == 1>;
  constexpr int KS = G::KS, LPS = G::LPS, MT = G::MT;
  // K slice of this workgroup (all of K on the invariant path; the split-K
  // twin launches several along y).  Rows keep stride Ktot.
  const int kbeg = blockIdx.y * kslice;
  const int K = min(kslice, Ktot - kbeg);
  const long ld = Ktot;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n0 = blockIdx.x * (16 * CT), m0 = blockIdx.z * (8 * MB);
  const int mend = min(M, m0 + 8 * MB);  // rows of this workgroup: m0 .. mend - 1
  const int KT = (K + 31) >> 5;
  const int NST = (KT + KS - 1) / KS;

  if (wave >= kSmallComputeWaves) {
    const int cw = wave - kSmallComputeWaves;
    if (cw < kSmallGroupWaves)
      small_copy_ring<MB, LPS, G::AD, false>(A, ld, m0, mend - 1, kbeg, K, NST, smem, cw, lane);
    else if constexpr (OUTF32 == 4)
      // RoPE: strip x holds pair tiles CT x .. CT x + CT - 1 (N % 16 == 0)
      small_copy_ring<2 * CT, LPS, G::WD, true, 2, true>(W, (Ktot + 63) / 64, n0, N - 1, kbeg, K,
                                                         NST, smem + G::A_RING,
                                                         cw - kSmallGroupWaves, lane, ra.d_h);
    else
      small_copy_ring<2 * CT, LPS, G::WD, true, 0, true>(W, (Ktot + 63) / 64, n0, N - 1, kbeg, K,
                                                         NST, smem + G::A_RING,
                                                         cw - kSmallGroupWaves, lane);
    if constexpr (OUTF32 == 3 || OUTF32 == 4) {   // the compute waves' epilogue barriers
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      if constexpr (OUTF32 == 3)
        swiglu_from_lds<CT>(reinterpret_cast<const float*>(smem), C, m0, mend - m0, n0 / 2,
                            N / 2);
      else
        rope_from_lds<CT>(reinterpret_cast<const float*>(smem), ra, m0, mend - m0, n0 / 16, N);
    }
    return;
  }

  // ---- compute waves: wave (wm, wn) owns row tiles wm + WM i (< MT) and
  // column tiles wn + WN j.  A wave whose first row tile lies past MT idles.
  const int wn = wave % G::WN, wm = wave / G::WN;
  const bool active = wm < MT;
  const int r = lane & 15, g = lane >> 4;
  // fragment offset of row r, K-tile parity h inside a 16-row tile
  const uint32_t off0 = ((r >> 3) << 10) + ((r & 7) << 7) + ((g ^ (r & 7)) << 4);
  const uint32_t off1 = ((r >> 3) << 10) + ((r & 7) << 7) + (((4 + g) ^ (r & 7)) << 4);
  uint32_t aoff[G::IM], boff[G::JN];
#pragma unroll
  for (int i = 0; i < G::IM; ++i) aoff[i] = min(wm + G::WM * i, MT - 1) * 2048;
#pragma unroll
  for (int j = 0; j < G::JN; ++j) boff[j] = (wn + G::WN * j) * 2048;
  f32x4_t acc[G::IM][G::JN];
#pragma unroll
  for (int i = 0; i < G::IM; ++i)
#pragma unroll
    for (int j = 0; j < G::JN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // one stage: read every fragment of its (up to) KS K-tiles, then the MFMAs
  // in ascending K-tile order.  A unit past K enters both operands as zeros;
  // a stage that lies wholly below K (`inside`) has no such unit, so it skips
  // the selects (a compare and 8 v_cndmask per MFMA between dependent MFMAs).
  auto stage = [&](auto inside, const char* aslot, const char* wslot, int st, int nkt) {
    if constexpr (MB == 1) {
      // one chain per wave and long stages: one K-tile's fragments at a time
#pragma unroll
      for (int kt = 0; kt < KS; ++kt) {
        if (kt < nkt) {
          const uint32_t off = (kt & 1) ? off1 : off0;
          const char* abase = aslot + (kt >> 1) * (MB * 1024) + off;
          const char* wbase = wslot + (kt >> 1) * (2 * CT * 1024) + off;
          u32x4_t a1[G::IM], b1[G::JN];
#pragma unroll
          for (int i = 0; i < G::IM; ++i) a1[i] = *reinterpret_cast<const u32x4_t*>(abase + aoff[i]);
#pragma unroll
          for (int j = 0; j < G::JN; ++j) b1[j] = *reinterpret_cast<const u32x4_t*>(wbase + boff[j]);
          const bool tail = !decltype(inside)::value && (st * KS + kt) * 32 + 8 * g >= K;
#pragma unroll
          for (int i = 0; i < G::IM; ++i) {
            const u32x4_t av = tail ? u32x4_t{0, 0, 0, 0} : a1[i];
#pragma unroll
            for (int j = 0; j < G::JN; ++j)
              acc[i][j] = mfma(av, tail ? u32x4_t{0, 0, 0, 0} : b1[j], acc[i][j]);
          }
        }
      }
      return;
    }
    u32x4_t a[KS][G::IM], b[KS][G::JN];
#pragma unroll
    for (int kt = 0; kt < KS; ++kt) {
      if (kt < nkt) {
        const uint32_t off = (kt & 1) ? off1 : off0;
        const char* abase = aslot + (kt >> 1) * (MB * 1024) + off;
        const char* wbase = wslot + (kt >> 1) * (2 * CT * 1024) + off;
#pragma unroll
        for (int i = 0; i < G::IM; ++i) a[kt][i] = *reinterpret_cast<const u32x4_t*>(abase + aoff[i]);
#pragma unroll
        for (int j = 0; j < G::JN; ++j) b[kt][j] = *reinterpret_cast<const u32x4_t*>(wbase + boff[j]);
      }
    }
#pragma unroll
    for (int kt = 0; kt < KS; ++kt) {
      if (kt < nkt) {
        const bool tail = !decltype(inside)::value && (st * KS + kt) * 32 + 8 * g >= K;
#pragma unroll
        for (int i = 0; i < G::IM; ++i) {
          const u32x4_t av = tail ? u32x4_t{0, 0, 0, 0} : a[kt][i];
#pragma unroll
          for (int j = 0; j < G::JN; ++j)
            acc[i][j] = mfma(av, tail ? u32x4_t{0, 0, 0, 0} : b[kt][j], acc[i][j]);
        }
      }
    }
  };
  for (int st = 0; st < NST; ++st) {
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    const char* aslot = smem + (st % G::AD) * (G::A_ITEMS * 1024);
    const char* wslot = smem + G::A_RING + (st % G::WD) * (G::W_ITEMS * 1024);
    const int nkt = KT - st * KS;
    if (active) {
      if (nkt >= KS) {
        if ((st + 1) * KS * 32 <= K) stage(std::true_type{}, aslot, wslot, st, KS);
        else stage(std::false_type{}, aslot, wslot, st, KS);
      } else {
#pragma unroll
        for (int n = 1; n < KS; ++n)
          if (nkt == n) stage(std::false_type{}, aslot, wslot, st, n);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  }
  if constexpr (OUTF32 == 3 || OUTF32 == 4) {   // tiles to LDS once every wave is past the ring
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    float* at = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int i = 0; i < G::IM; ++i)
#pragma unroll
      for (int j = 0; j < G::JN; ++j) {
        const int m = wm + G::WM * i, c = wn + G::WN * j;
        if (active && m < MT) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            at[((m * CT + c) * 16 + 4 * g + q) * 16 + r] = acc[i][j][q];
        }
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if constexpr (OUTF32 == 3)
      swiglu_from_lds<CT>(at, C, m0, mend - m0, n0 / 2, N / 2);
    else
      rope_from_lds<CT>(at, ra, m0, mend - m0, n0 / 16, N);
    return;
  }
#pragma unroll
  for (int i = 0; i < G::IM; ++i)
#pragma unroll
    for (int j = 0; j < G::JN; ++j) {
      const int m = wm + G::WM * i, c = wn + G::WN * j;
      if constexpr (OUTF32 == 2) {   // split-K twin: this slice's partial sums
        if (m < MT)
          store_tile<1>(static_cast<float*>(C) + (long)blockIdx.y * M * N, acc[i][j],
                        m0 + m * 16, n0 + c * 16, mend, N, lane);
      } else if (m < MT) {
        store_tile<OUTF32>(C, acc[i][j], m0 + m * 16, n0 + c * 16, mend, N, lane);
      }
    }
}

// ---------------------------------------------------------------------------
// Small batch with the RMSNorm in the prologue (at most kNormRows rows, K <=
// 4096): x = RMSNorm(h [+ o]) * gamma is computed by every workgroup for
// itself, into LDS, while its W ring fills, and then feeds the one-strip
// skinny GEMM in place of A.  At a few rows a separate norm launch costs
// several microseconds of fixed time for a few KiB of work; here it costs
// one barrier.  The arithmetic is the norm kernels' (same lanes, same
// vectors, the helpers of rownorm.h: bit for bit bi_add_rmsnorm /
// bi_rmsnorm) followed by the skinny kernel's chain (ascending K-tiles, the
// same fragment of each operand), so every output equals the two launches'.
// Workgroup 0 alone stores the new residual h_out = round(h + o) and x, so
// h_out must not alias h or o (other workgroups still read them).
// LDS: [W ring: WD stages][x: M rows of ceil(K/64) lines of 128 bytes,
// unit u of a line of row m at slot u ^ (m & 7)][4 x 4 wave sums].
// ---------------------------------------------------------------------------
// W ring stages: 7 for up to 2 rows, 5 for 3 and 4 (x takes the rest of
// the 80 KiB that lets two workgroups share a CU)
constexpr int kNormRows = 4, kNormMaxK = 4096;
constexpr int kNormThreads = (kSmallComputeWaves + kSmallGroupWaves) * 64;
constexpr int norm_ring_bytes(int wd) { return wd * SmallCfg<1, 1>::W_ITEMS * 1024; }
constexpr int kNormLdsMax = 80 * 1024;
static_assert(norm_ring_bytes(7) + 2 * (kNormMaxK / 64) * 128 + 64 <= kNormLdsMax &&
                  norm_ring_bytes(5) + 4 * (kNormMaxK / 64) * 128 + 64 <= kNormLdsMax,
              "two workgroups per CU");

struct NormArgs {
  const uint16_t* h;
  const uint16_t* o;   // NULL: no residual add
  const uint16_t* gamma;
  uint16_t* h_out;     // with o: round(h + o), stored by workgroup 0
  uint16_t* x_out;     // NULL or the normalised rows, stored by workgroup 0
  float eps;
};

// Row of W that lane row `crow` of 8-row block b copies for strip s: PAIR 0
// the strip's 16 rows (also SwiGLU: 8 gate rows then the matching 8 up rows
// in the weight's 8-row blocks), 2 (RoPE) the two rotation halves of a head
// of `arg` rows -- the skinny kernel's copy layouts for one strip.
template <int PAIR>
__device__ __forceinline__ int norm_strip_row(int s, int b, int crow, int N, int arg) {
  if constexpr (PAIR == 2) {
    const int per_head = arg / 16, hh = s / per_head;
    return hh * arg + b * (arg / 2) + (s - hh * per_head) * 8 + crow;
  } else {
    return min(s * 16 + b * 8 + crow, N - 1);
  }
}

// Workgroup b takes strips b, b + gridDim.x, ... of the product (the grid is
// at most two workgroups per CU), so the norm runs once per workgroup and
// its W ring streams on across strips: stage g of the ring is stage g % NST
// of its strip g / NST.
template <bool ADD, int OUTF32, int WD>
__global__ __launch_bounds__(kNormThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_gemm_norm(
    NormArgs na, const uint16_t* __restrict__ W, void* C, int M, int N, int K, RopeArgs ra) {
  constexpr int RING = norm_ring_bytes(WD);
  using G = SmallCfg<1, 1>;
  constexpr int KS = G::KS, NIT = G::W_ITEMS, QB = NIT / kSmallGroupWaves;
  constexpr int PAIR = OUTF32 == 4 ? 2 : 0;
  static_assert(G::LPS * 2 == NIT && NIT % kSmallGroupWaves == 0, "one strip of 16 rows");
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int rowb = ((K + 63) >> 6) * 128;   // LDS bytes per x row
  char* xr = smem + RING;
  float* ws = reinterpret_cast<float*>(xr + M * rowb);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int KT = (K + 31) >> 5;
  const int NST = (KT + KS - 1) / KS;
  const int nstrips = (N + 15) >> 4;
  const int mine = (nstrips - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  const int total = mine * NST;   // ring stages of this workgroup

  if (wave >= kSmallComputeWaves) {   // W copies; one extra barrier: the prologue's
    const int cw = wave - kSmallComputeWaves;
    const int crow = lane >> 3, koff = ((lane & 7) ^ crow) * 8;
    const int arg = PAIR == 2 ? ra.d_h : 0, kbw = (K + 63) / 64;   // W packed
    auto issue = [&](int gs) {
      const int i = gs / NST, st = gs - i * NST;
      const int strip = blockIdx.x + i * gridDim.x;
      char* slot = smem + (gs % WD) * (NIT * 1024);
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        const int j = cw + kSmallGroupWaves * q, line = j >> 1;
        const int row = norm_strip_row<PAIR>(strip, j & 1, crow, N, arg);
        const int k = st * (32 * KS) + line * 64 + koff;   // this lane's first k
        dma16_nt(W + (k < K ? wp_off(row, k, kbw) : 0), slot + j * 1024);
      }
    };
#pragma unroll
    for (int g = 0; g < WD - 1; ++g)
      if (g < total) issue(g);
    __builtin_amdgcn_s_barrier();
    for (int g = 0; g < total; ++g) {
      if (g + WD - 1 > total) BI_WAIT_VMCNT(0);
      else BI_WAIT_VMCNT((WD - 2) * QB);
      __builtin_amdgcn_s_barrier();
      if (g + WD - 1 < total) issue(g + WD - 1);
    }
    return;
  }

  // ---- the norm, by the four compute waves (lane t of the row's 256) ----
  const int t = threadIdx.x, nv = K >> 3;
  const bool writer = blockIdx.x == 0;
  u32x4_t gv[2], xv[kNormRows][2];   // gamma and the rounded rows, as bf16 bits
  float a[kNormRows];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    if (t + 256 * j < nv) gv[j] = *reinterpret_cast<const u32x4_t*>(na.gamma + 8 * (t + 256 * j));
#pragma unroll
  for (int m = 0; m < kNormRows; ++m) {
    a[m] = 0.0f;
    if (m < M) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int v = t + 256 * j;
        if (v < nv) {
          const long i0 = (long)m * K + 8 * v;
          float hs[8], xs[8];
          load8<1>(na.h, i0, hs);
          if constexpr (ADD) {
            float os[8];
            load8<1>(na.o, i0, os);
#pragma unroll
            for (int e = 0; e < 8; ++e) hs[e] = hs[e] + os[e];
          }
          xv[m][j] = u32x4_t{pack_bf16x2(hs[0], hs[1]), pack_bf16x2(hs[2], hs[3]),
                             pack_bf16x2(hs[4], hs[5]), pack_bf16x2(hs[6], hs[7])};
          if (ADD && writer) *reinterpret_cast<u32x4_t*>(na.h_out + i0) = xv[m][j];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            xs[e] = bf16_bits_to_f32((uint16_t)(xv[m][j][e >> 1] >> (16 * (e & 1))));
          a[m] = rn_fold8(xs, a[m]);
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < kNormRows; ++m) {
    const float sum = rn_wave_sum(a[m]);
    if (m < M && lane == 0) ws[4 * m + wave] = sum;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
  for (int m = 0; m < kNormRows; ++m) {
    if (m < M) {
      const float r = rn_inv_rms(ws + 4 * m, K, na.eps);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int v = t + 256 * j;
        if (v < nv) {
          float xs[8], gs[8], ys[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            xs[e] = bf16_bits_to_f32((uint16_t)(xv[m][j][e >> 1] >> (16 * (e & 1))));
            gs[e] = bf16_bits_to_f32((uint16_t)(gv[j][e >> 1] >> (16 * (e & 1))));
          }
          rn_scale8(xs, gs, r, ys);
          const u32x4_t y = {pack_bf16x2(ys[0], ys[1]), pack_bf16x2(ys[2], ys[3]),
                             pack_bf16x2(ys[4], ys[5]), pack_bf16x2(ys[6], ys[7])};
          *reinterpret_cast<u32x4_t*>(xr + m * rowb + (v >> 3) * 128 + (((v & 7) ^ (m & 7)) << 4)) =
              y;
          if (writer && na.x_out) *reinterpret_cast<u32x4_t*>(na.x_out + (long)m * K + 8 * v) = y;
        }
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");

  // ---- the skinny kernel's chain per strip: wave 0 holds the 16 x 16 tile ----
  const int r = lane & 15, g = lane >> 4, rr = min(r, M - 1);
  const uint32_t woff0 = ((r >> 3) << 10) + ((r & 7) << 7) + ((g ^ (r & 7)) << 4);
  const uint32_t woff1 = ((r >> 3) << 10) + ((r & 7) << 7) + (((4 + g) ^ (r & 7)) << 4);
  const char* xrow = xr + rr * rowb;
  for (int i = 0; i < mine; ++i) {
    const int strip = blockIdx.x + i * gridDim.x;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    RopePre rpre;
    if constexpr (OUTF32 == 4)
      if (wave == 0) rpre = rope_prefetch(ra, 0, strip, M, N, lane);
    for (int st = 0; st < NST; ++st) {
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      const char* wslot = smem + ((i * NST + st) % WD) * (NIT * 1024);
      const int nkt = min(KS, KT - st * KS);
      if (wave == 0) {   // half a stage's fragments at a time (registers)
#pragma unroll
        for (int hf = 0; hf < KS; hf += KS / 2) {
          u32x4_t av[KS / 2], bv[KS / 2];
#pragma unroll
          for (int u = 0; u < KS / 2; ++u) {
            const int kt = hf + u, ktg = st * KS + kt;
            if (kt < nkt) {
              av[u] = *reinterpret_cast<const u32x4_t*>(
                  xrow + (ktg >> 1) * 128 + (((((ktg & 1) << 2) | g) ^ (rr & 7)) << 4));
              bv[u] = *reinterpret_cast<const u32x4_t*>(wslot + (kt >> 1) * 2048 +
                                                        ((kt & 1) ? woff1 : woff0));
            }
          }
#pragma unroll
          for (int u = 0; u < KS / 2; ++u) {
            const int kt = hf + u;
            if (kt < nkt) {
              const bool tail = (st * KS + kt) * 32 + 8 * g >= K;
              acc = mfma(tail ? u32x4_t{0, 0, 0, 0} : av[u],
                         tail ? u32x4_t{0, 0, 0, 0} : bv[u], acc);
            }
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    }
    if (wave == 0) {
      if constexpr (OUTF32 == 3)
        store_swiglu(C, acc, 0, strip * 8, M, N / 2, lane);
      else if constexpr (OUTF32 == 4)
        store_rope(ra, acc, rpre, 0, strip, M, N, lane);
      else
        store_tile<OUTF32>(C, acc, 0, strip * 16, M, N, lane);
    }
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
      else   // W packed
        src = W + wp_off(min(n0 + tile * 16 + lrow, N - 1), kk, (K + 63) / 64);
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
template <int MB, int CT, int OUTF32>
static void launch_small_k(const void* A, const void* W, void* C, int M, int N, int K,
                           hipStream_t s, int splits, int kslice, const RopeArgs& ra) {
  constexpr int lds = SmallCfg<MB, CT, MB == 1>::LDS;
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)k_gemm_small<MB, CT, OUTF32>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    attr = true;
  }
  hipLaunchKernelGGL((k_gemm_small<MB, CT, OUTF32>),
                     dim3((N + 16 * CT - 1) / (16 * CT), splits, (M + 8 * MB - 1) / (8 * MB)),
                     dim3(kSmallThreads), lds, s,
                     (const uint16_t*)A, (const uint16_t*)W, C, M, N, K, kslice, ra);
}

// Rows (8 MB) and 16-column strips (CT) per workgroup, chosen from M and N:
// a workgroup moves its rows of A plus its strips of W, one workgroup per CU
// at a time, so the time goes with rounds * (MB + 2 CT) (KiB per 32 k).  At
// M <= 8 it is always one 8-row block and one strip: A is then negligible,
// two such workgroups share a CU, and HBM streams best when each CU sweeps
// few rows of W at a time (measured faster than the model's pick there).
struct SmallShape {
  int mb, ct;
  long cost;   // rounds of 256 workgroups x (MB + 2 CT): KiB per CU per 32 k
};
static SmallShape small_shape(int M, int N) {
  const long tiles = (N + 15) / 16;
  if (M <= 8) return SmallShape{1, 1, ((tiles + 255) / 256) * 3};
  SmallShape best{8, 1, -1};
  long best_wgs = 0;
  for (int mb : {1, 2, 4, 6, 8}) {
    const long rg = (M + 8 * mb - 1) / (8 * mb);
    for (int ct : {1, 2, 3, 4, 7, 8}) {
      if (mb == 1 && ct != 1) continue;   // 8-row blocks: 16-row strips, two per CU
      const long wgs = rg * ((tiles + ct - 1) / ct);
      const long cost = ((wgs + 255) / 256) * (mb + 2 * ct);
      if (best.cost < 0 || cost < best.cost || (cost == best.cost && wgs < best_wgs))
        best = SmallShape{mb, ct, cost}, best_wgs = wgs;
    }
  }
  // From 9 to 32 rows, where a shape fits in one round of 256 workgroups,
  // the fastest of all shapes (timed alone) was the one-round shape with the
  // most workgroups, then the fewest padded rows, then the most rows per
  // workgroup: the QKV projection at 32 rows 17.0 us against 18.9, O 13.2
  // against 14.0.  At 64 rows the same rule timed faster alone but slower
  // inside the decode step, so from 33 rows the byte count above decides.
  if (M <= 32) {
    SmallShape pick{0, 0, 0};
    long pick_wgs = 0, pick_pad = 0;
    for (int mb : {2, 4, 6, 8}) {
      const long rg = (M + 8 * mb - 1) / (8 * mb), pad = rg * 8 * mb - M;
      for (int ct : {1, 2, 3, 4, 7, 8}) {
        const long wgs = rg * ((tiles + ct - 1) / ct);
        if (wgs > 256) continue;
        if (wgs > pick_wgs || (wgs == pick_wgs && (pad < pick_pad ||
                                                   (pad == pick_pad && mb > pick.mb))))
          pick = SmallShape{mb, ct, mb + 2 * ct}, pick_wgs = wgs, pick_pad = pad;
      }
    }
    if (pick_wgs > 0) return pick;
  }
  return best;
}

template <int OUTF32>
static void dispatch_small(const void* A, const void* W, void* C, int M, int N, int K,
                           hipStream_t s, int splits = 1, int kslice = 0,
                           const RopeArgs& ra = RopeArgs{}) {
  if (splits == 1) kslice = K;
  const SmallShape sh = small_shape(M, N);
#define BI_SMALL(MB_, CT_)                                                      \
  if (sh.mb == MB_ && sh.ct == CT_) {                                           \
    launch_small_k<MB_, CT_, OUTF32>(A, W, C, M, N, K, s, splits, kslice, ra);  \
    return;                                                                     \
  }
#define BI_SMALL_M(MB_) \
  BI_SMALL(MB_, 1) BI_SMALL(MB_, 2) BI_SMALL(MB_, 3) BI_SMALL(MB_, 4) BI_SMALL(MB_, 7)          \
  BI_SMALL(MB_, 8)
  BI_SMALL_M(1) BI_SMALL_M(2) BI_SMALL_M(4) BI_SMALL_M(6) BI_SMALL_M(8)
#undef BI_SMALL_M
#undef BI_SMALL
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
// workgroup, eight waves in two groups that take turns ("ping-pong").  Group
// g = wave / 4 holds one wave on each SIMD and owns output rows 128 g ..
// 128 g + 127; wave wn of a group owns columns 64 wn .. 64 wn + 63 (8 x 4
// MFMA tiles).  Phases are separated by workgroup barriers: in every phase
// one group reads its fragments of a line stage (two K-tiles) from LDS and
// issues direct copies while the other runs its 64 MFMAs on the stage it read
// in the phase before, so each SIMD's matrix core has work while its other
// wave feeds LDS.  Group 0 takes stage L in phases 2L (memory) and 2L + 1
// (MFMA), group 1 one phase later.  Each output element is still one MFMA
// chain over the K-tiles in ascending order, as on every other path.
//
// LDS holds two line stages of 64 KiB: 128-byte lines (two K-tiles) of 256 A
// rows then 256 W rows, 8 rows per 1 KiB block, the 16-byte unit u of row r at
// slot u ^ (r & 7); each copy moves 8 whole lines.  Copies are buffer loads
// to LDS: the tile's rows of A and of W are two buffers, so one lane offset
// serves every copy (the block's row offset rides in the scalar offset) and
// rows past M or N read as zeros (they feed only outputs that are not
// stored).  Stage L + 1 goes to the slot that stage L - 1 used, which group 1
// finished reading in phase 2L - 1: group 0 copies the W rows and its own A
// rows in phase 2L (12 per wave), group 1 its A rows in phase 2L + 1 (4 per
// wave), and each group waits for its copies at the end of its next MFMA
// phase, before the first read that needs them.  Workgroups are mapped so
// that each XCD (blockIdx % 8) takes a contiguous range of tiles in grouped
// order (4 row-blocks at a time), so the tiles resident on one XCD share A
// rows and W columns in its L2.
// ---------------------------------------------------------------------------
// a[i] = LDS[ba + 2048 i] (i < 8), b[j] = LDS[bb + 2048 j] (j < 4), not waited for
__device__ __forceinline__ void lds_read_8_4_nowait(u32x4_t (&a)[8], u32x4_t (&b)[4],
                                                    uint32_t ba, uint32_t bb) {
  asm volatile(
      "ds_read_b128 %0, %12\n\tds_read_b128 %1, %12 offset:2048\n\t"
      "ds_read_b128 %2, %12 offset:4096\n\tds_read_b128 %3, %12 offset:6144\n\t"
      "ds_read_b128 %4, %12 offset:8192\n\tds_read_b128 %5, %12 offset:10240\n\t"
      "ds_read_b128 %6, %12 offset:12288\n\tds_read_b128 %7, %12 offset:14336\n\t"
      "ds_read_b128 %8, %13\n\tds_read_b128 %9, %13 offset:2048\n\t"
      "ds_read_b128 %10, %13 offset:4096\n\tds_read_b128 %11, %13 offset:6144"
      : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5]),
        "=&v"(a[6]), "=&v"(a[7]), "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]), "=&v"(b[3])
      : "v"(ba), "v"(bb)
      : "memory");
}

// waits for the reads above; the operands tie every later use of a and b to it
__device__ __forceinline__ void lds_wait_8_4(u32x4_t (&a)[8], u32x4_t (&b)[4]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]),
                 "+v"(a[6]), "+v"(a[7]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3])
               :
               : "memory");
}

template <int OUTF32>
__global__ __launch_bounds__(512) void k_gemm_big(const uint16_t* __restrict__ A,
                                                   const uint16_t* __restrict__ W, void* C,
                                                   int M, int N, int K, int tiles_m, int tiles_n) {
  constexpr int NS = 2, STAGE = 64 * 1024;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int nt = tiles_m * tiles_n, bid = blockIdx.x;
  const int xcd = bid % 8, idx = bid / 8;
  const int per = nt / 8, rem = nt % 8;
  const int t = xcd * per + (xcd < rem ? xcd : rem) + idx;
  constexpr int GM = 4;
  const int grp = t / (GM * tiles_n), first = grp * GM;
  const int gm = min(GM, tiles_m - first);
  const int tm = first + (t % (GM * tiles_n)) % gm, tn = (t % (GM * tiles_n)) / gm;
  const int m0 = tm * 256, n0 = tn * 256;
  const int g = wave >> 2, wn = wave & 3;
  const int KT = (K + 31) >> 5, NLS = (KT + 1) >> 1;
  // buffers over the tile's rows (word 3 = 0x20000: data format 32-bit, as a
  // raw buffer needs); record counts in bytes, so reads past them give zeros
  // W is packed (wp_off): the tile's 256 rows are one panel, K steps of 32
  // KiB; its padded rows are zeros
  const uint32_t rowbytes = (uint32_t)K * 2;
  const int kbw = (K + 63) >> 6;   // the tile's rows are packed panel n0 / 256
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(A + (long)m0 * K), (short)0, (int)(min(256, M - m0) * rowbytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t rW = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(W + (long)(n0 >> 8) * kbw * 16 * 1024), (short)0, (int)((long)kbw * 32768),
      0x00020000);
  const int crow = lane >> 3, cunit = (lane & 7) ^ crow;
  const uint32_t voff = crow * rowbytes + cunit * 16, voffw = crow * 128 + cunit * 16;
  // NB copies of line stage ls (64 k): row blocks base + wn + 4 i of the tile
  // into stage blocks sblk0 + ..  (lane: row crow of the block, unit cunit of
  // its 128-byte line, written to slot lane & 7); A rows by their stride, W
  // rows where the packed panel keeps them (8-row block b of the tile: half
  // b & 1 of 16-row block b / 2 of K step ls)
  auto issue = [&](auto nb_c, int ls, __amdgpu_buffer_rsrc_t r, int sblk0, int base) {
    constexpr int NB = decltype(nb_c)::value;
    char* slot = smem + (ls % NS) * STAGE;
    const bool w = sblk0 != 0;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int blk = base + wn + 4 * i;
      const uint32_t so = w ? ((uint32_t)ls * 16 + (blk >> 1)) * 2048 + (blk & 1) * 1024
                            : blk * 8 * rowbytes + ls * 128;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(slot + (sblk0 + blk) * 1024), 16,
                                               w ? voffw : voff, so, 0, 0);
    }
  };
  using I4 = std::integral_constant<int, 4>;
  using I8 = std::integral_constant<int, 8>;
  auto rd_off = [&](int kt) {
    const int r = lane & 15, u = 4 * kt + (lane >> 4);
    return (uint32_t)(((r >> 3) & 1) * 1024 + (r & 7) * 128 + 16 * (u ^ (r & 7)));
  };
  const uint32_t off0 = rd_off(0), off1 = rd_off(1);
  const uint32_t lds0 = lds_addr(smem);

  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  u32x4_t a0[8], b0[4], a1[8], b1[4];

  // prologue: stage 0, A rows by group 0 and W rows by group 1
  if (g == 0) issue(I8{}, 0, rA, 0, 0);
  else issue(I8{}, 0, rW, 32, 0);
  BI_WAIT_VMCNT(0);
  __builtin_amdgcn_s_barrier();
  if (g == 1) __builtin_amdgcn_s_barrier();   // phase 0: group 0 alone
  // one line stage: its memory phase, then its MFMA phase.  `tail` (the last
  // stage): units at k >= K enter both operands as zeros, and a stage with a
  // single K-tile runs only its MFMAs.
  auto step = [&](int L, bool tail) {
    const uint32_t sb = lds0 + (L % NS) * STAGE + (8 * g) * 2048;
    const uint32_t sw = lds0 + (L % NS) * STAGE + 32 * 1024 + (4 * wn) * 2048;
    const bool two = 2 * L + 1 < KT;
    lds_read_8_4_nowait(a0, b0, sb + off0, sw + off0);
    if (two) lds_read_8_4_nowait(a1, b1, sb + off1, sw + off1);
    if (L + 1 < NLS) {
      if (g == 0) {
        issue(I8{}, L + 1, rW, 32, 0);
        issue(I4{}, L + 1, rA, 0, 0);
      } else {
        issue(I4{}, L + 1, rA, 0, 16);
      }
    }
    lds_wait_8_4(a0, b0);
    if (two) lds_wait_8_4(a1, b1);
    if (tail) {
      const u32x4_t zero = {0, 0, 0, 0};
      const bool z0 = 2 * L * 32 + 8 * (lane >> 4) >= K;
      const bool z1 = (2 * L + 1) * 32 + 8 * (lane >> 4) >= K;
#pragma unroll
      for (int i = 0; i < 8; ++i) a0[i] = z0 ? zero : a0[i], a1[i] = z1 ? zero : a1[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b0[j] = z0 ? zero : b0[j], b1[j] = z1 ? zero : b1[j];
    }
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma(a0[i], b0[j], acc[i][j]);
    if (two) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma(a1[i], b1[j], acc[i][j]);
    }
    BI_WAIT_VMCNT(0);   // this group's copies of stage L + 1
    // the last phase (group 1's last MFMAs) ends without a barrier: group 0
    // goes on to its stores
    if (g == 0 || L + 1 < NLS) __builtin_amdgcn_s_barrier();
  };
  for (int L = 0; L < NLS - 1; ++L) step(L, false);
  step(NLS - 1, true);
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      store_tile<OUTF32>(C, acc[i][j], m0 + (8 * g + i) * 16, n0 + (4 * wn + j) * 16, M, N,
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

// Split-K for the batch-adaptive twin only: `splits` workgroup slices of
// kslice columns of K (a multiple of 64), with the tile shape the twin picks
// (mb 8-row blocks, ct 16-column strips); slice j writes its fp32 partial
// sums to C32 + j M N.  Returns false for a shape it was not built for.
bool gemm_splitk_slices(const void* A, const void* W, float* C32, int M, int N, int K, int mb,
                        int ct, int splits, int kslice, hipStream_t s) {
  const RopeArgs ra{};
#define BI_SK(MB_, CT_)                                                              \
  if (mb == MB_ && ct == CT_) {                                                      \
    launch_small_k<MB_, CT_, 2>(A, W, C32, M, N, K, s, splits, kslice, ra);          \
    return true;                                                                     \
  }
#define BI_SK_M(MB_) BI_SK(MB_, 2) BI_SK(MB_, 4) BI_SK(MB_, 8)
  BI_SK_M(1) BI_SK_M(2) BI_SK_M(4) BI_SK_M(8)
#undef BI_SK_M
#undef BI_SK
  return false;
}

// Which kernel runs never changes a bit (every path keeps the same chain per
// element); the choice is speed alone.  Measured at N 4096-14336 and K
// 4096-14336 for 64 < M <= 1000: the skinny kernel takes about 0.48 ns x its
// cost x K and the large-tile kernel about 19 ns x its rounds of 256 tiles x
// K, and the 128-tile kernel was never the faster of the three.  So beyond 64
// rows the skinny kernel runs while its cost stays under 40 x the large-tile
// rounds; the 128-tile kernel remains for N < 2048.
void gemm_dispatch(const void* A, const void* W, void* C, int M, int N, int K, int out_f32,
                   hipStream_t s) {
  // (the large-tile kernel's buffers hold 256 rows of K: byte counts < 2^31)
  const bool big_ok = N >= 2048 && K < (1 << 22);
  bool small = M <= 64;
  if (!small && big_ok) {
    const long rounds = (((long)(M + 255) / 256) * ((N + 255) / 256) + 255) / 256;
    small = small_shape(M, N).cost < 40 * rounds;
  }
  if (small) {
    if (out_f32) dispatch_small<1>(A, W, C, M, N, K, s);
    else dispatch_small<0>(A, W, C, M, N, K, s);
  } else if (big_ok) {
    if (out_f32) launch_big<1>(A, W, C, M, N, K, s);
    else launch_big<0>(A, W, C, M, N, K, s);
  } else {
    if (out_f32) launch_tiled<1>(A, W, C, M, N, K, s);
    else launch_tiled<0>(A, W, C, M, N, K, s);
  }
}

// Packs a row-major bf16 [N][K] into the layout of wp_off: one thread per
// 16-byte unit of the packed weight (unit u: block u / 128 = (panel, K step,
// 16-row block of the panel), row (u % 128) / 8 of the block, 8 k at (u % 8)
// * 8); units past N or K are zeros.
__global__ __launch_bounds__(256) void k_pack_weight(const uint16_t* __restrict__ W,
                                                     uint16_t* __restrict__ P, int N, int K,
                                                     int kb, long units) {
  const long u = (long)blockIdx.x * 256 + threadIdx.x;
  if (u >= units) return;
  const long blk = u >> 7;
  const long pk = blk >> 4;   // panel * kb + K step
  const int panel = (int)(pk / kb), ks = (int)(pk - (long)panel * kb);
  const int n = panel * 256 + (int)(blk & 15) * 16 + (int)((u & 127) >> 3);
  const int k = ks * 64 + (int)(u & 7) * 8;
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (n < N && k < K) v = *reinterpret_cast<const u32x4_t*>(W + (long)n * K + k);
  reinterpret_cast<u32x4_t*>(P)[u] = v;
}

}  // namespace bi

extern "C" size_t bi_packed_weight_bytes(int N, int K) {
  if (N < 1 || K < 1) return 0;
  return (size_t)((K + 63) / 64) * (size_t)((N + 255) / 256) * 32768;
}

extern "C" bi_status bi_pack_weight(const void* W, void* Wp, int N, int K, bi_stream stream) {
  using namespace bi;
  BI_REQUIRE(N >= 1 && K >= 1, BI_ERR_INVALID, "bi_pack_weight: bad shape N=%d K=%d", N, K);
  BI_REQUIRE(K % 8 == 0, BI_ERR_UNSUPPORTED, "bi_pack_weight: bf16 needs K %% 8 == 0 (K=%d)", K);
  BI_REQUIRE(W && Wp && aligned16(W) && aligned16(Wp), BI_ERR_INVALID,
             "bi_pack_weight: null or misaligned pointer");
  const long units = (long)bi_packed_weight_bytes(N, K) / 16;
  BI_REQUIRE(units / 256 < 0x7fffffffL, BI_ERR_INVALID, "bi_pack_weight: too large");
  hipLaunchKernelGGL(k_pack_weight, dim3((unsigned)((units + 255) / 256)), dim3(256), 0,
                     as_stream(stream), (const uint16_t*)W, (uint16_t*)Wp, N, K, (K + 63) / 64,
                     units);
  return launched("bi_pack_weight");
}

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

extern "C" bi_status bi_gemm_swiglu(const void* A, const void* W, void* act, int M, int I, int K,
                                    bi_stream stream) {
  using namespace bi;
  BI_REQUIRE(M >= 0 && M <= 64 && I >= 8 && I % 8 == 0 && K >= 8 && K % 8 == 0,
             BI_ERR_INVALID, "bi_gemm_swiglu: need 0 <= M <= 64, I %% 8 == 0, K %% 8 == 0 "
             "(M=%d I=%d K=%d)", M, I, K);
  if (M == 0) return BI_OK;
  BI_REQUIRE(A && W && act, BI_ERR_INVALID, "bi_gemm_swiglu: null pointer");
  BI_REQUIRE(aligned16(A) && aligned16(W) && aligned16(act), BI_ERR_INVALID,
             "bi_gemm_swiglu: pointers must be 16-byte aligned");
  BI_REQUIRE(2L * I * K < (1L << 40), BI_ERR_INVALID, "bi_gemm_swiglu: tensor too large");
  dispatch_small<3>(A, W, act, M, 2 * I, K, as_stream(stream));
  return launched("bi_gemm_swiglu");
}

extern "C" bi_status bi_gemm_qkv_rope(const void* A, const void* W, int M, int K, int h,
                                      int h_kv, int d_h, const int32_t* pos, const float* cos_t,
                                      const float* sin_t, const int32_t* slot_mapping,
                                      int page_size, void* q_out, void* k_pool, void* v_pool,
                                      bi_stream stream) {
  using namespace bi;
  BI_REQUIRE(M >= 0 && M <= 64 && K >= 8 && K % 8 == 0 && h >= 1 && h_kv >= 1 && d_h >= 16 &&
                 d_h % 16 == 0 && page_size >= 1,
             BI_ERR_INVALID, "bi_gemm_qkv_rope: need 0 <= M <= 64, K %% 8 == 0, d_h %% 16 == 0 "
             "(M=%d K=%d d_h=%d)", M, K, d_h);
  BI_REQUIRE((cos_t == nullptr) == (sin_t == nullptr), BI_ERR_INVALID,
             "bi_gemm_qkv_rope: cos_t and sin_t must both be given or both be NULL");
  if (M == 0) return BI_OK;
  BI_REQUIRE(A && W && slot_mapping && q_out && k_pool && v_pool && (pos || !cos_t),
             BI_ERR_INVALID, "bi_gemm_qkv_rope: null pointer");
  BI_REQUIRE(aligned16(A) && aligned16(W), BI_ERR_INVALID,
             "bi_gemm_qkv_rope: A and W must be 16-byte aligned");
  const long N = (long)(h + 2 * h_kv) * d_h;
  BI_REQUIRE(N * K < (1L << 40) && N < (1L << 30), BI_ERR_INVALID,
             "bi_gemm_qkv_rope: tensor too large");
  RopeArgs ra{pos, cos_t, sin_t, slot_mapping, q_out, k_pool, v_pool, page_size, h, h_kv, d_h};
  dispatch_small<4>(A, W, nullptr, M, (int)N, K, as_stream(stream), 1, 0, ra);
  return launched("bi_gemm_qkv_rope");
}

// ---------------------------------------------------------------------------
// The same three products with the residual add and RMSNorm in the prologue
// (k_gemm_norm): a few rows only.
// ---------------------------------------------------------------------------
namespace bi {

// Compute units of the current device (queried once per device).
static int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev < 0 || dev >= 64) dev = 0;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

template <bool ADD, int OUTF32, int WD>
static void launch_norm(const NormArgs& na, const void* W, void* C, int M, int N, int K,
                        hipStream_t s, const RopeArgs& ra) {
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)k_gemm_norm<ADD, OUTF32, WD>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, kNormLdsMax);
    attr = true;
  }
  const int lds = norm_ring_bytes(WD) + M * (((K + 63) / 64) * 128) + 64;
  const int strips = (N + 15) / 16;
  const int grid = std::min(strips, 2 * device_cus());
  hipLaunchKernelGGL((k_gemm_norm<ADD, OUTF32, WD>), dim3(grid), dim3(kNormThreads), lds, s, na,
                     (const uint16_t*)W, C, M, N, K, ra);
}

template <int OUTF32>
static void dispatch_norm(const NormArgs& na, const void* W, void* C, int M, int N, int K,
                          hipStream_t s, const RopeArgs& ra = RopeArgs{}) {
  if (M <= 2) {
    if (na.o) launch_norm<true, OUTF32, 7>(na, W, C, M, N, K, s, ra);
    else launch_norm<false, OUTF32, 7>(na, W, C, M, N, K, s, ra);
  } else {
    if (na.o) launch_norm<true, OUTF32, 5>(na, W, C, M, N, K, s, ra);
    else launch_norm<false, OUTF32, 5>(na, W, C, M, N, K, s, ra);
  }
}

// Checks shared by the three entry points; returns BI_OK or the status set.
static bi_status check_norm(const char* fn, const void* h, const void* o, const void* gamma,
                            float eps, const void* h_out, const void* x_out, const void* W,
                            int M, int K) {
  BI_REQUIRE(M >= 0 && K >= 8 && K % 8 == 0, BI_ERR_INVALID,
             "%s: need M >= 0, K >= 8, K %% 8 == 0 (M=%d K=%d)", fn, M, K);
  BI_REQUIRE(M <= kNormRows && K <= kNormMaxK, BI_ERR_UNSUPPORTED,
             "%s: at most %d rows and K <= %d (M=%d K=%d); larger: the norm, then the product",
             fn, kNormRows, kNormMaxK, M, K);
  BI_REQUIRE((o == nullptr) == (h_out == nullptr), BI_ERR_INVALID,
             "%s: o and h_out must both be given or both be NULL", fn);
  BI_REQUIRE(eps >= 0.0f, BI_ERR_INVALID, "%s: eps must be >= 0", fn);
  if (M == 0) return BI_OK;
  BI_REQUIRE(h && gamma && W, BI_ERR_INVALID, "%s: null pointer", fn);
  BI_REQUIRE(aligned16(h) && aligned16(gamma) && aligned16(W) && aligned16(o) &&
                 aligned16(h_out) && aligned16(x_out),
             BI_ERR_INVALID, "%s: pointers must be 16-byte aligned", fn);
  BI_REQUIRE(!h_out || (h_out != h && h_out != o), BI_ERR_INVALID,
             "%s: h_out must not alias h or o", fn);
  BI_REQUIRE(!x_out || (x_out != h && x_out != o && x_out != h_out), BI_ERR_INVALID,
             "%s: x_out must not alias h, o or h_out", fn);
  return BI_OK;
}

}  // namespace bi

extern "C" bi_status bi_norm_gemm(const void* h, const void* o, const void* gamma, float eps,
                                  void* h_out, void* x_out, const void* W, void* C, int M,
                                  int N, int K, int out_dtype, bi_stream stream) {
  using namespace bi;
  const bi_status st = check_norm("bi_norm_gemm", h, o, gamma, eps, h_out, x_out, W, M, K);
  if (st != BI_OK || M == 0) return st;
  BI_REQUIRE(N >= 1 && C, BI_ERR_INVALID, "bi_norm_gemm: N >= 1 and C needed (N=%d)", N);
  BI_REQUIRE(aligned16(C), BI_ERR_INVALID, "bi_norm_gemm: C must be 16-byte aligned");
  BI_REQUIRE(out_dtype == BI_BF16 || out_dtype == BI_F32, BI_ERR_UNSUPPORTED,
             "bi_norm_gemm: out_dtype %d not supported", out_dtype);
  BI_REQUIRE((long)N * K < (1L << 40), BI_ERR_INVALID, "bi_norm_gemm: tensor too large");
  const NormArgs na{(const uint16_t*)h, (const uint16_t*)o, (const uint16_t*)gamma,
                    (uint16_t*)h_out, (uint16_t*)x_out, eps};
  if (out_dtype == BI_F32) dispatch_norm<1>(na, W, C, M, N, K, as_stream(stream));
  else dispatch_norm<0>(na, W, C, M, N, K, as_stream(stream));
  return launched("bi_norm_gemm");
}

extern "C" bi_status bi_norm_gemm_swiglu(const void* h, const void* o, const void* gamma,
                                         float eps, void* h_out, void* x_out, const void* W,
                                         void* act, int M, int I, int K, bi_stream stream) {
  using namespace bi;
  const bi_status st =
      check_norm("bi_norm_gemm_swiglu", h, o, gamma, eps, h_out, x_out, W, M, K);
  if (st != BI_OK || M == 0) return st;
  BI_REQUIRE(I >= 8 && I % 8 == 0 && act, BI_ERR_INVALID,
             "bi_norm_gemm_swiglu: need I %% 8 == 0 and act (I=%d)", I);
  BI_REQUIRE(aligned16(act), BI_ERR_INVALID, "bi_norm_gemm_swiglu: act must be 16-byte aligned");
  BI_REQUIRE(2L * I * K < (1L << 40), BI_ERR_INVALID, "bi_norm_gemm_swiglu: tensor too large");
  const NormArgs na{(const uint16_t*)h, (const uint16_t*)o, (const uint16_t*)gamma,
                    (uint16_t*)h_out, (uint16_t*)x_out, eps};
  dispatch_norm<3>(na, W, act, M, 2 * I, K, as_stream(stream));
  return launched("bi_norm_gemm_swiglu");
}

extern "C" bi_status bi_norm_gemm_qkv_rope(const void* h, const void* o, const void* gamma,
                                           float eps, void* h_out, void* x_out, const void* W,
                                           int M, int K, int nh, int h_kv, int d_h,
                                           const int32_t* pos, const float* cos_t,
                                           const float* sin_t, const int32_t* slot_mapping,
                                           int page_size, void* q_out, void* k_pool,
                                           void* v_pool, bi_stream stream) {
  using namespace bi;
  const bi_status st =
      check_norm("bi_norm_gemm_qkv_rope", h, o, gamma, eps, h_out, x_out, W, M, K);
  if (st != BI_OK) return st;
  BI_REQUIRE(nh >= 1 && h_kv >= 1 && d_h >= 16 && d_h % 16 == 0 && page_size >= 1,
             BI_ERR_INVALID, "bi_norm_gemm_qkv_rope: need d_h %% 16 == 0 (d_h=%d)", d_h);
  BI_REQUIRE((cos_t == nullptr) == (sin_t == nullptr), BI_ERR_INVALID,
             "bi_norm_gemm_qkv_rope: cos_t and sin_t must both be given or both be NULL");
  if (M == 0) return BI_OK;
  BI_REQUIRE(slot_mapping && q_out && k_pool && v_pool && (pos || !cos_t), BI_ERR_INVALID,
             "bi_norm_gemm_qkv_rope: null pointer");
  const long N = (long)(nh + 2 * h_kv) * d_h;
  BI_REQUIRE(N * K < (1L << 40) && N < (1L << 30), BI_ERR_INVALID,
             "bi_norm_gemm_qkv_rope: tensor too large");
  const NormArgs na{(const uint16_t*)h, (const uint16_t*)o, (const uint16_t*)gamma,
                    (uint16_t*)h_out, (uint16_t*)x_out, eps};
  RopeArgs ra{pos, cos_t, sin_t, slot_mapping, q_out, k_pool, v_pool, page_size, nh, h_kv, d_h};
  dispatch_norm<4>(na, W, nullptr, M, (int)N, K, as_stream(stream), ra);
  return launched("bi_norm_gemm_qkv_rope");
}
