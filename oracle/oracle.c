/*
 * oracle.c -- plain, slow CPU oracle for the batch-invariant forward-pass
 * reductions.  TEST INFRASTRUCTURE ONLY: it is loaded by the test-suite, by
 * the package smoke check and by the benchmark's CPU-baseline leg, never by
 * the product path.  It shares no source, header or table with the HIP
 * library.
 *
 * What it computes (sources are the pages' titles and sections):
 *  - "Lockstep", section "The fix": every reduction of the forward pass runs
 *    in one fixed order with fixed split points that do not depend on the
 *    batch; attention splits come from the request's own length.
 *  - "Batch invariance and reproducible inference", sections
 *    "Non-associativity, concretely" (Figure 1: different trees give
 *    different binary32 sums), "1 . Split-K and segmented attention
 *    reductions" (split count = ceil(seq_len / split tile), independent of
 *    the batch), "From batch size to reduction tree" (fp32 partials added by
 *    a merge step), and the closing list of dull one-block-per-row kernels
 *    (rms_norm, log_softmax) and the fixed-K-order persistent matmul.
 *
 * The pages fix that order is fixed, not which order.  The order written
 * here is the one this project chose for every reduction; each function
 * spells it out.  All arithmetic is IEEE binary32 with round-to-nearest-even,
 * fused multiply-add only where fmaf() is written, built with
 * -ffp-contract=off and without fast-math.  Values of bf16 tensors are passed
 * in widened to float (exact); results that the kernels store in bf16 are
 * rounded here by bf16_rne() and handed back as floats.
 *
 * Parallelism: OpenMP splits only independent rows / heads / output
 * elements; no reduction is ever split across threads.
 *
 * Parity status: RMSNorm, fp32 GEMM, attention partials, merge, prefill and
 * the glue functions are pinned by the tests (fp64 brute force within
 * Higham-style bounds, closed forms, the Figure 1 witness, integer-exact
 * GEMMs).  None is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* scalar helpers                                                      */
/* ------------------------------------------------------------------ */

static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* Narrow binary32 to bfloat16 with round-to-nearest-even; the result is
 * returned widened back to float.  NaN stays a (quiet) NaN. */
float oracle_bf16_rne(float x)
{
    uint32_t u = f2u(x);
    if ((u & 0x7f800000u) == 0x7f800000u) {
        if (u & 0x007fffffu)
            return u2f((u | 0x00400000u) & 0xffff0000u);
        return u2f(u & 0xffff0000u);
    }
    u = (u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u;
    return u2f(u);
}

static float out_round(float x, int round_bf16)
{
    return round_bf16 ? oracle_bf16_rne(x) : x;
}

/* 2^k as a float for k in [-126, 127] (exact). */
static float pow2i(int k) { return u2f((uint32_t)(k + 127) << 23); }

/*
 * Natural exponential in binary32.  The pages do not name an exp routine;
 * the softmax and SiLU steps need one that both sides of the parity check
 * evaluate identically, so the project fixes this one (Cody & Waite range
 * reduction, "Software Manual for the Elementary Functions", 1980, followed
 * by the degree-7 Taylor polynomial of e^r in Horner form):
 *   n  = rint(x * log2(e))                 (binary32 multiply, RNE rint)
 *   r  = fma(-n, LN2_HI, x); r = fma(-n, LN2_LO, r)
 *   p  = sum_{i=0..7} r^i / i!             (Horner, fma at every step)
 *   result = (p * 2^floor-half(n)) * 2^(n - half)
 * LN2_HI carries 15 significant bits so n * LN2_HI is exact for |n| < 512;
 * LN2_LO = fp32(ln 2 - LN2_HI).  |r| <= ln(2)/2 so the truncation error of
 * the polynomial is below 2^-27 relative.  Inputs below -104 give +0 and
 * above 88.75 give +inf.
 */
#define EXP_LOG2E  1.44269502162933349609375f     /* fp32(log2 e) */
#define EXP_LN2_HI 0.693145751953125f              /* 0x3f317200 */
#define EXP_LN2_LO 1.428606765330187045037746429443359375e-06f
float oracle_exp(float x)
{
    if (x != x) return x;
    if (x > 88.75f) return INFINITY;
    if (x < -104.0f) return 0.0f;
    float n = rintf(x * EXP_LOG2E);
    float r = fmaf(-n, EXP_LN2_HI, x);
    r = fmaf(-n, EXP_LN2_LO, r);
    float p = 1.0f / 5040.0f;
    p = fmaf(p, r, 1.0f / 720.0f);
    p = fmaf(p, r, 1.0f / 120.0f);
    p = fmaf(p, r, 1.0f / 24.0f);
    p = fmaf(p, r, 1.0f / 6.0f);
    p = fmaf(p, r, 0.5f);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    int ni = (int)n;
    int n1 = ni / 2;          /* C division truncates toward zero */
    int n2 = ni - n1;
    p = p * pow2i(n1);
    p = p * pow2i(n2);
    return p;
}

void oracle_exp_vec(const float *x, float *y, long n)
{
#pragma omp parallel for schedule(static)
    for (long i = 0; i < n; ++i) y[i] = oracle_exp(x[i]);
}

/* In-place xor butterfly on n values (n a power of two): for each mask m in
 * order, every slot i becomes a[i] + a[i ^ m].  Both slots of a pair compute
 * the same sum (binary32 addition commutes), so after the last mask every
 * slot holds the same value; slot 0 is returned.  This is the tree a
 * wavefront builds with lane exchanges. */
static float xor_butterfly(float *a, int n, const int *masks, int nm)
{
    float tmp[64];
    for (int s = 0; s < nm; ++s) {
        int m = masks[s];
        for (int i = 0; i < n; ++i) tmp[i] = a[i] + a[i ^ m];
        memcpy(a, tmp, sizeof(float) * (size_t)n);
    }
    return a[0];
}

/* Exposed reduction primitives (used by the Figure 1 witness check). */
float oracle_sum_serial(const float *x, int n)
{
    float s = x[0];
    for (int i = 1; i < n; ++i) s = s + x[i];
    return s;
}

/* Pairwise tree over n = 2^k values, adjacent pairs first:
 * ((x0+x1)+(x2+x3))+... -- Figure 1's "pairwise" grouping for n = 4. */
float oracle_sum_pairwise(const float *x, int n)
{
    float a[64];
    memcpy(a, x, sizeof(float) * (size_t)n);
    for (int w = n; w > 1; w /= 2)
        for (int i = 0; i < w / 2; ++i) a[i] = a[2 * i] + a[2 * i + 1];
    return a[0];
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* RMSNorm -- one row, one fixed tree                                  */
/* ------------------------------------------------------------------ */
/*
 * y = x * (1 / sqrt(mean(x^2) + eps)) * gamma, per row of d elements
 * ("Batch invariance and reproducible inference": rms_norm is one of the
 * dull one-block-per-row kernels with no cross-block reduction; "Lockstep",
 * "The fix": fixed order regardless of batch shape).
 *
 * Fixed order of the sum of squares:
 *   - the row is cut into vectors of 8 consecutive elements, vector v holding
 *     elements 8v .. 8v+7 (the tail vector is short);
 *   - 256 lanes; lane t visits vectors t, t+256, t+512, ... in that order and
 *     each vector's elements in index order: a_t = fma(x, x, a_t) from +0;
 *   - lanes 64w .. 64w+63 form wave w; each wave is reduced by the xor
 *     butterfly with masks 32, 16, 8, 4, 2, 1;
 *   - the four wave sums are added serially: ((w0 + w1) + w2) + w3.
 * Then mean = ss / d, r = 1 / sqrt(mean + eps) (each step correctly rounded)
 * and y_i = round((x_i * r) * gamma_i).
 */
void oracle_rmsnorm(const float *x, const float *gamma, float *y,
                    int M, int d, float eps, int round_bf16)
{
    static const int masks[6] = {32, 16, 8, 4, 2, 1};
#pragma omp parallel for schedule(dynamic)
    for (int row = 0; row < M; ++row) {
        const float *xr = x + (size_t)row * d;
        float *yr = y + (size_t)row * d;
        float lane[256];
        int nv = (d + 7) / 8;
        for (int t = 0; t < 256; ++t) {
            float a = 0.0f;
            for (int v = t; v < nv; v += 256)
                for (int e = 0; e < 8; ++e) {
                    int i = 8 * v + e;
                    if (i < d) a = fmaf(xr[i], xr[i], a);
                }
            lane[t] = a;
        }
        float ws[4];
        for (int w = 0; w < 4; ++w) ws[w] = xor_butterfly(lane + 64 * w, 64, masks, 6);
        float ss = ((ws[0] + ws[1]) + ws[2]) + ws[3];
        float mean = ss / (float)d;
        float r = 1.0f / sqrtf(mean + eps);
        for (int i = 0; i < d; ++i) yr[i] = out_round((xr[i] * r) * gamma[i], round_bf16);
    }
}

/* ------------------------------------------------------------------ */
/* GEMM -- C = A W^T, one ascending K chain per element                */
/* ------------------------------------------------------------------ */
/*
 * C[i][j] = sum_k A[i][k] * W[j][k], A [M][K], W [N][K], C [M][N], computed
 * as acc = +0; for k = 0 .. K-1: acc = fma(A[i][k], W[j][k], acc).  One
 * chain per output element in one fixed order, no split of K and nothing
 * that depends on M ("Batch invariance and reproducible inference",
 * "2 . Cross-block accumulation": split-K leaves the order undefined; the
 * persistent matmul accumulates its K loop in one fixed order per tile;
 * "3 . Kernel selection changing with shape": the config must not read M).
 */
void oracle_gemm(const float *A, const float *W, float *C,
                 int M, int N, int K, int round_bf16)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int i = 0; i < M; ++i)
        for (int j = 0; j < N; ++j) {
            const float *a = A + (size_t)i * K;
            const float *w = W + (size_t)j * K;
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) acc = fmaf(a[k], w[k], acc);
            C[(size_t)i * N + j] = out_round(acc, round_bf16);
        }
}

/* ------------------------------------------------------------------ */
/* split-KV attention: one chunk partial                               */
/* ------------------------------------------------------------------ */

/* Address of the d_h-vector of token j of kv head g in a paged pool laid out
 * [page][h_kv][page_size][d_h]; bt is the request's block-table row. */
static const float *kv_row(const float *pool, const int32_t *bt, int j,
                           int g, int h_kv, int page_size, int d_h)
{
    int page = bt[j / page_size];
    int slot = j % page_size;
    return pool + (((size_t)page * h_kv + g) * page_size + slot) * (size_t)d_h;
}

/*
 * Partial of one chunk for one query head ("Lockstep", "The fix": attention
 * split points come from the request; "Batch invariance and reproducible
 * inference", "1 . Split-K and segmented attention reductions": each split
 * covers split_tile tokens; "From batch size to reduction tree": fp32
 * partials are combined by a merge step).  Keys j0 .. j0+n-1, with
 * 1 <= n <= chunk length:
 *   S_u = fl(dot(q, k_u)) * scale, dot serial over d = 0 .. d_h-1 in fma;
 *   m   = max_u S_u, then m + 0 (turns -0 into +0);
 *   p_u = exp(S_u - m)                        (oracle_exp);
 *   with p_bf16, p_u = bf16(p_u): the weights a matrix-core PV product
 *     consumes (the multiply-accumulate order below is then the oracle's own;
 *     a matrix core sums in its hardware order, so parity is the derived
 *     tolerance, or exact where every partial sum is exact);
 *   keys in blocks of 64 (u = 0..63, 64..127, ...): inside block b,
 *     L_b = serial sum of p_u (L = L + p_u from +0), and
 *     A_b[d] = serial fma(p_u, v_u[d], A_b[d]) from +0, u ascending;
 *   l = ((L_0 + L_1) + L_2) + ...,  acc[d] = ((A_0 + A_1) + A_2) + ...
 */
static void attn_chunk_partial(const float *q, const float *k_pool, const float *v_pool,
                               const int32_t *bt, int g, int h_kv, int page_size, int d_h,
                               int j0, int n, float scale,
                               float *m_out, float *l_out, float *acc_out,
                               float *S, float *blk /* [d_h] scratch */, int p_bf16)
{
    for (int u = 0; u < n; ++u) {
        const float *k = kv_row(k_pool, bt, j0 + u, g, h_kv, page_size, d_h);
        float dot = 0.0f;
        for (int d = 0; d < d_h; ++d) dot = fmaf(q[d], k[d], dot);
        S[u] = dot * scale;
    }
    float m = S[0];
    for (int u = 1; u < n; ++u) if (S[u] > m) m = S[u];
    m = m + 0.0f;
    for (int u = 0; u < n; ++u) S[u] = oracle_exp(S[u] - m);   /* S now holds p */
    if (p_bf16)  /* weights carried in bf16 (matrix-core PV): P = bf16(p) */
        for (int u = 0; u < n; ++u) S[u] = oracle_bf16_rne(S[u]);

    float l = 0.0f;
    for (int b = 0; b * 64 < n; ++b) {
        int u1 = (b + 1) * 64 < n ? (b + 1) * 64 : n;
        float L = 0.0f;
        for (int d = 0; d < d_h; ++d) blk[d] = 0.0f;
        for (int u = b * 64; u < u1; ++u) {
            const float *v = kv_row(v_pool, bt, j0 + u, g, h_kv, page_size, d_h);
            L = L + S[u];
            for (int d = 0; d < d_h; ++d) blk[d] = fmaf(S[u], v[d], blk[d]);
        }
        if (b == 0) {
            l = L;
            for (int d = 0; d < d_h; ++d) acc_out[d] = blk[d];
        } else {
            l = l + L;
            for (int d = 0; d < d_h; ++d) acc_out[d] = acc_out[d] + blk[d];
        }
    }
    *m_out = m;
    *l_out = l;
}

/* Number of chunks of a request with kv_len tokens: ceil(kv_len / chunk)
 * ("Batch invariance and reproducible inference", "1 . Split-K and
 * segmented attention reductions": s = 2560 with a 256 tile gives 10 splits
 * alone or in any batch). */
int oracle_num_chunks(int kv_len, int chunk)
{
    return (kv_len + chunk - 1) / chunk;
}

/*
 * Decode partials for B requests.  q [B][h][d_h]; request r has kv_len[r]
 * tokens (the current one included), chunk c covering absolute positions
 * [c*chunk, min((c+1)*chunk, kv_len)).  Partial rows are numbered
 * chunk_off[r] + c, chunk_off the prefix sum of the per-request chunk counts.
 * part_ml [rows][h][2] holds (m, l), part_acc [rows][h][d_h] holds acc.
 * q head i reads kv head i / (h / h_kv) (contiguous query groups).
 */
void oracle_decode_partials(const float *q, const float *k_pool, const float *v_pool,
                            const int32_t *block_table, const int32_t *kv_len,
                            const int32_t *chunk_off, int B, int h, int h_kv, int d_h,
                            int page_size, int max_pages, int chunk, float scale,
                            float *part_ml, float *part_acc, int p_bf16)
{
    int group = h / h_kv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int r = 0; r < B; ++r)
        for (int hi = 0; hi < h; ++hi) {
            float *S = (float *)malloc(sizeof(float) * (size_t)chunk);
            float *blk = (float *)malloc(sizeof(float) * (size_t)d_h);
            const int32_t *bt = block_table + (size_t)r * max_pages;
            int nch = oracle_num_chunks(kv_len[r], chunk);
            for (int c = 0; c < nch; ++c) {
                int j0 = c * chunk;
                int n = kv_len[r] - j0 < chunk ? kv_len[r] - j0 : chunk;
                size_t row = (size_t)(chunk_off[r] + c) * h + hi;
                attn_chunk_partial(q + ((size_t)r * h + hi) * d_h, k_pool, v_pool, bt,
                                   hi / group, h_kv, page_size, d_h, j0, n, scale,
                                   &part_ml[2 * row], &part_ml[2 * row + 1],
                                   &part_acc[row * d_h], S, blk, p_bf16);
            }
            free(S);
            free(blk);
        }
}

/*
 * Serial merge of one (request, head): chunks c = 0 .. n-1 in order
 * ("From batch size to reduction tree": the merge adds the fp32 partials;
 * the combine is the rescaled softmax merge):
 *   (M, L, Acc) = (m_0, l_0, acc_0);
 *   for c >= 1: M' = max(M, m_c); a = exp(M - M'); b = exp(m_c - M');
 *               L = fma(l_c, b, L * a); Acc[d] = fma(acc_c[d], b, Acc[d] * a);
 *               M = M'
 *   out[d] = round(Acc[d] / L)
 */
static void merge_one(const float *ml, const float *acc, int n, int h, int d_h,
                      float *out, int round_bf16)
{
    float M = ml[0], L = ml[1];
    float Acc[512];
    for (int d = 0; d < d_h; ++d) Acc[d] = acc[d];
    for (int c = 1; c < n; ++c) {
        const float *mlc = ml + (size_t)c * h * 2;
        const float *accc = acc + (size_t)c * h * d_h;
        float mc = mlc[0];
        float Mn = M > mc ? M : mc;
        float a = oracle_exp(M - Mn);
        float b = oracle_exp(mc - Mn);
        L = fmaf(mlc[1], b, L * a);
        for (int d = 0; d < d_h; ++d) Acc[d] = fmaf(accc[d], b, Acc[d] * a);
        M = Mn;
    }
    for (int d = 0; d < d_h; ++d) out[d] = out_round(Acc[d] / L, round_bf16);
}

void oracle_merge_partials(const float *part_ml, const float *part_acc,
                           const int32_t *chunk_off, int B, int h, int d_h,
                           float *out, int round_bf16)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int r = 0; r < B; ++r)
        for (int hi = 0; hi < h; ++hi) {
            size_t row0 = (size_t)chunk_off[r] * h + hi;
            merge_one(part_ml + 2 * row0, part_acc + row0 * d_h,
                      chunk_off[r + 1] - chunk_off[r], h, d_h,
                      out + ((size_t)r * h + hi) * d_h, round_bf16);
        }
}

/*
 * Causal prefill over packed query rows.  Request r owns rows
 * q_start[r] .. q_start[r+1]-1; row t sits at absolute position
 * pos = q_pos0[r] + (t - q_start[r]) and attends to positions 0 .. pos,
 * which must already be in the pool.  Each row is computed exactly as a
 * decode of kv_len = pos + 1: chunks aligned at absolute multiples of the
 * chunk length, partials by attn_chunk_partial, then the serial merge --
 * so the result does not depend on how the prompt was cut into prefill
 * chunks ("Batch invariance and reproducible inference": chunked prefill
 * must not move the split boundaries; the pages snap the chunk length to a
 * multiple of the split tile, absolute alignment gives the same guarantee
 * for any cut).
 */
void oracle_prefill_attn(const float *q, const int32_t *q_start, const int32_t *q_pos0, int R,
                         const float *k_pool, const float *v_pool, const int32_t *block_table,
                         int h, int h_kv, int d_h, int page_size, int max_pages, int chunk,
                         float scale, float *out, int round_bf16, int p_bf16)
{
    int group = h / h_kv;
    int T = q_start[R];
#pragma omp parallel for schedule(dynamic)
    for (int t = 0; t < T; ++t) {
        int r = 0;
        while (q_start[r + 1] <= t) ++r;
        int pos = q_pos0[r] + (t - q_start[r]);
        int kvl = pos + 1;
        int nch = oracle_num_chunks(kvl, chunk);
        const int32_t *bt = block_table + (size_t)r * max_pages;
        float *ml = (float *)malloc(sizeof(float) * (size_t)nch * h * 2);
        float *acc = (float *)malloc(sizeof(float) * (size_t)nch * h * d_h);
        float *S = (float *)malloc(sizeof(float) * (size_t)chunk);
        float *blk = (float *)malloc(sizeof(float) * (size_t)d_h);
        for (int hi = 0; hi < h; ++hi) {
            for (int c = 0; c < nch; ++c) {
                int j0 = c * chunk;
                int n = kvl - j0 < chunk ? kvl - j0 : chunk;
                size_t row = (size_t)c * h + hi;
                attn_chunk_partial(q + ((size_t)t * h + hi) * d_h, k_pool, v_pool, bt,
                                   hi / group, h_kv, page_size, d_h, j0, n, scale,
                                   &ml[2 * row], &ml[2 * row + 1], &acc[row * d_h], S, blk,
                                   p_bf16);
            }
            merge_one(ml + 2 * hi, acc + (size_t)hi * d_h, nch, h, d_h,
                      out + ((size_t)t * h + hi) * d_h, round_bf16);
        }
        free(ml); free(acc); free(S); free(blk);
    }
}

/* ------------------------------------------------------------------ */
/* elementwise glue of a Llama-shaped layer (no reductions)            */
/* ------------------------------------------------------------------ */

/* Rotate-half RoPE on nh heads of d_h per row at position pos[row]:
 * for i < d_h/2 with a = x[i], b = x[i + d_h/2], c = cos[pos][i],
 * s = sin[pos][i]:  x'[i] = fma(a, c, -(b*s)),  x'[i+d_h/2] = fma(b, c, a*s).
 * cos/sin tables [P][d_h/2] are inputs.  (RoPE is not on the pages; it is
 * elementwise, so it has no order to fix.) */
void oracle_rope(const float *x, const int32_t *pos, const float *cos_t, const float *sin_t,
                 float *y, int M, int nh, int d_h, int round_bf16)
{
    int half = d_h / 2;
#pragma omp parallel for schedule(static)
    for (int row = 0; row < M; ++row)
        for (int hh = 0; hh < nh; ++hh) {
            const float *xr = x + ((size_t)row * nh + hh) * d_h;
            float *yr = y + ((size_t)row * nh + hh) * d_h;
            const float *c = cos_t + (size_t)pos[row] * half;
            const float *s = sin_t + (size_t)pos[row] * half;
            for (int i = 0; i < half; ++i) {
                float a = xr[i], b = xr[i + half];
                yr[i] = out_round(fmaf(a, c[i], -(b * s[i])), round_bf16);
                yr[i + half] = out_round(fmaf(b, c[i], a * s[i]), round_bf16);
            }
        }
}

/* y = round(a + b) elementwise (residual add). */
void oracle_add(const float *a, const float *b, float *y, long n, int round_bf16)
{
#pragma omp parallel for schedule(static)
    for (long i = 0; i < n; ++i) y[i] = out_round(a[i] + b[i], round_bf16);
}

/* SwiGLU: gu [M][2F] holds gate in columns 0..F-1 and up in F..2F-1;
 * y[i] = round((g / (1 + exp(-g))) * u). */
void oracle_silu_mul(const float *gu, float *y, int M, int F, int round_bf16)
{
#pragma omp parallel for schedule(static)
    for (int row = 0; row < M; ++row)
        for (int i = 0; i < F; ++i) {
            float g = gu[(size_t)row * 2 * F + i];
            float u = gu[(size_t)row * 2 * F + F + i];
            float s = g / (1.0f + oracle_exp(-g));
            y[(size_t)row * F + i] = out_round(s * u, round_bf16);
        }
}

/* Index of the largest value of each row; the lowest index wins ties. */
void oracle_argmax(const float *x, int32_t *idx, int M, int V)
{
#pragma omp parallel for schedule(static)
    for (int row = 0; row < M; ++row) {
        const float *xr = x + (size_t)row * V;
        int best = 0;
        for (int i = 1; i < V; ++i) if (xr[i] > xr[best]) best = i;
        idx[row] = best;
    }
}

/* ------------------------------------------------------------------ */
/* log-softmax (logprobs)                                              */
/* ------------------------------------------------------------------ */

/*
 * Natural log in binary32, fixed for the same reason as the exp (the pages
 * name no log routine; both sides of the parity check must evaluate the same
 * one).  x = 2^e * m with e and m taken from the bits, m in [1, 2); if m >
 * fp32(sqrt 2) then m = m / 2 and e = e + 1, so m lies in [sqrt(1/2),
 * sqrt(2)].  log m = 2 atanh(s), s = (m - 1) / (m + 1), |s| <= 0.1716, by the
 * series 2 s sum_{k=0..6} s^(2k) / (2k + 1) in Horner form in z = s^2 with
 * fma (the first omitted term, z^7 / 15, is below 2^-39 relative); then
 * log x = fma(e, LN2_HI, fma(e, LN2_LO, log m)) with the exp's split of ln 2.
 * Defined for positive normal x; +inf and NaN pass through.
 */
float oracle_log(float x)
{
    if (x != x || x == INFINITY) return x;
    uint32_t b = f2u(x);
    int e = (int)((b >> 23) & 0xffu) - 127;
    float m = u2f((b & 0x7fffffu) | 0x3f800000u);
    if (m > 1.41421353816986083984375f) { m = 0.5f * m; e = e + 1; }
    float s = (m - 1.0f) / (m + 1.0f);
    float z = s * s;
    float q = 1.0f / 13.0f;
    q = fmaf(q, z, 1.0f / 11.0f);
    q = fmaf(q, z, 1.0f / 9.0f);
    q = fmaf(q, z, 1.0f / 7.0f);
    q = fmaf(q, z, 1.0f / 5.0f);
    q = fmaf(q, z, 1.0f / 3.0f);
    q = fmaf(q, z, 1.0f);
    float lm = (s + s) * q;
    float fe = (float)e;
    return fmaf(fe, EXP_LN2_HI, fmaf(fe, EXP_LN2_LO, lm));
}

void oracle_log_vec(const float *x, float *y, long n)
{
#pragma omp parallel for schedule(static)
    for (long i = 0; i < n; ++i) y[i] = oracle_log(x[i]);
}

/*
 * y = (x - m) - log(sum exp(x - m)) per row, m the row maximum
 * ("Batch invariance and reproducible inference": the replacement
 * log_softmax of the dispatcher overrides, one block per row looping the row
 * serially; "Mathematically equivalent is not bitwise equivalent" for why
 * logprobs come from it).  The order is the one a block of 1024 threads
 * gives: thread t takes elements t, t + 1024, ... ascending -- their maximum
 * (a NaN never wins: v > m is false), then a serial binary32 sum of
 * exp(x - m); each wave of 64 threads adds its sums with the xor butterfly
 * (masks 32 .. 1) and the 16 wave sums are added in wave order.  A row with
 * no entry above -inf gives -inf throughout.
 */
void oracle_log_softmax(const float *x, float *y, int M, int V)
{
    static const int masks[6] = {32, 16, 8, 4, 2, 1};
#pragma omp parallel for schedule(dynamic)
    for (int row = 0; row < M; ++row) {
        const float *xr = x + (size_t)row * V;
        float *yr = y + (size_t)row * V;
        float m = -INFINITY;
        for (int i = 0; i < V; ++i) if (xr[i] > m) m = xr[i];
        float lane[1024];
        for (int t = 0; t < 1024; ++t) {
            float a = 0.0f;
            for (int i = t; i < V; i += 1024) a = a + oracle_exp(xr[i] - m);
            lane[t] = a;
        }
        float sum = 0.0f;
        for (int w = 0; w < 16; ++w) {
            float ws = xor_butterfly(lane + 64 * w, 64, masks, 6);
            sum = (w == 0) ? ws : sum + ws;
        }
        int none = (m == -INFINITY);
        float ls = oracle_log(sum);
        for (int i = 0; i < V; ++i) yr[i] = none ? -INFINITY : (xr[i] - m) - ls;
    }
}

/* ------------------------------------------------------------------ */
/* seeded sampling                                                     */
/* ------------------------------------------------------------------ */

/* MurmurHash3_x86_32 (Austin Appleby's public-domain definition) of the
 * 8-byte key made of the two little-endian 32-bit words w0, w1. */
static uint32_t rotl32(uint32_t x, int r) { return (x << r) | (x >> (32 - r)); }

uint32_t oracle_murmur3_2w(uint32_t seed, uint32_t w0, uint32_t w1)
{
    const uint32_t c1 = 0xcc9e2d51u, c2 = 0x1b873593u;
    uint32_t words[2] = {w0, w1};
    uint32_t h = seed;
    for (int i = 0; i < 2; ++i) {
        uint32_t k = words[i];
        k *= c1;
        k = rotl32(k, 15);
        k *= c2;
        h ^= k;
        h = rotl32(h, 13);
        h = h * 5u + 0xe6546b64u;
    }
    h ^= 8u;                       /* key length in bytes */
    h ^= h >> 16;
    h *= 0x85ebca6bu;
    h ^= h >> 13;
    h *= 0xc2b2ae35u;
    h ^= h >> 16;
    return h;
}

/* Binary64 natural log for the sampler, fixed like the binary32 one: x =
 * 2^e m, m in [sqrt(1/2), sqrt(2)], log m = 2 atanh(s), s = (m - 1)/(m + 1),
 * by 2 s sum_{k=0..11} z^k / (2k + 1), z = s^2, Horner with fma (the first
 * omitted term, z^12 / 25, is below 2^-60 relative); log x = fma(e, LN2H,
 * fma(e, LN2L, log m)) with LN2H the binary64 value of ln 2 with its last 21
 * mantissa bits cleared (e * LN2H exact) and LN2L = ln 2 - LN2H rounded.
 * Positive normal x only. */
double oracle_log64(double x)
{
    uint64_t b;
    memcpy(&b, &x, 8);
    int e = (int)((b >> 52) & 0x7ffu) - 1023;
    uint64_t mb = (b & 0xfffffffffffffULL) | 0x3ff0000000000000ULL;
    double m;
    memcpy(&m, &mb, 8);
    if (m > 1.4142135623730951) { m = 0.5 * m; e = e + 1; }
    double s = (m - 1.0) / (m + 1.0);
    double z = s * s;
    double q = 1.0 / 23.0;
    q = fma(q, z, 1.0 / 21.0);
    q = fma(q, z, 1.0 / 19.0);
    q = fma(q, z, 1.0 / 17.0);
    q = fma(q, z, 1.0 / 15.0);
    q = fma(q, z, 1.0 / 13.0);
    q = fma(q, z, 1.0 / 11.0);
    q = fma(q, z, 1.0 / 9.0);
    q = fma(q, z, 1.0 / 7.0);
    q = fma(q, z, 1.0 / 5.0);
    q = fma(q, z, 1.0 / 3.0);
    q = fma(q, z, 1.0);
    double lm = (s + s) * q;
    double fe = (double)e;
    return fma(fe, 6.93147180369123816490e-01, fma(fe, 1.90821492927058770002e-10, lm));
}

void oracle_log64_vec(const double *x, double *y, long n)
{
    for (long i = 0; i < n; ++i) y[i] = oracle_log64(x[i]);
}

/* Gumbel-max draw per row ("Batch invariance and reproducible inference",
 * "The weaker guarantees, which are usually enough": noise from a 32-bit
 * murmur hash of (seed, position, column) in float64): score_j =
 * x_j * (1 / T) + (-log(-log(u_j))), u_j = (hash(seed; pos, j) + 1/2) 2^-32,
 * all in binary64; the token is the first j with the largest score.  T <= 0:
 * the argmax of x. */
void oracle_sample(const float *x, const uint32_t *seed, const int32_t *pos, const float *temp,
                   int32_t *out, int M, int V)
{
#pragma omp parallel for schedule(dynamic)
    for (int row = 0; row < M; ++row) {
        const float *xr = x + (size_t)row * V;
        int noise = temp[row] > 0.0f;
        double invT = noise ? 1.0 / (double)temp[row] : 1.0;
        double best = -INFINITY;
        int bi = -1;
        for (int j = 0; j < V; ++j) {
            double sc = (double)xr[j] * invT;
            if (noise) {
                uint32_t h = oracle_murmur3_2w(seed[row], (uint32_t)pos[row], (uint32_t)j);
                double u = ((double)h + 0.5) * 0x1p-32;
                sc = sc + -oracle_log64(-oracle_log64(u));
            }
            if (bi < 0 || sc > best) { best = sc; bi = j; }
        }
        out[row] = bi < 0 ? 0 : bi;
    }
}
