/*
 * bi.h -- C ABI of libbi.so: batch-invariant forward-pass kernels for
 * MI355X (gfx950).
 *
 * The property every invariant entry point keeps ("Lockstep", sections "The
 * fix" and "Proving it"): the bits of output row r depend only on row r's
 * own inputs (and on the shared weights, or on request r's own KV pages) and
 * on the call's shape constants other than the batch -- never on how many
 * other rows share the call, their order, padding, or which physical pages
 * hold r's KV.  Every reduction runs in one fixed order with split points
 * fixed by the hidden size or by the request's own KV length.
 *
 * Each invariant entry point has a batch-adaptive "free" twin (suffix
 * _free) that computes the same mathematics but picks its split points and
 * tiles from the batch and the device's 256 compute units, as ordinary
 * serving kernels do ("Batch invariance and reproducible inference",
 * section "From batch size to reduction tree").  The twins exist to price
 * invariance and to prove the harness notices a batch-dependent kernel.
 *
 * Conventions for every function:
 *  - Pointers named as device data are device pointers (hipMalloc / torch
 *    CUDA tensors) aligned to 16 bytes; tensors are dense row-major with the
 *    shapes given.  bf16 data is raw IEEE bfloat16 bits (uint16).  The
 *    caller owns every buffer; the invariant path allocates nothing.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls
 *    only enqueue work: a BI_OK return means "launched"; device faults
 *    surface at the caller's next synchronisation.
 *  - Arguments are validated on the host before anything is launched.  A
 *    rejected call launches nothing and returns BI_ERR_INVALID (null
 *    pointer, bad size), BI_ERR_UNSUPPORTED (a dtype, head size, group
 *    ratio or chunk the kernels do not implement -- they fail closed rather
 *    than fall back, as the pages ask of kernels that cannot keep the
 *    property: "Batch invariance and reproducible inference", the
 *    fused-MoE opt-out and the Mamba refusal) or BI_ERR_WORKSPACE (a
 *    workspace that is too small).  BI_ERR_HIP reports a launch error.
 *    bi_last_error() returns a message for the calling thread's last
 *    failure.
 *  - Preconditions that live in device memory (kv_len >= 1, block-table
 *    entries naming valid pages, positions inside the RoPE tables) are the
 *    caller's to keep; they are not checked on the device.
 */
#ifndef BI_H
#define BI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int bi_status;
#define BI_OK 0
#define BI_ERR_INVALID 1
#define BI_ERR_UNSUPPORTED 2
#define BI_ERR_WORKSPACE 3
#define BI_ERR_HIP 4

/* element types */
#define BI_F32 0
#define BI_BF16 1

typedef void *bi_stream; /* hipStream_t */

/* Version of this ABI: changes when a signature or the layout an argument
 * must have changes (3: bf16 product weights in the packed layout below). */
int bi_abi_version(void);
/* Static text for a status code. */
const char *bi_status_string(bi_status s);
/* Message of the calling thread's last failed call ("" if none). */
const char *bi_last_error(void);

/* ---------------------------------------------------------------------- */
/* RMSNorm                                                                */
/* ---------------------------------------------------------------------- */
/*
 * y[i][:] = x[i][:] * (1 / sqrt(mean_j x[i][j]^2 + eps)) * gamma[:], one
 * workgroup per row, no cross-workgroup reduction ("Batch invariance and
 * reproducible inference": rms_norm is one of the dull one-block-per-row
 * kernels).  Fixed order of the fp32 sum of squares: vectors of 8
 * consecutive elements; 256 lanes, lane t visits vectors t, t+256, ... with
 * fma(x, x, acc); each 64-lane wave reduces by xor butterfly 32,16,8,4,2,1;
 * the four wave sums are added in order.  Then r = 1/sqrt(ss/d + eps) and
 * y = round((x * r) * gamma), each step correctly rounded.
 *   x, y   : device [M][d] of `dtype` (y may alias x);  gamma: device [d].
 *   M >= 0 (0 is a no-op), d >= 1.  dtype BI_F32 or BI_BF16.
 */
bi_status bi_rmsnorm(const void *x, const void *gamma, void *y, int M, int d, float eps,
                     int dtype, bi_stream stream);

/* Residual add fused with the RMSNorm that follows it (the transformer's
 * "h = h + sublayer(x); x = norm(h)"): h[i][j] = round(h[i][j] + o[i][j]) is
 * written back to h, then y = bi_rmsnorm(h) with the same tree.  The result
 * equals bi_add followed by bi_rmsnorm bit for bit; one launch instead of
 * two, one pass over h.
 *   h : device [M][d] of `dtype`, read and written;  o : device [M][d];
 *   gamma : device [d];  y : device [M][d], must not alias h or o.
 *   Same shapes, dtypes and errors as bi_rmsnorm. */
bi_status bi_add_rmsnorm(void *h, const void *o, const void *gamma, void *y, int M, int d,
                         float eps, int dtype, bi_stream stream);

/* Twin: when M is too small to fill the device, each row is split over
 * several workgroups whose partial sums meet through fp32 atomics (order
 * set by scheduling); otherwise one workgroup per row with a different
 * tree.  Needs bi_rmsnorm_free_workspace_bytes(M, d) bytes of device
 * workspace. */
size_t bi_rmsnorm_free_workspace_bytes(int M, int d);
bi_status bi_rmsnorm_free(const void *x, const void *gamma, void *y, int M, int d, float eps,
                          int dtype, void *workspace, size_t workspace_bytes, bi_stream stream);

/* ---------------------------------------------------------------------- */
/* GEMM  C = A W^T                                                        */
/* ---------------------------------------------------------------------- */
/*
 * Packed weights.  The bf16 products read W [N][K] (the weight's [out][in]
 * matrix) in a packed layout: [ceil(N/256)][ceil(K/64)][16][16][64], element
 * (n, k) at (((n / 256) * ceil(K/64) + k / 64) * 16 + (n / 16) % 16) * 1024 +
 * (n % 16) * 64 + k % 64, the padding zero.  A 16-row x 64-k block is 2 KiB
 * in a row, the 16 blocks of a 256-row panel at one 64-wide K step 32 KiB,
 * and a panel's K steps follow each other: a decode strip reads 2 KiB runs
 * and a 256 x 256 prefill tile one contiguous panel.  No passage fixes a
 * layout: this is the library's.  bi_pack_weight writes it from a row-major bf16 [N][K]
 * (16-byte aligned) into bi_packed_weight_bytes(N, K) bytes (16-byte
 * aligned); K % 8 != 0 returns BI_ERR_UNSUPPORTED, other errors
 * BI_ERR_INVALID, and nothing is launched on an error.
 */
size_t bi_packed_weight_bytes(int N, int K);
bi_status bi_pack_weight(const void *W, void *Wp, int N, int K, bi_stream stream);

/*
 * C[i][j] = sum_k A[i][k] W[j][k].  A: device [M][K], C: device [M][N]; W:
 * with in_dtype BI_BF16 the packed weight of the [N][K] matrix (above), with
 * BI_F32 the row-major [N][K] matrix.
 * in_dtype BI_BF16: out_dtype BI_BF16 or BI_F32; every output element is one
 * chain of v_mfma_f32_16x16x32_bf16 over K-tiles of 32 in ascending order,
 * fp32 accumulation, no split of K across workgroups, and the same chain
 * whatever M is (small M and large M use different tilings of the same
 * per-element arithmetic) -- "Batch invariance and reproducible inference",
 * "2 . Cross-block accumulation" (no split-K; one fixed K order per output
 * tile) and "3 . Kernel selection changing with shape" (nothing that
 * changes the arithmetic reads M).  K % 8 == 0.
 * in_dtype BI_F32 (out BI_F32): one serial fp32 fma chain per element over
 * k ascending.
 * M >= 0 (0 is a no-op), N >= 1, K >= 1.
 */
bi_status bi_gemm(const void *A, const void *W, void *C, int M, int N, int K, int in_dtype,
                  int out_dtype, bi_stream stream);

/* The fused gate/up weight of an MLP comes in 8-row blocks: rows 16p ..
 * 16p + 7 of W [2I][K] are the gate rows 8p .. 8p + 7 and rows 16p + 8 ..
 * 16p + 15 the matching up rows, so C = A W^T holds gate column 8p + i at
 * column 16p + i and up column 8p + i at column 16p + 8 + i.  (A 16-row strip
 * of W is then one contiguous run that carries a gate/up pair of 8 columns
 * each.  No passage fixes a layout: this is the library's.)
 *
 * SwiGLU projection of a decode batch in one pass: act[i][j] =
 * round(g / (1 + exp(-g)) * u) with g = C[i][16(j/8) + j%8], u = C[i][16(j/8)
 * + 8 + j%8] of C = A W^T as bi_gemm computes it (bf16 out), so the result
 * is bit-identical to bi_gemm into [M][2I] followed by bi_silu_mul, without
 * the [M][2I] intermediate.  A: device bf16 [M][K]; W: the packed weight
 * (above) of the bf16 [2I][K] matrix in 8-row gate/up blocks; act: device bf16 [M][I].  The K reduction is the same
 * chain as bi_gemm's ("2 . Cross-block accumulation").  0 <= M <= 64 (larger
 * M: bi_gemm then bi_silu_mul), I % 8 == 0, K % 8 == 0, pointers 16-byte
 * aligned; anything else returns BI_ERR_INVALID and launches nothing. */
bi_status bi_gemm_swiglu(const void *A, const void *W, void *act, int M, int I, int K,
                         bi_stream stream);

/* QKV projection of a decode batch with RoPE and the KV append in its
 * epilogue: the result is bit-identical to bi_gemm of A and W into a bf16
 * [M][(h + 2 h_kv) d_h] buffer followed by bi_rope_kv_append of it (same
 * arguments, dtype BI_BF16), without the intermediate.  Each output element is
 * bi_gemm's K chain ("2 . Cross-block accumulation"); only which W rows share a
 * 16-column MFMA tile changes (dims i and i + d_h/2 of a head), which does not
 * touch any element's arithmetic.  A: device bf16 [M][K]; W: the packed
 * weight (above) of the bf16 [(h + 2 h_kv) d_h][K] matrix, rows [q | k | v]
 * as for bi_rope_kv_append; the other
 * arguments as there (q_out device bf16 [M][h][d_h], pools bf16).  0 <= M <=
 * 64 (larger M: bi_gemm then bi_rope_kv_append), K % 8 == 0, d_h % 16 == 0, A
 * and W 16-byte aligned; anything else returns BI_ERR_INVALID and launches
 * nothing.  Slots of different rows must differ (as for bi_rope_kv_append). */
bi_status bi_gemm_qkv_rope(const void *A, const void *W, int M, int K, int h, int h_kv, int d_h,
                           const int32_t *pos, const float *cos_t, const float *sin_t,
                           const int32_t *slot_mapping, int page_size, void *q_out,
                           void *k_pool, void *v_pool, bi_stream stream);

/* The three products above with the residual add and the RMSNorm that
 * precede them in a transformer layer done in their prologue, for batches
 * of a few rows: first h_out = round(h + o) and x = RMSNorm(h_out) * gamma,
 * exactly as bi_add_rmsnorm computes them (with o == NULL: x =
 * RMSNorm(h) * gamma as bi_rmsnorm, and h_out must be NULL), then the
 * product of x with W as bi_gemm / bi_gemm_swiglu / bi_gemm_qkv_rope compute
 * it.  Every output is bit-identical to the two launches' ("Batch invariance
 * and reproducible inference": rms_norm reduces each row inside one block;
 * "2 . Cross-block accumulation": one K chain per output); this is one
 * launch instead of two, which matters when a launch's fixed cost exceeds
 * the work.  No passage defines the fusion itself.
 *   h : device bf16 [M][K] (the residual stream), read only;
 *   o : device bf16 [M][K] or NULL;  gamma : device bf16 [K];
 *   h_out : device bf16 [M][K], written, must not alias h or o (NULL iff o is);
 *   x_out : device bf16 [M][K] or NULL: the normalised rows, if wanted;
 *   the rest as for the plain call (packed bf16 W, bf16 outputs; C of bi_norm_gemm
 *   bf16 or fp32 by out_dtype).
 * 0 <= M <= 4 and K <= 4096 (BI_ERR_UNSUPPORTED beyond: use the two calls),
 * K % 8 == 0, pointers 16-byte aligned; other violations return
 * BI_ERR_INVALID.  Nothing is launched on an error. */
bi_status bi_norm_gemm(const void *h, const void *o, const void *gamma, float eps, void *h_out,
                       void *x_out, const void *W, void *C, int M, int N, int K, int out_dtype,
                       bi_stream stream);
bi_status bi_norm_gemm_swiglu(const void *h, const void *o, const void *gamma, float eps,
                              void *h_out, void *x_out, const void *W, void *act, int M, int I,
                              int K, bi_stream stream);
bi_status bi_norm_gemm_qkv_rope(const void *h, const void *o, const void *gamma, float eps,
                                void *h_out, void *x_out, const void *W, int M, int K, int h_q,
                                int h_kv, int d_h, const int32_t *pos, const float *cos_t,
                                const float *sin_t, const int32_t *slot_mapping, int page_size,
                                void *q_out, void *k_pool, void *v_pool, bi_stream stream);

/* Twin: picks its tiling from M and, when M x N offers too few tiles to fill
 * the device, splits K over workgroups that add fp32 partials with atomics
 * (order undefined) -- the split-K the pages describe.  W as for bi_gemm
 * (packed for bf16).  Needs
 * bi_gemm_free_workspace_bytes(M, N, K) bytes of device workspace. */
size_t bi_gemm_free_workspace_bytes(int M, int N, int K);
bi_status bi_gemm_free(const void *A, const void *W, void *C, int M, int N, int K, int in_dtype,
                       int out_dtype, void *workspace, size_t workspace_bytes, bi_stream stream);

/* ---------------------------------------------------------------------- */
/* split-KV attention over a paged KV cache                               */
/* ---------------------------------------------------------------------- */
/*
 * KV cache layout: each pool is num_pages pages of h_kv blocks of page_size
 * tokens x d_h elements of `dtype` (page p, kv head g: the block at element
 * offset (p * h_kv + g) * page_size * d_h); token j of a request lives in
 * page block_table[r][j / page_size] at slot j % page_size.  Within a block,
 * V is token-major rows ([slot][d_h]), and K is stored by 16-byte units:
 * unit u (elements 16/esize * u ..) of slot t at byte (u * page_size + t) *
 * 16, so that one matrix-core operand of K (16 tokens x 32 dims) is a
 * contiguous KiB.  bi_rope_kv_append and bi_gemm_qkv_rope write this layout;
 * a cache held as token-major rows converts by that permutation of 16-byte
 * units alone.  block_table: device int32 [B][max_pages].
 * Query head i reads kv head i / (h / h_kv).
 *
 * Chunking ("Lockstep", "The fix": attention split points come from the
 * request, not the batch; "Batch invariance and reproducible inference",
 * "1 . Split-K and segmented attention reductions": split count =
 * ceil(seq_len / split tile) alone or in any batch): request r with
 * kv_len[r] tokens has ceil(kv_len[r] / kv_chunk) chunks, chunk c covering
 * absolute positions [c*kv_chunk, min((c+1)*kv_chunk, kv_len[r])).
 * chunk_off[r] (int32 [B+1], prefix sum of those counts) numbers the
 * partial rows; bi_chunk_offsets computes it on the host.
 *
 * Per (request, query head, chunk) partial, all fp32:
 *   S_u = fl(q . k_u) * scale (dot: one fma chain over d ascending);
 *   m = max_u S_u (+0 for -0);  p_u = exp(S_u - m);
 *   keys in blocks of 64: L_b = serial sum of p_u, A_b[d] = serial
 *   fma(p_u, v_u[d], .); l = ((L_0 + L_1) + L_2) + ..., acc likewise.
 * exp is one fixed binary32 routine (Cody-Waite reduction, degree-7 Taylor
 * polynomial), not the hardware approximation.
 */

/* Host helper: chunk_off[0] = 0, chunk_off[r+1] = chunk_off[r] +
 * ceil(kv_len[r] / kv_chunk).  Host arrays.  Returns the total. */
int bi_chunk_offsets(const int32_t *kv_len_host, int B, int kv_chunk, int32_t *chunk_off_host);

/* Bytes of the partial buffers for `total_chunks` chunk rows:
 * part_ml = total_chunks * h * 2 floats (m, l), part_acc = total_chunks * h
 * * d_h floats. */
size_t bi_attn_partials_bytes(int total_chunks, int h, int d_h);

/*
 * Decode: one query row per request.  q: device [B][h][d_h] of `dtype`;
 * kv_len: device int32 [B] (the current token included, >= 1); chunk_off:
 * device int32 [B+1]; total_chunks == chunk_off[B] (host copy of the last
 * entry).  Writes part_ml [total_chunks][h][2] and part_acc
 * [total_chunks][h][d_h] (device fp32).
 * Supported (anything else returns BI_ERR_UNSUPPORTED): d_h in {64, 128};
 * h % h_kv == 0 with h/h_kv in {2, 4}; kv_chunk in {64, 256}; page_size 16;
 * dtype BI_F32 or BI_BF16.  Every row of q, k and v is
 * 16-byte aligned.
 */
bi_status bi_decode_attn(const void *q, const void *k_pool, const void *v_pool,
                         const int32_t *block_table, const int32_t *kv_len,
                         const int32_t *chunk_off, int B, int total_chunks, int h, int h_kv,
                         int d_h, int page_size, int max_pages, int kv_chunk, float scale,
                         int dtype, float *part_ml, float *part_acc, bi_stream stream);

/*
 * Serial merge of each (request, head) over its chunks in order c = 0..n-1
 * ("Batch invariance and reproducible inference", "From batch size to
 * reduction tree": a merge kernel adds the fp32 partials):
 *   (M, L, Acc) = chunk 0; for c >= 1: M' = max(M, m_c), a = exp(M - M'),
 *   b = exp(m_c - M'), L = fma(l_c, b, L * a), Acc = fma(acc_c, b, Acc * a);
 *   out = round(Acc / L).
 * out: device [B][h][d_h] of out_dtype.
 */
bi_status bi_merge_partials(const float *part_ml, const float *part_acc,
                            const int32_t *chunk_off, int B, int h, int d_h, void *out,
                            int out_dtype, bi_stream stream);

/*
 * The softmax weight of the bf16 (matrix-core) attention paths, on its own:
 * p[i] = exp(x[i]) evaluated as decode and prefill attention evaluate
 * exp(s - m) -- the library's fixed exp (Cody & Waite reduction, degree-7
 * Taylor polynomial, scaling by 2^n) -- and p_bf16[i] its bf16 bits (round
 * to nearest even).  No passage defines this call: it exposes that one
 * evaluation so that it can be checked against the oracle's exp over any
 * set of arguments.  x: device fp32 [n], each x <= 0 or -inf (the arguments
 * the kernels use; larger values give unspecified results, NaN gives NaN);
 * p: device fp32 [n]; p_bf16: device uint16 [n], or NULL.  n >= 0 (0 is a
 * no-op); errors return BI_ERR_INVALID and launch nothing.
 */
bi_status bi_softmax_weights(const float *x, float *p, uint16_t *p_bf16, int n,
                             bi_stream stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): decode
 * attention straight to its output, bi_decode_attn followed by
 * bi_merge_partials with the same arguments, bit for bit, but with the fp32
 * partials held in a static device buffer of BI_NOALLOC_SCRATCH_BYTES inside
 * the library instead of caller workspace.  Nothing is allocated: the buffer
 * exists on each GPU from the library's load to the end of the process (its
 * address is looked up once per device, on the first call there).  The
 * partials (total_chunks * h * (d_h + 2) * 4 bytes, plus alignment) must fit,
 * else BI_ERR_WORKSPACE and nothing is launched; at h = 32, d_h = 128 that is
 * up to 2016 chunk rows (e.g. 64 requests of 7936 tokens at kv_chunk 256).
 * Every call on one GPU uses the same buffer, and the merge reads only rows
 * the same call has written, so nothing needs clearing between calls; calls
 * that overlap on one GPU (concurrent streams) race on it and must be
 * serialised by the caller.  out: device [B][h][d_h] of out_dtype; the other
 * arguments, limits and errors as for bi_decode_attn. */
#define BI_NOALLOC_SCRATCH_BYTES (32 * 1024 * 1024)
bi_status bi_decode_attn_noalloc(const void *q, const void *k_pool, const void *v_pool,
                                 const int32_t *block_table, const int32_t *kv_len,
                                 const int32_t *chunk_off, int B, int total_chunks, int h,
                                 int h_kv, int d_h, int page_size, int max_pages, int kv_chunk,
                                 float scale, int dtype, void *out, int out_dtype,
                                 bi_stream stream);

/*
 * Causal prefill over packed query rows.  q: device [T][h][d_h]; request r
 * owns rows q_start[r] .. q_start[r+1]-1 (device int32 [R+1], T ==
 * q_start[R]); row t sits at absolute position q_pos0[r] + t - q_start[r]
 * (device int32 [R]) and attends positions 0 .. pos, which must already be
 * in the cache.  Every row is computed exactly as the decode path computes
 * a request of kv_len = pos + 1 (same chunks at absolute multiples of
 * kv_chunk, same partial arithmetic, same serial merge), so a prompt gives
 * the same bits however it is cut into prefill chunks and whether a
 * position is produced by prefill or by decode ("Batch invariance and
 * reproducible inference": chunked prefill must not move split
 * boundaries).  out: device [T][h][d_h] of `dtype`.  Same support limits as
 * bi_decode_attn.
 */
bi_status bi_prefill_attn(const void *q, const int32_t *q_start, const int32_t *q_pos0, int R,
                          int T, const void *k_pool, const void *v_pool,
                          const int32_t *block_table, int h, int h_kv, int d_h, int page_size,
                          int max_pages, int kv_chunk, float scale, int dtype, void *out,
                          bi_stream stream);

/*
 * Twins.  bi_decode_attn_free picks one split length per request from the
 * batch, the longest sequence and the device's 256 compute units (the
 * occupancy policy quoted on "Batch invariance and reproducible
 * inference", "From batch size to reduction tree": the batch size divides
 * the core budget, which sets the split count and chunk length), runs the
 * partials and merges them, writing out [B][h][d_h].  max_kv_len is the
 * host's bound on kv_len.  Workspace: bi_decode_attn_free_workspace_bytes.
 * bi_merge_partials_free takes the same arguments as bi_merge_partials but
 * combines each request's chunks from the last to the first, another fixed
 * order whose results differ in ulps.  bi_prefill_attn_free splits each row's keys at multiples of a
 * length chosen from the row count, counted from the start of the prefill
 * chunk rather than from position 0.
 */
size_t bi_decode_attn_free_workspace_bytes(int B, int h, int d_h, int max_kv_len);
bi_status bi_decode_attn_free(const void *q, const void *k_pool, const void *v_pool,
                              const int32_t *block_table, const int32_t *kv_len, int B,
                              int max_kv_len, int h, int h_kv, int d_h, int page_size,
                              int max_pages, float scale, int dtype, void *workspace,
                              size_t workspace_bytes, void *out, bi_stream stream);
bi_status bi_merge_partials_free(const float *part_ml, const float *part_acc,
                                 const int32_t *chunk_off, int B, int h, int d_h, void *out,
                                 int out_dtype, bi_stream stream);
bi_status bi_prefill_attn_free(const void *q, const int32_t *q_start, const int32_t *q_pos0,
                               int R, int T, const void *k_pool, const void *v_pool,
                               const int32_t *block_table, int h, int h_kv, int d_h,
                               int page_size, int max_pages, float scale, int dtype, void *out,
                               bi_stream stream);

/* ---------------------------------------------------------------------- */
/* elementwise glue of a Llama-shaped layer (no reductions)               */
/* ---------------------------------------------------------------------- */
/* No passage of the pages defines these steps.  They are the decoder layer's
 * own arithmetic around the reductions (embedding gather, rotate-half RoPE
 * with the KV append, residual add, the SiLU-gated product, argmax), each a
 * function of its own row's inputs with no sum across rows, so none of them
 * can depend on the batch; the readings they follow (RoPE with theta =
 * 500000, SiLU through the library's exp, lowest index on argmax ties) are
 * stated with each function. */

/* out[i][:] = table[ids[i]][:]; table device [V][d], ids device int32 [M]. */
bi_status bi_embed(const void *table, const int32_t *ids, void *out, int M, int d, int dtype,
                   bi_stream stream);

/*
 * Split a fused QKV row [q (h*d_h) | k (h_kv*d_h) | v (h_kv*d_h)], apply
 * rotate-half RoPE to q and k at position pos[i] (x'[i] = fma(a, c, -(b*s)),
 * x'[i+d_h/2] = fma(b, c, a*s) with a = x[i], b = x[i+d_h/2]), write q to
 * q_out [M][h][d_h] and k, v into the pools at flat slot slot_mapping[i]
 * (= page * page_size + offset).  cos_t / sin_t: device fp32
 * [max_pos][d_h/2]; both NULL = no rotation.  Results rounded to `dtype`.
 */
bi_status bi_rope_kv_append(const void *qkv, int M, int h, int h_kv, int d_h,
                            const int32_t *pos, const float *cos_t, const float *sin_t,
                            const int32_t *slot_mapping, int page_size, void *q_out,
                            void *k_pool, void *v_pool, int dtype, bi_stream stream);

/* y = round(a + b) elementwise over n elements (y may alias a or b). */
bi_status bi_add(const void *a, const void *b, void *y, long n, int dtype, bi_stream stream);

/* Log-softmax of fp32 rows (logprobs): y[i][j] = (x[i][j] - m_i) -
 * log(sum_j exp(x[i][j] - m_i)), m_i the row maximum.  One
 * workgroup per row whatever M is, each row reduced in one fixed order (a
 * thread's strided elements serially, an xor butterfly per wave, the waves in
 * order), with the library's own exp and log -- "Batch invariance and
 * reproducible inference": the dispatcher's replacement log_softmax (one
 * block per row, no cross-block reduction, after "4 . Unsorted top-k in MoE
 * routing") and "Mathematically equivalent is not bitwise equivalent"
 * (logprobs come from this one kernel for prefill and decode rows alike, so
 * equal logit rows give equal logprob rows).  x, y: device fp32 [M][V]; y may
 * be x (in place) but must not partly overlap it.  A row with no entry above
 * -inf gives -inf throughout; NaN entries never win the maximum.  M >= 0 (0 is
 * a no-op), V >= 1; errors return BI_ERR_INVALID and launch nothing. */
bi_status bi_log_softmax(const float *x, float *y, int M, int V, bi_stream stream);

/* Seeded per-request sampling (Gumbel-max): out[i] = argmax_j of
 * x[i][j] * (1 / T_i) + g_ij in binary64, g_ij = -log(-log(u_ij)),
 * u_ij = (h_ij + 1/2) 2^-32, h_ij = MurmurHash3_x86_32 of the 8-byte key
 * (pos[i], j) (two little-endian uint32) under seed[i]; lowest index on ties;
 * T_i <= 0 gives the argmax of the row.  A request's draw depends only on its
 * own logits, seed and position, never on the batch -- "Batch invariance and
 * reproducible inference", "The weaker guarantees, which are usually enough"
 * (per-request sampling determinism: noise from a 32-bit murmur hash of seed,
 * position and column in float64).  log is the library's fixed binary64 log,
 * so the oracle reproduces every draw.  x: device fp32 [M][V]; seed: device
 * uint32 [M]; pos: device int32 [M] (the row's absolute position);
 * temperature: device fp32 [M]; out: device int32 [M].  M >= 0 (0 is a no-op),
 * V >= 1; errors return BI_ERR_INVALID and launch nothing. */
bi_status bi_sample(const float *x, const uint32_t *seed, const int32_t *pos,
                    const float *temperature, int32_t *out, int M, int V, bi_stream stream);

/* SwiGLU of a gate/up product in 8-column blocks (the layout above): gu
 * [M][2F], g = gu[i][16(j/8) + j%8], u = gu[i][16(j/8) + 8 + j%8];
 * y[i][j] = round(g / (1 + exp(-g)) * u), y [M][F].  F % 8 == 0. */
bi_status bi_silu_mul(const void *gu, void *y, int M, int F, int dtype, bi_stream stream);

/* idx[i] = argmax_j x[i][j] over fp32 x [M][V]; lowest index wins ties. */
bi_status bi_argmax(const float *x, int32_t *idx, int M, int V, bi_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* BI_H */
