/*
 * vq.h — C ABI of the batched K-token verify pass of MTP speculative decoding
 * on AMD Instinct MI355X (gfx950).
 *
 * Three operations, as the pages state the problem:
 *   vq_skinny_qmm     M = 1..16 bf16 rows times a 4-bit or 8-bit affine
 *                     group-quantized weight matrix, the weights read from HBM
 *                     once for all rows (page "Speculative decoding and MTP on
 *                     Apple silicon", Facts: the stock quantized matmul re-reads
 *                     the weights for every row of the M = 2..8 verify window; a
 *                     small-M kernel shares them across up to 16 rows; page "The
 *                     fastest way to run local LLMs on a Mac", section "Why
 *                     native MTP doubles decode": the verify pass reads the
 *                     weights once).
 *   vq_multirow_attn  M query rows, causal among the drafted rows, grouped-query
 *                     attention over a long bf16 KV cache, each KV tile read once
 *                     for all rows (same page, Facts: decode attention re-reads
 *                     the KV cache per query row; a multi-row kernel reads each
 *                     KV tile once).
 *   vq_spec_accept    exact Leviathan–Chen acceptance: accept with probability
 *                     min(1, p/q), resample from (p - q)+ at the first rejection,
 *                     identical top-k / top-p truncation of p and q (page "The
 *                     fastest way to run local LLMs on a Mac", section "Why exact
 *                     acceptance matters"; page "Speculative decoding and MTP on
 *                     Apple silicon", Facts: rejection sampling and identical
 *                     truncation of draft and verify distributions).
 *
 * Conventions shared by every entry point
 *   - Every pointer named as data is a device pointer owned by the caller. The
 *     library never allocates device memory in a call: scratch space comes from
 *     the caller's `workspace`, sized by the matching *_workspace() query.
 *   - A workspace holds a region of completion counters that must be zero
 *     before its first use (allocate it zero-filled). Every call leaves those
 *     counters zero again when it completes, so the same workspace can be
 *     reused by later calls on the same stream. Calls that run concurrently
 *     must not share a workspace.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and does not synchronise the host. Outputs are valid once the
 *     stream has reached the call. Outputs must not alias inputs.
 *   - All shapes, strides, pointers and parameters are validated on the host
 *     before anything is launched; a failed check returns VQ_ERR_INVALID_ARG
 *     and launches nothing. A launch failure returns VQ_ERR_HIP. The detail of
 *     the last error on the calling thread is in vq_last_error().
 *   - No call prints, aborts or throws across the ABI.
 *   - The library runs on gfx950 only.
 */
#ifndef VQ_H_
#define VQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define VQ_OK 0
#define VQ_ERR_INVALID_ARG 1
#define VQ_ERR_HIP 2
#define VQ_ERR_UNSUPPORTED_DEVICE 3

/* Output element types for vq_skinny_qmm. */
#define VQ_BF16 0
#define VQ_F32 1

/* Input kinds for vq_spec_accept. */
#define VQ_PROBS 0
#define VQ_LOGITS 1

/* Limits. */
#define VQ_MAX_ROWS 16      /* M of vq_skinny_qmm and vq_multirow_attn        */
#define VQ_MAX_DRAFTS 15    /* K of vq_spec_accept (M = K + 1 <= 16)          */
#define VQ_MAX_VOCAB (1 << 20)

/* Short text for a status code (static storage). */
const char* vq_status_string(int status);

/* Detail of the last failed call on the calling thread ("" if none). */
const char* vq_last_error(void);

/* Library version, e.g. "0.1.0". */
const char* vq_version(void);

/* ------------------------------------------------------------------------
 * Skinny quantized matmul
 *
 *   y[m, n] = sum_k x[m, k] * (s[n, k / gs] * q[n, k] + b[n, k / gs])
 *
 * x        bf16, M rows of K elements, row stride ldx (elements, >= K).
 * wq       packed unsigned codes of W[N, K], row-major by output n, each row
 *          K * bits / 8 bytes:
 *            bits = 4: element k of row n is the nibble at bits 4*(k%8) ..
 *                      4*(k%8)+3 of little-endian 32-bit word k/8 of that row;
 *            bits = 8: element k of row n is byte k of that row.
 * scales,  bf16 [N, K / gs] row-major: one affine scale s and bias b per group of
 * biases   gs consecutive elements along K.
 * bits     4 or 8.  gs: 64 (the only group size built).
 * M        1 .. 16 rows.  1 <= N <= 2^20.  K: a positive multiple of 64.
 * y        M rows of N outputs, row stride ldy (elements, >= N); y_dtype is
 *          VQ_BF16 (round to nearest even) or VQ_F32.
 * Alignment: x, wq and each row start of x must be 16-byte aligned (ldx a
 * multiple of 8); scales and biases 4-byte aligned; y 4-byte aligned.
 * Accumulation is float32 with a fixed reduction order, so repeated calls give
 * bit-identical results.
 * ---------------------------------------------------------------------- */
size_t vq_skinny_qmm_workspace(int bits, int group_size, int M, int N, int K);

int vq_skinny_qmm(const void* x, int64_t ldx,
                  const void* wq, const void* scales, const void* biases,
                  int bits, int group_size, int M, int N, int K,
                  void* y, int64_t ldy, int y_dtype,
                  void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * vq_skinny_qmm for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * The same product, arguments and result as vq_skinny_qmm (bit-identical), with
 * no workspace argument: the split-K partials and completion counters live in a
 * device array of VQ_NOALLOC_SCRATCH_BYTES (16 MiB) that the library holds on
 * every GPU it runs on, from its load until the process ends. The call neither
 * allocates nor frees memory; it clears the counters itself (a small kernel on
 * `stream`, so it can be captured).
 * Limits: a shape whose vq_skinny_qmm_workspace() exceeds 16 MiB is rejected
 * with VQ_ERR_INVALID_ARG (every projection of a 27B-shaped layer fits up to
 * M = 16; a 248320-wide output fits up to M = 3).
 * Concurrency: all calls on one GPU share that GPU's array, so calls that may
 * overlap on one GPU (different streams, or host threads) race and must be
 * serialised by the caller; calls in order on one stream are safe.
 * ---------------------------------------------------------------------- */
#define VQ_NOALLOC_SCRATCH_BYTES (16u << 20)

int vq_skinny_qmm_noalloc(const void* x, int64_t ldx,
                          const void* wq, const void* scales, const void* biases,
                          int bits, int group_size, int M, int N, int K,
                          void* y, int64_t ldy, int y_dtype, void* stream);

/* ------------------------------------------------------------------------
 * Skinny quantized matmul on a prepacked weight, with fused glue
 *
 * The same product as vq_skinny_qmm on a layout made once per weight by
 * vq_qmm_pack: for every tile of 32 output rows and every block of 256 (4-bit)
 * or 128 (8-bit) inputs, the tile's 32 x 128 bytes of codes followed by its
 * scales and biases, so that the kernel reads each block as one contiguous
 * run. The code bytes are stored as 256 units of 16 bytes, unit 64j + l holding
 * bytes 16(2j + l/32) .. +15 of row l%32: the 16 bytes that lane l of a 64-wide
 * wave loads with its j-th load are its matrix-core operand as they arrive.
 * Rows past N and groups past K are zero-filled. The pack is an opaque byte
 * buffer of vq_qmm_pack_bytes() bytes, 16-byte aligned.
 *
 * Fused around the product, for the verify pass of a pre-norm stack (the
 * verify rows go through every projection of every layer; page "The fastest
 * way to run local LLMs on a Mac", section "Why native MTP doubles decode"):
 *   prologue  if x_sumsq != NULL, x is RMS-normalised while it is staged:
 *             x'[m, k] = bf16(x[m, k] / sqrt(S[m] / K + eps)), where S[m] is
 *             the sum of x_sumsq[m * x_sumsq_parts + p] over the parts p
 *             (1 <= parts <= 256), as written by a residual epilogue or by
 *             vq_row_sumsq_bf16 (vq_glue.h). The weight of the norm is one.
 *   epilogue  VQ_EPI_STORE     y = acc, bf16 or float32 (y_dtype);
 *             VQ_EPI_RESIDUAL  y = bf16(residual + bf16(acc)), bf16; residual
 *                              may be y itself (in place, then ldr == ldy);
 *                              if y_sumsq != NULL, y_sumsq[m * P + c] = sum of
 *                              y[m, n]^2 over the 128 columns of block c,
 *                              P = vq_sumsq_parts(N) = ceil(N / 128);
 *             VQ_EPI_SWIGLU    the N rows of the pack are, per block of 128,
 *                              64 gate rows and then the 64 up rows of the
 *                              same outputs; y has N / 2 columns (N a
 *                              multiple of 128): y[m, j] = bf16(silu(g) * u)
 *                              with g, u the bf16-rounded products.
 * Shapes, strides and alignment as vq_skinny_qmm; bf16 outputs 2-byte aligned,
 * float32 outputs and the sums of squares 4-byte aligned. Deterministic.
 * ---------------------------------------------------------------------- */
#define VQ_EPI_STORE 0
#define VQ_EPI_RESIDUAL 1
#define VQ_EPI_SWIGLU 2

/* Bytes of the pack of a [N, K] weight (0 for an unsupported shape). */
size_t vq_qmm_pack_bytes(int bits, int group_size, int N, int K);

/* Writes the pack of (wq, scales, biases) — the row-major layout of
 * vq_skinny_qmm — into `packed` (device, packed_bytes >= vq_qmm_pack_bytes). */
int vq_qmm_pack(const void* wq, const void* scales, const void* biases, int bits, int group_size, int N,
                int K, void* packed, size_t packed_bytes, void* stream);

/* Number of sum-of-squares parts of an N-column bf16 matrix: ceil(N / 128). */
int vq_sumsq_parts(int N);

size_t vq_qmm_packed_workspace(int bits, int group_size, int M, int N, int K);

int vq_qmm_packed(const void* x, int64_t ldx, const float* x_sumsq, int x_sumsq_parts, float eps,
                  const void* packed, int bits, int group_size, int M, int N, int K,
                  int epilogue, const void* residual, int64_t ldr,
                  void* y, int64_t ldy, int y_dtype, float* y_sumsq,
                  void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Multi-row decode attention
 *
 * For query row i in [0, M), query head h, KV head g = h / (Hq / Hkv):
 *   out[i, h] = sum_{j <= T - M + i} softmax_j(scale * <q[i, h], k[g, j]>) v[g, j]
 * i.e. the M query rows are the last M of the T valid positions (causal among
 * the drafted rows, bottom-right aligned).
 *
 * q        bf16 [M, Hq, D]: heads of one row contiguous, consecutive rows
 *          q_row_stride elements apart (>= Hq * D, a multiple of 8).
 * k_cache, bf16 [Hkv, T_cap, D]: row stride D elements, head stride
 * v_cache  kv_head_stride elements (>= T * D, a multiple of 8).
 * M        1 .. 16.  Hq % Hkv == 0, Hq / Hkv * M <= 128.  D: 64, 128 or 256.
 * T        number of valid keys, M <= T.
 * out      bf16 [M, Hq, D], rows out_row_stride elements apart (>= Hq * D,
 *          a multiple of 8).
 * Alignment: q, k_cache, v_cache and out 16-byte aligned.
 * Float32 scores, softmax and accumulation; P is rounded to bf16 for the PV
 * product; deterministic.
 * ---------------------------------------------------------------------- */
size_t vq_multirow_attn_workspace(int M, int Hq, int Hkv, int D, int T);

int vq_multirow_attn(const void* q, int64_t q_row_stride, const void* k_cache,
                     const void* v_cache, int64_t kv_head_stride, int M, int Hq, int Hkv,
                     int D, int T, float scale, void* out, int64_t out_row_stride,
                     void* workspace, size_t workspace_bytes, void* stream);

/* The same attention with the append of the M verify rows fused in: the rows
 * k_new[m, h*D .. (h+1)*D) and v_new[m, ...] (m < M, KV head h, rows
 * new_row_stride elements apart, >= Hkv * D and a multiple of 8, 16-byte
 * aligned) become cache positions T-M+m of KV head h — the append-only cache
 * of the full-attention layers (page "The fastest way to run local LLMs on a
 * Mac", section "Why token 1,000 is faster than token 100,000") — and the
 * attention over the T keys uses them. The caches are written (rows T-M ..
 * T-1 only); everything else is as vq_multirow_attn, with the same
 * workspace. k_new and v_new must not overlap the caches. */
int vq_multirow_attn_append(const void* q, int64_t q_row_stride, const void* k_new,
                            const void* v_new, int64_t new_row_stride, void* k_cache,
                            void* v_cache, int64_t kv_head_stride, int M, int Hq, int Hkv,
                            int D, int T, float scale, void* out, int64_t out_row_stride,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Tree verify (page "Speculative decoding and MTP on Apple silicon", Facts:
 * tree verify runs the full-attention layers with tree-attention masks). The
 * M rows are the nodes of a draft tree at cache positions T-M .. T-1 (node i at
 * T-M+i); row i sees every committed position j < T-M and the drafted
 * position T-M+t iff t == i or bit t of tree_mask[i] is set — its ancestors.
 * Bits at or above M are ignored. tree_mask: device uint32 [M], 4-byte
 * aligned, read by the call (it may change between graph replays). A chain
 * (tree_mask[i] = 2^(i+1) - 1) gives vq_multirow_attn's causal result.
 * k_new and v_new are both NULL (the caches already hold the M rows; they are
 * then only read) or both given (the append of vq_multirow_attn_append, with
 * its rules). Everything else is as vq_multirow_attn, with the same workspace. */
int vq_multirow_attn_tree(const void* q, int64_t q_row_stride, const void* k_new,
                          const void* v_new, int64_t new_row_stride, void* k_cache,
                          void* v_cache, int64_t kv_head_stride, int M, int Hq, int Hkv,
                          int D, int T, float scale, const uint32_t* tree_mask, void* out,
                          int64_t out_row_stride, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Several sequences in one call (page "Speculative decoding and MTP on Apple
 * silicon", Facts: the verify window of several streams shares one pass over
 * the weights; each stream keeps its own cache and length). The rows of all
 * sequences are stacked in q and out; sequence b (b < B) owns rows
 * row_start[b] .. row_start[b+1]-1 (M_b rows, 1 <= M_b <= max_rows) and the
 * first T_b = seq_len[b] positions (M_b <= T_b <= max_T) of its caches
 * k_cache + b * kv_batch_stride, v_cache + b * kv_batch_stride ([Hkv, T_cap,
 * D] each, head stride kv_head_stride, kv_batch_stride >= Hkv *
 * kv_head_stride). Within a sequence everything is as vq_multirow_attn: causal
 * among its M_b rows, or tree_mask[r] for row r when tree_mask is given
 * (vq_multirow_attn_tree, the bits relative to the sequence's first row); with
 * k_new and v_new (rows in the same stacking as q) the M_b rows are appended at
 * positions T_b - M_b .. T_b - 1 of the sequence's caches.
 * row_start (int32 [B+1]) and seq_len (int32 [B]) are device arrays read by the
 * call (they may change between graph replays). Values outside these rules are
 * clamped into [0, total_rows] and [M_b, max_T]; the outputs are then undefined
 * but nothing outside the buffers is accessed. B <= VQ_MAX_SEQS. */
#define VQ_MAX_SEQS 4096
size_t vq_multirow_attn_batched_workspace(int B, int max_rows, int Hq, int Hkv, int D, int max_T);

int vq_multirow_attn_batched(const void* q, int64_t q_row_stride, const int32_t* row_start,
                             const int32_t* seq_len, int B, int total_rows, int max_rows,
                             int max_T, const void* k_new, const void* v_new,
                             int64_t new_row_stride, void* k_cache, void* v_cache,
                             int64_t kv_batch_stride, int64_t kv_head_stride, int Hq, int Hkv,
                             int D, float scale, const uint32_t* tree_mask, void* out,
                             int64_t out_row_stride, void* workspace, size_t workspace_bytes,
                             void* stream);

/* 8-bit KV cache (page "Speculative decoding and MTP on Apple silicon",
 * Facts: KV-quantized caches are used together with speculative decoding; the
 * format is not given and this one follows the affine group-64 quantization of
 * the weights). Per KV head and position, the D values are cut into groups of
 * 64; group g holds 64 codes q in [0, 255] and one uint32 word whose low half
 * is the bf16 scale s and whose high half is the bf16 bias b: value = s*q + b.
 *   k_codes, v_codes  u8 [Hkv, T_cap, D], head stride kv_head_stride (a
 *                     multiple of D), 16-byte aligned;
 *   k_sb, v_sb        uint32 [Hkv, T_cap, D/64], 4-byte aligned.
 * vq_multirow_attn_int8 is vq_multirow_attn (tree_mask NULL) or
 * vq_multirow_attn_tree without the append (tree_mask given) over the
 * dequantized caches: scores, softmax and accumulation in float32 on the values
 * s*q + b rounded to bf16. Workspace: vq_multirow_attn_workspace(). */
int vq_multirow_attn_int8(const void* q, int64_t q_row_stride, const void* k_codes,
                          const void* k_sb, const void* v_codes, const void* v_sb,
                          int64_t kv_head_stride, int M, int Hq, int Hkv, int D, int T,
                          float scale, const uint32_t* tree_mask, void* out,
                          int64_t out_row_stride, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Quantizes M rows into an 8-bit cache at positions pos .. pos+M-1, the keys
 * from src[m, k_off + h*D ...] and the values from src[m, v_off + h*D ...] (bf16
 * rows, stride ld_src elements; the q|k|v projection output). Per group of 64:
 * mn = min, mx = max, scale = (mx - mn) / 255 and code = rint((x - mn) / scale)
 * (round half to even), both in correctly rounded float32, clamped to [0, 255];
 * a constant group gets codes 0 and scale 0; stored scale = bf16(scale) (round
 * to nearest even), bias = mn. kv_head_stride >= (pos + M) * D, a multiple of
 * D. No workspace. */
int vq_kv8_append(const void* src, int64_t ld_src, int k_off, int v_off, void* k_codes,
                  void* k_sb, void* v_codes, void* v_sb, int64_t kv_head_stride, int M,
                  int Hkv, int D, int pos, void* stream);

/* ------------------------------------------------------------------------
 * Exact speculative acceptance
 *
 * One verify per batch entry b in [0, B):
 *   target rows  p + b * p_batch_stride : K+1 rows of V float32
 *   draft rows   q + b * q_batch_stride : K rows of V float32
 * (a stride of 0 shares the same rows across the batch).
 * input_kind   VQ_PROBS: rows are probabilities in [0, 1];
 *              VQ_LOGITS: rows are logits and p = softmax(logits / temperature)
 *              is computed in float32 first (temperature > 0). In VQ_PROBS mode
 *              temperature is ignored.
 * draft        int32 [B, K] drafted token ids.
 * uniforms     float32 [B, K+1] in [0, 1): u_0..u_{K-1} for the K accept tests,
 *              u_K for the final draw.
 * top_k        0 = off, else keep the top_k most probable tokens (ties: lower id).
 * top_p        (0, 1]: then keep the shortest prefix (same order) whose mass
 *              reaches top_p of the top-k mass; 1 = off.
 * out_tokens   int32 [B, K+1]: accepted drafts, then the drawn token, then -1.
 * out_n_accepted int32 [B]: number of accepted drafts, or -1 for an invalid
 *              entry (a NaN or a probability outside [0, 1], a row that keeps no
 *              mass, a draft id outside [0, V), a uniform outside [0, 1)); an
 *              invalid entry has every token -1.
 * probs_out    nullable; in VQ_LOGITS mode receives the float32 probabilities
 *              of every row, [B', 2K+1, V] (target rows then draft rows), with
 *              B' = 1 if both strides are 0 and B otherwise.
 * Limits       1 <= B, 0 <= K <= 15, 2 <= V <= 2^20.
 *
 * Decision arithmetic (bit-exact, reproducible on any implementation): masses
 * m(x) = floor(p(x) * 2^40); order by (p descending, id ascending); top-k keeps
 * the first top_k; top-p keeps token t iff (kept mass before t) * 2^24 <
 * max(1, floor(top_p * 2^24)) * (top-k mass); Z = kept mass. Draft d_i is
 * accepted iff floor(u_i*2^24) * mQ(d_i) * ZP < mP(d_i) * ZQ * 2^24. At the
 * first rejection j the token is drawn from r = max(0, mP_j*ZQ_j - mQ_j*ZP_j)
 * (from mP_j if r is all zero), after K acceptances from mP_K, as the smallest
 * t with r[0] + .. + r[t] > floor(floor(u_K*2^24) * sum(r) / 2^24).
 * ---------------------------------------------------------------------- */
size_t vq_spec_accept_workspace(int B, int K, int V, int input_kind,
                                int64_t p_batch_stride, int64_t q_batch_stride);

int vq_spec_accept(const float* p, const float* q, int input_kind,
                   int64_t p_batch_stride, int64_t q_batch_stride,
                   const int32_t* draft, const float* uniforms,
                   int B, int K, int V, float temperature, int top_k, float top_p,
                   int32_t* out_tokens, int32_t* out_n_accepted, float* probs_out,
                   void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VQ_H_ */
