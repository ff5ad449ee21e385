/*
 * vq_glue.h — element-wise kernels that join the three verify operations into
 * one verify step of a dense pre-norm stack (RMSNorm, SwiGLU, residual add,
 * KV append). The pages define no layer; this composition follows the hybrid
 * dense model they describe only as far as the data flow: the M verify rows go
 * through every layer's projections, and the full-attention layers append the
 * rows' keys and values to an append-only cache before attending (page "The
 * fastest way to run local LLMs on a Mac", sections "Why token 1,000 is faster
 * than token 100,000" and "Why native MTP doubles decode").
 *
 * Same conventions as vq.h: caller-owned device pointers, asynchronous on
 * `stream`, host-side validation (VQ_ERR_INVALID_ARG), no allocation. All
 * tensors are bf16 with float32 arithmetic and round-to-nearest-even stores.
 */
#ifndef VQ_GLUE_H_
#define VQ_GLUE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* y[m, :] = x[m, :] / sqrt(mean(x[m, :]^2) + eps); rows of N, strides ldx, ldy (elements).
 * 1 <= M, 1 <= N <= 65536. */
int vq_rmsnorm_bf16(const void* x, int64_t ldx, void* y, int64_t ldy, int M, int N, float eps,
                    void* stream);

/* Per-row sums of squares of a bf16 matrix x [M, N] (row stride ldx) per block
 * of 128 columns: out[m * P + c] = sum of x[m, n]^2 over the columns of block
 * c, P = ceil(N / 128); the x_sumsq input of vq_qmm_packed (vq.h). */
int vq_row_sumsq_bf16(const void* x, int64_t ldx, int M, int N, float* out, void* stream);

/* y[i] = a[i] + b[i] for i < n (y may alias a or b). */
int vq_add_bf16(const void* a, const void* b, void* y, int64_t n, void* stream);

/* y[m, i] = silu(gu[m, i]) * gu[m, I + i] for i < I; gu rows of 2I with stride ldgu,
 * y rows with stride ldy (elements). */
int vq_silu_mul_bf16(const void* gu, int64_t ldgu, void* y, int64_t ldy, int M, int I, void* stream);

/* Append M rows of keys and values taken from a fused projection output:
 *   k_cache[h, pos + m, :] = src[m, k_off + h*D : k_off + (h+1)*D]
 *   v_cache[h, pos + m, :] = src[m, v_off + h*D : v_off + (h+1)*D]
 * src rows have stride ld_src (elements); caches are [Hkv, T_cap, D] with head
 * stride kv_head_stride (elements). The caller guarantees pos + M <= T_cap.
 * D a multiple of 8; k_off, v_off, ld_src multiples of 8. */
int vq_kv_append_bf16(const void* src, int64_t ld_src, int k_off, int v_off, void* k_cache,
                      void* v_cache, int64_t kv_head_stride, int M, int Hkv, int D, int pos,
                      void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VQ_GLUE_H_ */
