// Internal declarations shared by the host API layer and the kernel files.
// Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vq {

// The library is built for one chip: 256 compute units in 8 XCDs (gfx950).
constexpr int kNumCU = 256;
constexpr int kNumXCD = 8;

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---------------------------------------------------------------- skinny QMM
struct QmmPlan {
  int mt;          // padded row count of the kernel variant (4, 8 or 16)
  int cols_per_wg; // output columns per workgroup
  int n_blocks;    // column blocks
  int splits;      // K splits (workgroups per column block)
  int groups_per_split;
  bool chunked;    // a workgroup walks more than one LDS chunk of x (tiled layout only)
  size_t counter_bytes;  // zeroed completion counters at the start of the workspace
  size_t partial_bytes;  // float32 partial sums [splits][M][N]
};

enum { kEpiStore = 0, kEpiResidual = 1, kEpiSwiGLU = 2 };

// One validated QMM call (row-major or tiled weights, any epilogue).
struct QmmCall {
  const void* x;
  int64_t ldx;
  const float* x_ss;  // nullable: RMSNorm prologue from per-row sums of squares [M][ss_parts]
  int ss_parts;
  float eps;
  const void* wq;     // row-major codes, or the tiled pack (then scales / biases unused)
  const void* scales;
  const void* biases;
  bool tiled;
  int bits, M, N, K;
  int epilogue;
  const void* res;    // residual epilogue
  int64_t ldr;
  void* y;
  int64_t ldy;
  int y_f32;
  float* y_ss;        // residual epilogue: per-row sums of squares per 128 columns (nullable)
  void* workspace;
};

QmmPlan qmm_plan(int bits, int M, int N, int K, bool tiled);
hipError_t qmm_launch(const QmmPlan& plan, const QmmCall& call, hipStream_t stream);
size_t qmm_pack_bytes(int bits, int N, int K);
hipError_t qmm_pack(const void* wq, const void* scales, const void* biases, int bits, int N, int K, void* out,
                    hipStream_t stream);
hipError_t row_sumsq(const void* x, int64_t ldx, int M, int N, float* out, hipStream_t stream);
int qmm_sumsq_parts(int N);

// ----------------------------------------------------------- attention
struct AttnPlan {
  int rows;        // M * G query rows per KV head
  int row_tiles;   // ceil(rows / 32)
  int splits;      // KV splits per head
  int keys_per_split;
  size_t partial_bytes;
};
AttnPlan attn_plan(int M, int Hq, int Hkv, int D, int T, int B = 1);
// Several sequences in one call: sequence b has query rows row_start[b] ..
// row_start[b+1]-1 (device int32 [B+1], clamped to [0, total_rows]) and
// seq_len[b] keys (device int32 [B], clamped to [rows, T]) of the caches at
// b * kv_batch_stride (elements of the cache's type); M and T of the launch are
// the largest rows and keys of any sequence.
struct AttnBatch {
  const int32_t* row_start;
  const int32_t* seq_len;
  int64_t kv_batch_stride;
  int total_rows;
  int B;
};
// k_new / v_new (nullable): the M rows appended at positions T-M .. T-1, rows
// new_rs elements apart, KV head h at offset h*D; they are written into the
// caches and read from their source by the attention itself.
hipError_t attn_launch(const AttnPlan& plan, const void* q, int64_t q_rs, const void* k, const void* v,
                       int64_t kv_head_stride, int M, int Hq, int Hkv, int D, int T, float scale,
                       void* out, int64_t out_rs, void* workspace, hipStream_t stream,
                       const void* k_new = nullptr, const void* v_new = nullptr, int64_t new_rs = 0,
                       const uint32_t* tree = nullptr, const uint32_t* k_sb = nullptr,
                       const uint32_t* v_sb = nullptr, const AttnBatch* batch = nullptr);
// 8-bit KV cache: quantize M rows of a fused projection output into the caches
// (codes u8 [Hkv, T_cap, D], one bf16 scale | bf16 bias word per 64 codes) at
// positions pos .. pos+M-1; hs = head stride of the codes (elements).
hipError_t kv8_append(const void* src, int64_t ld, int k_off, int v_off, void* k_codes, void* k_sb, void* v_codes,
                      void* v_sb, int64_t hs, int M, int Hkv, int D, int pos, hipStream_t stream);

// ---------------------------------------------------------- acceptance
struct AcceptPlan {
  int entries;        // batch entries whose rows are prepared (1 if all rows shared)
  int rows_per_entry; // 2K + 1
  bool shared;        // both strides zero: per-position tables, one thread per trial
  size_t meta_bytes;  // per-row results of truncation
  size_t probs_bytes; // float32 probabilities (logits mode without probs_out)
  size_t table_bytes; // shared mode: 128-bit running sums [K+1][V]
  // Chunked pipeline (few rows): rows and draws cut into chunks over the whole chip.
  bool chunked;        // rows stage chunked
  bool draw_chunked;   // draw stage chunked
  int chunks;          // chunks per row
  size_t state_bytes;  // per-row select state
  size_t hist_bytes;   // per-row 4096-bin histograms, counts and masses
  size_t cand_bytes;   // per-row gathered keys
  size_t stats_bytes;  // logits mode: per-chunk max and sum
  size_t esum_bytes;   // per-(entry, chunk) sums of the draw weights
};
AcceptPlan accept_plan(int B, int K, int V, int input_kind, int64_t p_stride, int64_t q_stride);
size_t accept_workspace_total(const AcceptPlan& plan);
hipError_t accept_launch(const AcceptPlan& plan, const float* p, const float* q, int input_kind,
                         int64_t p_stride, int64_t q_stride, const int32_t* draft,
                         const float* uniforms, int B, int K, int V, float temperature, int top_k,
                         float top_p, int32_t* out_tokens, int32_t* out_n, float* probs_out,
                         void* workspace, hipStream_t stream);

// ------------------------------------------------------------- stack glue
hipError_t glue_rmsnorm(const void* x, int64_t ldx, void* y, int64_t ldy, int M, int N, float eps,
                        hipStream_t s);
hipError_t glue_add(const void* a, const void* b, void* y, int64_t n, hipStream_t s);
hipError_t glue_silu_mul(const void* gu, int64_t ldgu, void* y, int64_t ldy, int M, int I, hipStream_t s);
hipError_t glue_kv_append(const void* src, int64_t ld, int k_off, int v_off, void* kc, void* vc, int64_t hs,
                          int M, int Hkv, int D, int pos, hipStream_t s);

// Streaming-read ceiling (stream.hip): reads `bytes` (a multiple of 16) from src
// with `workgroups` workgroups; sink receives workgroups * 4 words.
hipError_t stream_read_launch(const void* src, size_t bytes, bool nontemporal, int workgroups, uint32_t* sink,
                              hipStream_t stream);

}  // namespace vq
