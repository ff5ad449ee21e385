// Exact Leviathan–Chen acceptance with identical top-k / top-p truncation, gfx950.
//
// The rule (page "The fastest way to run local LLMs on a Mac", section "Why
// exact acceptance matters"; page "Speculative decoding and MTP on Apple
// silicon", Facts: rejection sampling, identical truncation of both sides):
// accept draft d with probability min(1, p(d)/q(d)); at the first rejection draw
// from the normalised (p - q)+; after K acceptances draw from the next target row.
//
// Every decision is made in integer arithmetic so that it is reproducible bit
// for bit by any implementation (integer sums are associative):
//   mass m(x) = floor(p(x) * 2^40), order = (p descending, id ascending),
//   top-k keeps the first top_k, top-p keeps token t iff
//   (kept mass before t) * 2^24 < max(1, floor(top_p * 2^24)) * (top-k mass),
//   accept iff mu * mQ(d) * ZP < mP(d) * ZQ * 2^24 (mu = floor(u * 2^24)),
//   residual r = max(0, mP*ZQ - mQ*ZP), draw = smallest t with
//   r[0] + ... + r[t] > floor(mu_K * R / 2^24).
//
// GPU structure:
//   rows kernel    one workgroup per probability row: optional float32 softmax,
//                  validity check, top-k and top-p as radix selects over the
//                  50-bit order key (probability bits << 20 | (V-1-id)), weighted
//                  by count (top-k) or by mass (top-p); the row is summarised by
//                  its threshold key (kept <=> key >= threshold) and kept mass Z.
//   entry kernel   one workgroup per verify: the K accept tests, then the draw by
//                  a blocked 128-bit prefix scan over the residual in id order.
//   shared rows    (both batch strides 0, e.g. 10^6 trials of one verify) the
//                  running sums of every position's residual are tabulated once
//                  and each trial is one thread: K tests and a binary search.
#include "vq_internal.h"

namespace vq {
namespace {

typedef unsigned __int128 u128;

constexpr int kRowThreads = 512;
constexpr int kEntryThreads = 1024;
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;
constexpr int kKeyShiftTop = 44;  // digits at bit 44, 33, 22, 11, 0 cover the 50-bit key
constexpr float kLog2e = 1.4426950408889634f;

struct RowMeta {
  unsigned long long thresh;  // kept <=> order key >= thresh
  unsigned long long z;       // kept mass
  int status;                 // 0 = valid, 1 = invalid
  int pad[3];
};

__device__ __forceinline__ bool prob_ok(float v) { return v >= 0.f && v <= 1.f; }  // false for NaN

__device__ __forceinline__ unsigned long long mass_of(float v) {
  // floor(v * 2^40): exact in double for a float v in [0, 1].
  return (unsigned long long)((double)v * 1099511627776.0);
}

__device__ __forceinline__ unsigned long long key_of(float v, int x, int V) {
  const uint32_t b = (v == 0.f) ? 0u : __float_as_uint(v);
  return ((unsigned long long)b << 20) | (unsigned long long)(V - 1 - x);
}

// --------------------------------------------------------------- block scans
__device__ __forceinline__ unsigned long long shfl_up_u64(unsigned long long v, int off) {
  const uint32_t lo = __shfl_up((uint32_t)v, off);
  const uint32_t hi = __shfl_up((uint32_t)(v >> 32), off);
  return ((unsigned long long)hi << 32) | lo;
}

__device__ __forceinline__ u128 shfl_up_u128(u128 v, int off) {
  const unsigned long long lo = shfl_up_u64((unsigned long long)v, off);
  const unsigned long long hi = shfl_up_u64((unsigned long long)(v >> 64), off);
  return ((u128)hi << 64) | lo;
}

// Exclusive prefix sum over the block in thread order; also returns the total.
template <typename T, int NT>
__device__ T block_excl_scan(T v, T* lds /* NT/64 + 1 entries */, T& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  T inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    T o;
    if constexpr (sizeof(T) == 16) o = shfl_up_u128(inc, off); else o = shfl_up_u64(inc, off);
    if (lane >= off) inc += o;
  }
  __syncthreads();
  if (lane == 63) lds[wave] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    T run = 0;
    for (int w = 0; w < NT / 64; ++w) {
      const T t = lds[w];
      lds[w] = run;
      run += t;
    }
    lds[NT / 64] = run;
  }
  __syncthreads();
  total = lds[NT / 64];
  return lds[wave] + inc - v;
}

__device__ float block_reduce_max(float v, float* lds) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  float r = lds[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = fmaxf(r, lds[w]);
  return r;
}

__device__ float block_reduce_sum(float v, float* lds) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  float r = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) r += lds[w];
  return r;
}

// ------------------------------------------------------------- radix select
struct SelectLds {
  unsigned long long hist[kBins];
  unsigned long long scan[kRowThreads / 64 + 1];
  unsigned long long res_key, res_above, res_total;
  int flag;
};

// Walking the row in order (key descending) among elements with key >= lo,
// find the first element at which the running weight reaches `thr` (weight = 1
// or the mass). For the mass walk, thr is derived from the first pass's total:
// thr = ceil(tp * total / 2^24). Returns that element's key, the weight of the
// elements before it, and the total weight of the elements with key >= lo.
__device__ void radix_select(const float* row, int V, unsigned long long lo, bool by_mass, uint32_t tp,
                             unsigned long long thr_count, SelectLds& s, unsigned long long& out_key,
                             unsigned long long& out_above, unsigned long long& out_total) {
  const int tid = threadIdx.x;
  unsigned long long prefix = 0, above = 0, thr = thr_count, total = 0;
  for (int shift = kKeyShiftTop; shift >= 0; shift -= kDigitBits) {
    for (int b = tid; b < kBins; b += kRowThreads) s.hist[b] = 0;
    __syncthreads();
    for (int x = tid; x < V; x += kRowThreads) {
      const float v = row[x];
      const unsigned long long key = key_of(v, x, V);
      if (key < lo) continue;
      if (shift != kKeyShiftTop && (key >> (shift + kDigitBits)) != prefix) continue;
      const unsigned long long w = by_mass ? mass_of(v) : 1ull;
      if (w) atomicAdd(&s.hist[(key >> shift) & (kBins - 1)], w);
    }
    __syncthreads();
    // Thread t owns bins [kBins - 4(t+1), kBins - 4t): prefix order = descending digit.
    unsigned long long loc[4];
    unsigned long long lsum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      loc[i] = s.hist[kBins - 1 - (4 * tid + i)];
      lsum += loc[i];
    }
    unsigned long long tot;
    const unsigned long long excl = block_excl_scan<unsigned long long, kRowThreads>(lsum, s.scan, tot);
    if (shift == kKeyShiftTop) {
      total = tot;
      if (by_mass) {
        const u128 t = (u128)tp * tot;
        thr = (unsigned long long)((t + ((u128)1 << 24) - 1) >> 24);
      }
    }
    if (tid == 0) s.flag = 0;
    __syncthreads();
    if (above + excl < thr && thr <= above + excl + lsum) {
      unsigned long long run = above + excl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (run + loc[i] >= thr) {
          s.res_key = (prefix << kDigitBits) | (unsigned long long)(kBins - 1 - (4 * tid + i));
          s.res_above = run;
          s.flag = 1;
          break;
        }
        run += loc[i];
      }
    }
    __syncthreads();
    if (!s.flag) {  // thr exceeds the total weight (only when thr == 0 or total == 0)
      out_key = 0;
      out_above = 0;
      out_total = total;
      return;
    }
    prefix = s.res_key;
    above = s.res_above;
    __syncthreads();
  }
  out_key = prefix;
  out_above = above;
  out_total = total;
}

// ---------------------------------------------------------------- rows kernel
__global__ __launch_bounds__(kRowThreads) void accept_rows_kernel(
    const float* __restrict__ p, const float* __restrict__ q, int input_kind, int64_t p_stride,
    int64_t q_stride, int K, int V, float t_scale, int top_k, uint32_t tp, float* __restrict__ probs,
    RowMeta* __restrict__ meta) {
  __shared__ SelectLds s;
  __shared__ float red[kRowThreads / 64];
  __shared__ int bad;
  const int r = blockIdx.x;
  const int e = blockIdx.y;
  const int nrows = 2 * K + 1;
  const int tid = threadIdx.x;
  const float* src = (r <= K) ? p + (int64_t)e * p_stride + (int64_t)r * V
                              : q + (int64_t)e * q_stride + (int64_t)(r - K - 1) * V;
  const float* row = src;
  if (input_kind == 1) {  // logits -> float32 probabilities (each thread keeps its own elements)
    float* dst = probs + ((int64_t)e * nrows + r) * V;
    float mx = -INFINITY;
    for (int x = tid; x < V; x += kRowThreads) mx = fmaxf(mx, src[x]);
    mx = block_reduce_max(mx, red);
    float sum = 0.f;
    for (int x = tid; x < V; x += kRowThreads) sum += exp2f((src[x] - mx) * t_scale);
    sum = block_reduce_sum(sum, red);
    const float inv = 1.f / sum;
    for (int x = tid; x < V; x += kRowThreads) dst[x] = exp2f((src[x] - mx) * t_scale) * inv;
    __syncthreads();
    row = dst;
  }
  if (tid == 0) bad = 0;
  __syncthreads();
  int local_bad = 0;
  for (int x = tid; x < V; x += kRowThreads) local_bad |= !prob_ok(row[x]);
  if (local_bad) bad = 1;
  __syncthreads();
  RowMeta out{};
  if (bad) {
    if (tid == 0) {
      out.status = 1;
      meta[(int64_t)e * nrows + r] = out;
    }
    return;
  }
  const bool use_k = top_k > 0 && top_k < V;
  const bool use_p = tp < (1u << 24);
  unsigned long long lo = 0, key, above, total;
  if (use_k) {
    radix_select(row, V, 0, false, 0, (unsigned long long)top_k, s, key, above, total);
    lo = key;
  }
  unsigned long long z;
  unsigned long long thresh = lo;
  if (use_p) {
    radix_select(row, V, lo, true, tp, 0, s, key, above, total);
    thresh = key;
    // kept mass = mass before the crossing element + its own mass
    if (tid == 0) s.res_total = 0;
    __syncthreads();
    unsigned long long mine = 0;
    for (int x = tid; x < V; x += kRowThreads)
      if (key_of(row[x], x, V) == key) mine = mass_of(row[x]);
    if (mine) atomicAdd(&s.res_total, mine);
    __syncthreads();
    z = total ? above + s.res_total : 0;
  } else {
    // no top-p: kept mass = mass of every element with key >= lo
    unsigned long long ms = 0;
    for (int x = tid; x < V; x += kRowThreads) {
      const float v = row[x];
      if (key_of(v, x, V) >= lo) ms += mass_of(v);
    }
    unsigned long long tot;
    block_excl_scan<unsigned long long, kRowThreads>(ms, s.scan, tot);
    z = tot;
  }
  if (tid == 0) {
    out.thresh = thresh;
    out.z = z;
    out.status = z == 0 ? 1 : 0;
    meta[(int64_t)e * nrows + r] = out;
  }
}

// ---------------------------------------------------------- 128-bit helpers
__device__ __forceinline__ unsigned long long kept_mass(const float* row, int x, int V, const RowMeta& m) {
  const float v = row[x];
  return key_of(v, x, V) >= m.thresh ? mass_of(v) : 0ull;
}

// floor(mu * R / 2^24) for mu < 2^24 and R < 2^120 without overflowing 128 bits.
__device__ __forceinline__ u128 scaled_draw(uint32_t mu, u128 R) {
  const unsigned long long rh = (unsigned long long)(R >> 64);
  const unsigned long long rl = (unsigned long long)R;
  return (((u128)mu * rh) << 40) + (((u128)mu * rl) >> 24);
}

__device__ __forceinline__ bool accept_test(uint32_t mu, unsigned long long mq, unsigned long long zp,
                                            unsigned long long mp, unsigned long long zq) {
  return (u128)mu * mq * zp < ((u128)mp * zq << 24);
}

__device__ __forceinline__ bool uniform_ok(float u) { return u >= 0.f && u < 1.f; }
__device__ __forceinline__ uint32_t mu_of(float u) { return (uint32_t)((double)u * 16777216.0); }

// ---------------------------------------------------------------- entry kernel
__global__ __launch_bounds__(kEntryThreads) void accept_entry_kernel(
    const float* __restrict__ probs_p, const float* __restrict__ probs_q, int64_t pp_stride,
    int64_t qq_stride, const RowMeta* __restrict__ meta, int64_t meta_stride, const int32_t* __restrict__ draft,
    const float* __restrict__ uniforms, int K, int V, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ out_n) {
  __shared__ u128 scan[kEntryThreads / 64 + 1];
  __shared__ int s_j, s_bad, s_tok;
  __shared__ u128 s_tau;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const RowMeta* mrow = meta + (int64_t)b * meta_stride;
  const float* P = probs_p + (int64_t)b * pp_stride;  // row i at P + i*V
  const float* Q = probs_q + (int64_t)b * qq_stride;
  const int32_t* dr = draft + (int64_t)b * K;
  const float* us = uniforms + (int64_t)b * (K + 1);
  if (tid == 0) {
    int bad = 0;
    for (int i = 0; i < 2 * K + 1; ++i) bad |= mrow[i].status;
    for (int i = 0; i <= K; ++i) bad |= !uniform_ok(us[i]);
    for (int i = 0; i < K; ++i) bad |= (dr[i] < 0 || dr[i] >= V);
    int j = K;
    if (!bad) {
      for (int i = 0; i < K; ++i) {
        const int d = dr[i];
        const RowMeta mp = mrow[i], mq = mrow[K + 1 + i];
        const unsigned long long a = kept_mass(P + (int64_t)i * V, d, V, mp);
        const unsigned long long c = kept_mass(Q + (int64_t)i * V, d, V, mq);
        if (!accept_test(mu_of(us[i]), c, mp.z, a, mq.z)) {
          j = i;
          break;
        }
      }
    }
    s_bad = bad;
    s_j = j;
    s_tok = -1;
  }
  __syncthreads();
  const int j = s_j;
  if (s_bad) {
    for (int i = tid; i <= K; i += kEntryThreads) out_tokens[(int64_t)b * (K + 1) + i] = -1;
    if (tid == 0) out_n[b] = -1;
    return;
  }
  const float* Pj = P + (int64_t)j * V;
  const RowMeta mp = mrow[j];
  const bool resid = j < K;
  const float* Qj = resid ? Q + (int64_t)j * V : nullptr;
  const RowMeta mq = resid ? mrow[K + 1 + j] : RowMeta{};
  // Contiguous chunk of ids per thread (token-id order).
  const int per = (V + kEntryThreads - 1) / kEntryThreads;
  const int x0 = min(V, tid * per), x1 = min(V, x0 + per);
  auto weight = [&](int x, bool use_resid) -> u128 {
    const unsigned long long a = kept_mass(Pj, x, V, mp);
    if (!use_resid) return (u128)a;
    const unsigned long long c = kept_mass(Qj, x, V, mq);
    const u128 lhs = (u128)a * mq.z, rhs = (u128)c * mp.z;
    return lhs > rhs ? lhs - rhs : (u128)0;
  };
  bool use_resid = resid;
  u128 local = 0;
  for (int x = x0; x < x1; ++x) local += weight(x, use_resid);
  u128 R;
  u128 excl = block_excl_scan<u128, kEntryThreads>(local, scan, R);
  if (use_resid && R == 0) {  // p~_j == q~_j and the draft lay outside both supports: draw from p~_j
    use_resid = false;
    local = 0;
    for (int x = x0; x < x1; ++x) local += weight(x, false);
    excl = block_excl_scan<u128, kEntryThreads>(local, scan, R);
  }
  const u128 tau = scaled_draw(mu_of(us[K]), R);
  if (excl <= tau && tau < excl + local) {
    u128 run = excl;
    for (int x = x0; x < x1; ++x) {
      run += weight(x, use_resid);
      if (run > tau) {
        s_tok = x;
        break;
      }
    }
  }
  __syncthreads();
  for (int i = tid; i <= K; i += kEntryThreads) {
    int32_t t = -1;
    if (i < j) t = dr[i];
    else if (i == j) t = s_tok;
    out_tokens[(int64_t)b * (K + 1) + i] = t;
  }
  if (tid == 0) out_n[b] = j;
  (void)s_tau;
}

// ------------------------------------------------------------- shared rows
// Running sums of each position's draw weights: table[j][x] = sum_{t <= x} r_j(t).
__global__ __launch_bounds__(kEntryThreads) void accept_table_kernel(
    const float* __restrict__ P, const float* __restrict__ Q, const RowMeta* __restrict__ meta, int K,
    int V, u128* __restrict__ table) {
  __shared__ u128 scan[kEntryThreads / 64 + 1];
  const int j = blockIdx.x;
  const int tid = threadIdx.x;
  int bad = 0;
  for (int i = 0; i < 2 * K + 1; ++i) bad |= meta[i].status;
  if (bad) return;
  const float* Pj = P + (int64_t)j * V;
  const RowMeta mp = meta[j];
  const bool resid = j < K;
  const float* Qj = resid ? Q + (int64_t)j * V : nullptr;
  const RowMeta mq = resid ? meta[K + 1 + j] : RowMeta{};
  const int per = (V + kEntryThreads - 1) / kEntryThreads;
  const int x0 = min(V, tid * per), x1 = min(V, x0 + per);
  auto weight = [&](int x, bool use_resid) -> u128 {
    const unsigned long long a = kept_mass(Pj, x, V, mp);
    if (!use_resid) return (u128)a;
    const unsigned long long c = kept_mass(Qj, x, V, mq);
    const u128 lhs = (u128)a * mq.z, rhs = (u128)c * mp.z;
    return lhs > rhs ? lhs - rhs : (u128)0;
  };
  bool use_resid = resid;
  u128 local = 0;
  for (int x = x0; x < x1; ++x) local += weight(x, use_resid);
  u128 R;
  u128 excl = block_excl_scan<u128, kEntryThreads>(local, scan, R);
  if (use_resid && R == 0) {
    use_resid = false;
    local = 0;
    for (int x = x0; x < x1; ++x) local += weight(x, false);
    excl = block_excl_scan<u128, kEntryThreads>(local, scan, R);
  }
  u128* out = table + (int64_t)j * V;
  u128 run = excl;
  for (int x = x0; x < x1; ++x) {
    run += weight(x, use_resid);
    out[x] = run;
  }
}

__global__ __launch_bounds__(256) void accept_trials_kernel(
    const float* __restrict__ P, const float* __restrict__ Q, const RowMeta* __restrict__ meta,
    const u128* __restrict__ table, const int32_t* __restrict__ draft, const float* __restrict__ uniforms,
    int B, int K, int V, int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_n) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int32_t* dr = draft + (int64_t)b * K;
  const float* us = uniforms + (int64_t)b * (K + 1);
  int32_t* ot = out_tokens + (int64_t)b * (K + 1);
  int bad = 0;
  for (int i = 0; i < 2 * K + 1; ++i) bad |= meta[i].status;
  for (int i = 0; i <= K; ++i) bad |= !uniform_ok(us[i]);
  for (int i = 0; i < K; ++i) bad |= (dr[i] < 0 || dr[i] >= V);
  if (bad) {
    for (int i = 0; i <= K; ++i) ot[i] = -1;
    out_n[b] = -1;
    return;
  }
  int j = K;
  for (int i = 0; i < K; ++i) {
    const int d = dr[i];
    const RowMeta mp = meta[i], mq = meta[K + 1 + i];
    const unsigned long long a = kept_mass(P + (int64_t)i * V, d, V, mp);
    const unsigned long long c = kept_mass(Q + (int64_t)i * V, d, V, mq);
    if (!accept_test(mu_of(us[i]), c, mp.z, a, mq.z)) {
      j = i;
      break;
    }
  }
  const u128* tj = table + (int64_t)j * V;
  const u128 tau = scaled_draw(mu_of(us[K]), tj[V - 1]);
  int lo = 0, hi = V - 1;  // smallest x with tj[x] > tau; tj[V-1] > tau always
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (tj[mid] > tau) hi = mid; else lo = mid + 1;
  }
  for (int i = 0; i <= K; ++i) ot[i] = i < j ? dr[i] : (i == j ? lo : -1);
  out_n[b] = j;
}

}  // namespace

AcceptPlan accept_plan(int B, int K, int V, int input_kind, int64_t p_stride, int64_t q_stride) {
  AcceptPlan p{};
  p.shared = (p_stride == 0 && q_stride == 0);
  p.entries = p.shared ? 1 : B;
  p.rows_per_entry = 2 * K + 1;
  p.meta_bytes = align_up((size_t)p.entries * p.rows_per_entry * sizeof(RowMeta), 256);
  p.probs_bytes = input_kind == 1 ? align_up((size_t)p.entries * p.rows_per_entry * V * sizeof(float), 256) : 0;
  p.table_bytes = p.shared ? align_up((size_t)(K + 1) * V * sizeof(u128), 256) : 0;
  return p;
}

hipError_t accept_launch(const AcceptPlan& plan, const float* p, const float* q, int input_kind,
                         int64_t p_stride, int64_t q_stride, const int32_t* draft,
                         const float* uniforms, int B, int K, int V, float temperature, int top_k,
                         float top_p, int32_t* out_tokens, int32_t* out_n, float* probs_out,
                         void* workspace, hipStream_t stream) {
  char* ws = reinterpret_cast<char*>(workspace);
  RowMeta* meta = reinterpret_cast<RowMeta*>(ws);
  ws += plan.meta_bytes;
  float* probs = nullptr;
  if (input_kind == 1) {
    probs = probs_out ? probs_out : reinterpret_cast<float*>(ws);
    ws += plan.probs_bytes;
  }
  u128* table = plan.shared ? reinterpret_cast<u128*>(ws) : nullptr;
  const float t_scale = input_kind == 1 ? kLog2e / temperature : 0.f;
  uint32_t tp = (uint32_t)((double)top_p * 16777216.0);
  if (tp < 1) tp = 1;
  if (tp > (1u << 24)) tp = 1u << 24;
  if (q == nullptr) q = p;  // K == 0: no draft rows are read
  hipLaunchKernelGGL(accept_rows_kernel, dim3(plan.rows_per_entry, plan.entries), dim3(kRowThreads), 0,
                     stream, p, q, input_kind, p_stride, q_stride, K, V, t_scale, top_k, tp, probs, meta);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Rows to read from now on: the probabilities (computed or given).
  const float* PP;
  const float* QQ;
  int64_t pps, qqs;
  if (input_kind == 1) {
    PP = probs;
    QQ = probs + (int64_t)(K + 1) * V;
    pps = qqs = (int64_t)plan.rows_per_entry * V;
  } else {
    PP = p;
    QQ = q;
    pps = p_stride;
    qqs = q_stride;
  }
  if (plan.shared) {
    hipLaunchKernelGGL(accept_table_kernel, dim3(K + 1), dim3(kEntryThreads), 0, stream, PP, QQ, meta, K, V,
                       table);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(accept_trials_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, PP, QQ, meta, table,
                       draft, uniforms, B, K, V, out_tokens, out_n);
    return hipGetLastError();
  }
  if (input_kind == 1) pps = qqs = (int64_t)plan.rows_per_entry * V;
  hipLaunchKernelGGL(accept_entry_kernel, dim3(B), dim3(kEntryThreads), 0, stream, PP, QQ, pps, qqs, meta,
                     (int64_t)plan.rows_per_entry, draft, uniforms, K, V, out_tokens, out_n);
  return hipGetLastError();
}

}  // namespace vq
