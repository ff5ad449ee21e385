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
#include "vq.h"
#include "lanes.h"
#include "vq_internal.h"

namespace vq {
namespace {

typedef unsigned __int128 u128;
typedef unsigned long long u64;

constexpr int kRowThreads = 1024;
constexpr int kEntryThreads = 1024;
constexpr int kUnroll = 8;          // independent loads in flight per thread per pass
constexpr int kDigitBits = 12;
constexpr int kBins = 1 << kDigitBits;
constexpr float kLog2e = 1.4426950408889634f;
// Radix levels over the 50-bit order key: bits [49:38], [37:26], [25:14], [13:2], [1:0].
__constant__ int kLevelShift[5] = {38, 26, 14, 2, 0};
__constant__ int kLevelBits[5] = {12, 12, 12, 12, 2};

struct RowMeta {
  u64 thresh;  // kept <=> order key >= thresh
  u64 z;       // kept mass
  int status;  // 0 = valid, 1 = invalid
  int pad[3];
};

// logit * (log2(e) / T), rounded to float32 on its own: never fused with the
// subtraction of the row maximum, which is taken over these rounded values.
__device__ __forceinline__ float scaled_logit(float v, float t_scale) {
#pragma clang fp contract(off)
  return v * t_scale;
}

__device__ __forceinline__ bool prob_ok(float v) { return v >= 0.f && v <= 1.f; }  // false for NaN

__device__ __forceinline__ u64 mass_of(float v) {
  // floor(v * 2^40): exact in double for a float v in [0, 1].
  return (u64)((double)v * 1099511627776.0);
}

__device__ __forceinline__ u64 key_of(float v, int x, int V) {
  const uint32_t b = (v == 0.f) ? 0u : __float_as_uint(v);
  return ((u64)b << 20) | (u64)(V - 1 - x);
}

// Apply f(x, v) to every element of a row. The body of the row is read as
// float4 (a scalar head up to 16-byte alignment and a scalar tail around it);
// thread t takes float4 units t + i*blockDim (coalesced), kUnroll units in
// flight before any is used.
template <typename F>
__device__ __forceinline__ void for_row(const float* __restrict__ row, int V, F&& f) {
  const int nt = blockDim.x;
  const int head = min(V, (int)(((16u - (uint32_t)(reinterpret_cast<uintptr_t>(row) & 15u)) & 15u) >> 2));
  for (int x = threadIdx.x; x < head; x += nt) f(x, row[x]);
  const float4* body = reinterpret_cast<const float4*>(row + head);
  const int nb = (V - head) >> 2;
  for (int base = threadIdx.x; base < nb; base += nt * kUnroll) {
    float4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = body[min(base + u * nt, nb - 1)];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = base + u * nt;
      if (i < nb) {
        const int x = head + 4 * i;
        f(x, v[u].x);
        f(x + 1, v[u].y);
        f(x + 2, v[u].z);
        f(x + 3, v[u].w);
      }
    }
  }
  for (int x = head + 4 * nb + threadIdx.x; x < V; x += nt) f(x, row[x]);
}

// --------------------------------------------------------------- block scans
__device__ __forceinline__ u64 shfl_up_u64(u64 v, int off) {
  const uint32_t lo = __shfl_up((uint32_t)v, off);
  const uint32_t hi = __shfl_up((uint32_t)(v >> 32), off);
  return ((u64)hi << 32) | lo;
}

__device__ __forceinline__ u128 shfl_up_u128(u128 v, int off) {
  const u64 lo = shfl_up_u64((u64)v, off);
  const u64 hi = shfl_up_u64((u64)(v >> 64), off);
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
  v = max64_lanes(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  float r = lds[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = fmaxf(r, lds[w]);
  return r;
}

__device__ float block_reduce_sum(float v, float* lds) {
  v = sum64_lanes(v);
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
  u64 mass[kBins];
  uint32_t cnt[kBins];
  u64 scan[kRowThreads / 64 + 1];
  u64 res_key, res_above, res_total;
  uint32_t res_cnt;
  int flag;
};

// ------------------------------------------- state of the chunked pipeline
constexpr int kChunk = 4096;      // elements per (chunk, row) workgroup (4096 measured fastest of 2048-32768)
constexpr int kCT = 256;           // threads of the chunk kernels
constexpr int kStage = 8192;       // keys a compact pass stages in LDS
constexpr int kCandCap = 16384;    // keys gathered per row (2^14: a level-2 region never holds more)
constexpr int kTopShift = 38;      // level 0: the histogram bin of a key is key >> 38 (12 bits)
constexpr int kLevels = 3;         // histogram levels: shifts 38, 26, 14 (12 bits each)
constexpr int kCandBits = 8;       // digit width of the selects over gathered keys

// The select state of a row. A region is the set of keys with
// (key >> shift) == prefix; the select is known to cross inside the current
// region. A region too crowded to gather is refined by one more histogram level
// over the whole chip (shift 38 -> 26 -> 14); a level-2 region holds at most
// 2^14 distinct keys, so it can always be gathered.
struct RowState {
  u64 total;         // mass of the row
  u64 above;         // select weight (count or mass) of the keys above the region
  u64 above_mass;    // mass of the keys above the region
  u64 thr;           // weight the select must reach
  u64 prefix;        // the region
  uint32_t bad;      // an invalid probability was seen
  uint32_t cand_n;   // keys gathered
  int shift;         // 38, 26 or 14
  int phase;         // 0 top-k select, 1 top-p select, 3 left to the rows kernel
  int pending;       // a compact + resolve is due
  int refine;        // the histogram level due (1 or 2), 0 none
  int levels;        // levels the top-k select went through (1..3)
  int kbin[kLevels]; // its crossing bin at each of them
};

// Clears a row's level-0 histogram and select state: the first kernel of every
// call (the workspace layout depends on the shapes, so nothing is assumed zero;
// the level-1 and level-2 histograms are cleared when a row needs them).
__global__ __launch_bounds__(256) void rows_clear_kernel(RowState* __restrict__ st, uint32_t* __restrict__ hcnt,
                                                         u64* __restrict__ hmass) {
  const int r = blockIdx.x;
  for (int b = threadIdx.x; b < kBins; b += blockDim.x) {
    hcnt[(int64_t)r * kBins + b] = 0u;
    hmass[(int64_t)r * kBins + b] = 0ull;
  }
  if (threadIdx.x == 0) st[r] = RowState{};
}

// Walking the row in order (key descending) among elements with key >= lo,
// find the first element at which the running weight reaches `thr` (weight 1 for
// count, the mass for by_mass). For the mass walk thr is derived from the
// first level's total: thr = ceil(tp * total / 2^24). Returns the element's
// key and mass, the weight before it and the total weight of the elements with
// key >= lo. The walk ends at the first level whose crossing bin holds a single
// element; one more pass then reads that element.
__device__ void radix_select(const float* __restrict__ row, int V, u64 lo, bool by_mass, uint32_t tp,
                             u64 thr_count, SelectLds& s, u64& out_key, u64& out_mass, u64& out_above,
                             u64& out_total) {
  const int tid = threadIdx.x;
  u64 prefix = 0, above = 0, thr = thr_count, total = 0;
  int hi_shift = 50;  // bits above the current digit are fixed to `prefix`
  for (int level = 0; level < 5; ++level) {
    const int shift = kLevelShift[level];
    const int bits = kLevelBits[level];
    const int nb = 1 << bits;
    for (int b = tid; b < nb; b += kRowThreads) {
      s.mass[b] = 0;
      s.cnt[b] = 0;
    }
    __syncthreads();
    for_row(row, V, [&](int x, float v) {
      const u64 key = key_of(v, x, V);
      if (key < lo) return;
      if (level > 0 && (key >> hi_shift) != prefix) return;
      const int bin = (int)((key >> shift) & (u64)(nb - 1));
      atomicAdd(&s.cnt[bin], 1u);
      if (by_mass) {
        const u64 w = mass_of(v);
        if (w) atomicAdd(&s.mass[bin], w);
      }
    });
    __syncthreads();
    // Thread t owns bins nb-1-4t, ..., nb-4-4t: thread order = descending digit.
    u64 w0, w1, w2, w3;
    uint32_t c0, c1, c2, c3;
    {
      const int b = nb - 1 - 4 * tid;
      c0 = b >= 0 ? s.cnt[b] : 0u;
      c1 = b >= 1 ? s.cnt[b - 1] : 0u;
      c2 = b >= 2 ? s.cnt[b - 2] : 0u;
      c3 = b >= 3 ? s.cnt[b - 3] : 0u;
      if (by_mass) {
        w0 = b >= 0 ? s.mass[b] : 0ull;
        w1 = b >= 1 ? s.mass[b - 1] : 0ull;
        w2 = b >= 2 ? s.mass[b - 2] : 0ull;
        w3 = b >= 3 ? s.mass[b - 3] : 0ull;
      } else {
        w0 = c0; w1 = c1; w2 = c2; w3 = c3;
      }
    }
    const u64 lsum = w0 + w1 + w2 + w3;
    u64 tot;
    const u64 excl = block_excl_scan<u64, kRowThreads>(lsum, s.scan, tot);
    if (level == 0) {
      total = tot;
      if (by_mass) {
        const u128 t = (u128)tp * tot;
        thr = (u64)((t + ((u128)1 << 24) - 1) >> 24);
      }
    }
    if (tid == 0) s.flag = 0;
    __syncthreads();
    const u64 r0 = above + excl;
    if (r0 < thr && thr <= r0 + lsum) {
      const u64 r1 = r0 + w0, r2 = r1 + w1, r3 = r2 + w2;
      int i;
      u64 run;
      uint32_t c;
      if (r1 >= thr) { i = 0; run = r0; c = c0; }
      else if (r2 >= thr) { i = 1; run = r1; c = c1; }
      else if (r3 >= thr) { i = 2; run = r2; c = c2; }
      else { i = 3; run = r3; c = c3; }
      s.res_key = (prefix << bits) | (u64)(nb - 1 - (4 * tid + i));
      s.res_above = run;
      s.res_cnt = c;
      s.flag = 1;
    }
    __syncthreads();
    if (!s.flag) {  // thr exceeds the total weight (only when thr == 0 or total == 0)
      out_key = 0;
      out_mass = 0;
      out_above = 0;
      out_total = total;
      return;
    }
    prefix = s.res_key;
    above = s.res_above;
    hi_shift = shift;
    const uint32_t c = s.res_cnt;
    __syncthreads();
    if (c == 1 || level == 4) {
      // The crossing bin holds one element (always so once the whole key is fixed).
      for_row(row, V, [&](int x, float v) {
        const u64 key = key_of(v, x, V);
        if (key >= lo && (key >> hi_shift) == prefix) {
          s.res_key = key;
          s.res_total = mass_of(v);
        }
      });
      __syncthreads();
      out_key = s.res_key;
      out_mass = s.res_total;
      out_above = above;
      out_total = total;
      __syncthreads();
      return;
    }
  }
}

// ---------------------------------------------------------------- rows kernel
__global__ __launch_bounds__(kRowThreads) void accept_rows_kernel(
    const float* __restrict__ p, const float* __restrict__ q, int input_kind, int64_t p_stride,
    int64_t q_stride, int K, int V, float t_scale, int top_k, uint32_t tp, float* __restrict__ probs,
    RowMeta* __restrict__ meta, RowState* __restrict__ gate, uint32_t* __restrict__ hcnt, u64* __restrict__ hmass) {
  __shared__ SelectLds s;
  __shared__ float red[kRowThreads / 64];
  __shared__ int bad;
  const int r = blockIdx.x;
  const int e = blockIdx.y;
  const int nrows = 2 * K + 1;
  const int tid = threadIdx.x;
  // After the chunked pipeline only the rows it left over (crossing bin too
  // crowded to gather) are done here.
  const int ri = e * nrows + r;
  if (gate && gate[ri].phase != 3) return;
  const float* src = (r <= K) ? p + (int64_t)e * p_stride + (int64_t)r * V
                              : q + (int64_t)e * q_stride + (int64_t)(r - K - 1) * V;
  const float* row = src;
  if (tid == 0) bad = 0;
  int local_bad = 0;
  u64 msum = 0;  // mass of the whole row (used when nothing is truncated)
  if (input_kind == 1) {
    // float32 softmax(logits * t_scale in base 2): one pass for the running
    // (max, sum) of every thread, merged over the block, one pass to write the
    // probabilities, check them and sum their masses. A NaN logit gives a NaN
    // probability, a +inf logit makes every probability NaN: both are invalid.
    // The scaled logit is rounded to float32 before the max is subtracted in
    // both passes (no fused multiply-subtract), so the largest element gets
    // exp2(0) = 1 and no probability exceeds 1 however large the logits are.
    float* dst = probs + ((int64_t)e * nrows + r) * V;
    float mx = -INFINITY, sm = 0.f;
    for_row(src, V, [&](int, float v) {
      const float a = scaled_logit(v, t_scale);
      if (a > mx) {
        sm = sm * exp2f(mx - a) + 1.f;
        mx = a;
      } else if (a > -INFINITY) {
        sm += exp2f(a - mx);
      }
    });
    const float gmx = block_reduce_max(mx, red);
    const float part = (mx == -INFINITY) ? 0.f : sm * exp2f(mx - gmx);
    const float sum = block_reduce_sum(part, red);
    const float inv = 1.f / sum;
    for_row(src, V, [&](int x, float v) {
      const float pv = exp2f(scaled_logit(v, t_scale) - gmx) * inv;
      dst[x] = pv;
      if (prob_ok(pv)) msum += mass_of(pv); else local_bad = 1;
    });
    row = dst;
  } else {
    for_row(row, V, [&](int, float v) {
      if (prob_ok(v)) msum += mass_of(v); else local_bad = 1;
    });
  }
  __syncthreads();
  if (local_bad) bad = 1;
  u64 mtot;
  block_excl_scan<u64, kRowThreads>(msum, s.scan, mtot);  // ends with a barrier
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
  u64 lo = 0, key, kmass, above, total;
  if (use_k) {
    radix_select(row, V, 0, false, 0, (u64)top_k, s, key, kmass, above, total);
    lo = key;
  }
  u64 z = mtot;
  u64 thresh = lo;
  if (use_p) {
    radix_select(row, V, lo, true, tp, 0, s, key, kmass, above, total);
    thresh = key;
    z = total ? above + kmass : 0;  // kept mass = mass before the last kept element + its own
  } else if (use_k) {
    u64 ms = 0;
    for_row(row, V, [&](int x, float v) {
      if (key_of(v, x, V) >= lo) ms += mass_of(v);
    });
    block_excl_scan<u64, kRowThreads>(ms, s.scan, z);
  }
  if (tid == 0) {
    out.thresh = thresh;
    out.z = z;
    out.status = z == 0 ? 1 : 0;
    meta[(int64_t)e * nrows + r] = out;
  }
}

// ---------------------------------------------------------- 128-bit helpers
__device__ __forceinline__ u64 kept_mass_v(float v, int x, int V, const RowMeta& m) {
  return key_of(v, x, V) >= m.thresh ? mass_of(v) : 0ull;
}

__device__ __forceinline__ u64 kept_mass(const float* row, int x, int V, const RowMeta& m) {
  return kept_mass_v(row[x], x, V, m);
}

// floor(mu * R / 2^24) for mu < 2^24 and R < 2^120 without overflowing 128 bits.
__device__ __forceinline__ u128 scaled_draw(uint32_t mu, u128 R) {
  const u64 rh = (u64)(R >> 64);
  const u64 rl = (u64)R;
  return (((u128)mu * rh) << 40) + (((u128)mu * rl) >> 24);
}

__device__ __forceinline__ bool accept_test(uint32_t mu, u64 mq, u64 zp, u64 mp, u64 zq) {
  return (u128)mu * mq * zp < ((u128)mp * zq << 24);
}

__device__ __forceinline__ bool uniform_ok(float u) { return u >= 0.f && u < 1.f; }
__device__ __forceinline__ uint32_t mu_of(float u) { return (uint32_t)((double)u * 16777216.0); }

// Draw weight of token x: the residual max(0, mP*ZQ - mQ*ZP) or the mass mP.
struct DrawRow {
  const float* P;
  const float* Q;  // null: weight = mP
  RowMeta mp, mq;
  int V;
  __device__ __forceinline__ u128 w(int x, float pv, float qv) const {
    const u64 a = kept_mass_v(pv, x, V, mp);
    if (!Q) return (u128)a;
    if (a == 0) return 0;
    const u64 c = kept_mass_v(qv, x, V, mq);
    const u128 lhs = (u128)a * mq.z, rhs = (u128)c * mp.z;
    return lhs > rhs ? lhs - rhs : (u128)0;
  }
};

// Smallest x with w(0) + ... + w(x) > floor(mu * R / 2^24), R = total weight.
// Pass 1: every wave sums a contiguous chunk of ids (coalesced 64 at a time).
// Pass 2: the whole block refines the one chunk that holds the draw, with a
// contiguous sub-chunk per thread. Returns -1 if R == 0 (only then).
__device__ int draw_token(const DrawRow& d, uint32_t mu, u128* scan, u128* wsum, int* s_tok) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NW = kEntryThreads / 64;
  const int V = d.V;
  const int chunk = ((V + NW - 1) / NW + 3) & ~3;  // multiple of 4: chunk starts stay 16-byte aligned
  const int c0 = min(V, wave * chunk), c1 = min(V, c0 + chunk);
  u128 local = 0;
  {
    // Scalar up to a multiple of 4 elements from the chunk start when the rows
    // are not 16-byte aligned there; float4 otherwise, 4 units per lane in flight.
    const bool vec = ((reinterpret_cast<uintptr_t>(d.P + c0) | (d.Q ? reinterpret_cast<uintptr_t>(d.Q + c0) : 0)) & 15) == 0;
    const int nv = vec ? (c1 - c0) >> 2 : 0;
    const float4* P4 = reinterpret_cast<const float4*>(d.P + c0);
    const float4* Q4 = reinterpret_cast<const float4*>(d.Q ? d.Q + c0 : d.P + c0);
    for (int base = lane; base < nv; base += 64 * 4) {
      float4 pv[4], qv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = min(base + 64 * u, nv - 1);
        pv[u] = P4[i];
        qv[u] = Q4[i];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = base + 64 * u;
        if (i < nv) {
          const int x = c0 + 4 * i;
          local += d.w(x, pv[u].x, qv[u].x);
          local += d.w(x + 1, pv[u].y, qv[u].y);
          local += d.w(x + 2, pv[u].z, qv[u].z);
          local += d.w(x + 3, pv[u].w, qv[u].w);
        }
      }
    }
    for (int x = c0 + 4 * nv + lane; x < c1; x += 64) local += d.w(x, d.P[x], d.Q ? d.Q[x] : 0.f);
  }
  // wave total
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const u64 lo = (u64)local, hi = (u64)(local >> 64);
    const u64 olo = ((u64)__shfl_xor((uint32_t)(lo >> 32), off) << 32) | __shfl_xor((uint32_t)lo, off);
    const u64 ohi = ((u64)__shfl_xor((uint32_t)(hi >> 32), off) << 32) | __shfl_xor((uint32_t)hi, off);
    local += ((u128)ohi << 64) | olo;
  }
  if (tid == 0) *s_tok = -1;
  if (lane == 0) wsum[wave] = local;
  __syncthreads();
  u128 R = 0, before = 0;
  int cw = -1;
  for (int w = 0; w < NW; ++w) R += wsum[w];
  if (R == 0) return -1;
  const u128 tau = scaled_draw(mu, R);
  for (int w = 0; w < NW; ++w) {  // the chunk that holds the draw
    if (cw < 0 && before + wsum[w] > tau) cw = w;
    if (cw < 0) before += wsum[w];
  }
  // Refine chunk cw: thread t sums a contiguous sub-chunk.
  const int q0 = min(V, cw * chunk), q1 = min(V, q0 + chunk);
  const int per = (q1 - q0 + kEntryThreads - 1) / kEntryThreads;
  const int x0 = min(q1, q0 + tid * per), x1 = min(q1, x0 + per);
  u128 mine = 0;
  for (int x = x0; x < x1; ++x) mine += d.w(x, d.P[x], d.Q ? d.Q[x] : 0.f);
  u128 tot;
  const u128 excl = before + block_excl_scan<u128, kEntryThreads>(mine, scan, tot);
  if (excl <= tau && tau < excl + mine) {
    u128 run = excl;
    for (int x = x0; x < x1; ++x) {
      run += d.w(x, d.P[x], d.Q ? d.Q[x] : 0.f);
      if (run > tau) {
        *s_tok = x;
        break;
      }
    }
  }
  __syncthreads();
  return *s_tok;
}

// ---------------------------------------------------------------- entry kernel
// The K accept tests of one verify entry (and the validity of its rows, draft
// ids and uniforms): the first rejected position j (K if every draft passes).
__device__ int entry_decide(const float* P, const float* Q, const RowMeta* mrow, const int32_t* dr, const float* us,
                            int K, int V, int* bad_out) {
  // Called by one whole wave (K <= 15, so lane i holds draft i, uniform i and the
  // meta of rows i and K + 1 + i): the loads of every test go out together and
  // the first rejection is the lowest lane whose test fails.
  // Indices are clamped so that every lane loads (a load under a per-lane
  // condition is followed by a full wait in the compiled code, one round trip
  // each); lanes past the data select the defaults.
  const int lane = threadIdx.x & 63;
  const RowMeta mp_l = mrow[min(lane, 2 * K)];
  const RowMeta mq_l = mrow[min(K + 1 + lane, 2 * K)];
  const float u_l = us[min(lane, K)];
  int d_l = 0;
  if (K > 0) d_l = dr[min(lane, K - 1)];  // K is the same for the whole wave
  const RowMeta mp = lane < 2 * K + 1 ? mp_l : RowMeta{};
  const RowMeta mq = lane < K ? mq_l : RowMeta{};
  const float u = lane <= K ? u_l : 0.f;
  const int d = lane < K ? d_l : 0;
  int bad = 0;
  if (lane < 2 * K + 1) bad |= mp.status;
  if (lane <= K) bad |= !uniform_ok(u);
  if (lane < K) bad |= (d < 0 || d >= V);
  const bool any_bad = __ballot(bad != 0) != 0ull;
  int j = K;
  if (!any_bad) {
    bool fail = false;
    if (lane < K) {
      const u64 a = kept_mass(P + (int64_t)lane * V, d, V, mp);
      const u64 c = kept_mass(Q + (int64_t)lane * V, d, V, mq);
      fail = !accept_test(mu_of(u), c, mp.z, a, mq.z);
    }
    const unsigned long long m = __ballot(fail);
    if (m) j = __ffsll((long long)m) - 1;
  }
  *bad_out = any_bad ? 1 : 0;
  return j;
}

__global__ __launch_bounds__(kEntryThreads) void accept_entry_kernel(
    const float* __restrict__ probs_p, const float* __restrict__ probs_q, int64_t pp_stride,
    int64_t qq_stride, const RowMeta* __restrict__ meta, int64_t meta_stride, const int32_t* __restrict__ draft,
    const float* __restrict__ uniforms, int K, int V, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ out_n) {
  __shared__ u128 scan[kEntryThreads / 64 + 1];
  __shared__ u128 wsum[kEntryThreads / 64];
  __shared__ int s_j, s_bad, s_tok;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const RowMeta* mrow = meta + (int64_t)b * meta_stride;
  const float* P = probs_p + (int64_t)b * pp_stride;  // row i at P + i*V
  const float* Q = probs_q + (int64_t)b * qq_stride;
  const int32_t* dr = draft + (int64_t)b * K;
  const float* us = uniforms + (int64_t)b * (K + 1);
  if (tid < 64) {
    int bad;
    const int j = entry_decide(P, Q, mrow, dr, us, K, V, &bad);
    if (tid == 0) {
      s_bad = bad;
      s_j = j;
    }
  }
  __syncthreads();
  const int j = s_j;
  if (s_bad) {
    for (int i = tid; i <= K; i += kEntryThreads) out_tokens[(int64_t)b * (K + 1) + i] = -1;
    if (tid == 0) out_n[b] = -1;
    return;
  }
  DrawRow d;
  d.P = P + (int64_t)j * V;
  d.mp = mrow[j];
  d.Q = j < K ? Q + (int64_t)j * V : nullptr;
  d.mq = j < K ? mrow[K + 1 + j] : RowMeta{};
  d.V = V;
  const uint32_t mu = mu_of(us[K]);
  int tok = draw_token(d, mu, scan, wsum, &s_tok);
  if (tok < 0) {  // p~_j == q~_j and the draft lay outside both supports: draw from p~_j
    __syncthreads();
    d.Q = nullptr;
    tok = draw_token(d, mu, scan, wsum, &s_tok);
  }
  for (int i = tid; i <= K; i += kEntryThreads) {
    int32_t t = -1;
    if (i < j) t = dr[i];
    else if (i == j) t = tok;
    out_tokens[(int64_t)b * (K + 1) + i] = t;
  }
  if (tid == 0) out_n[b] = j;
}

// ----------------------------------------------------------- chunked pipeline
// The rows and the draw spread over the whole chip: every row is cut into
// chunks of kChunk elements, one 256-thread workgroup per (chunk, row).
//   stats    (logits) per-chunk running max and sum of exp2
//   hist     probabilities (written in logits mode), validity, the row's mass,
//            and the 4096-bin histogram (count, mass) of the top 12 key bits,
//            merged into a per-row histogram with global atomics
//   find     (one workgroup per row) the bin where the first select crosses;
//            rows without truncation, invalid rows or an empty select finish
//   refine   (levels 1 and 2, a chunked histogram pass + a per-row find each)
//            a crossing bin holding more than kCandCap keys is narrowed by the
//            next 12 key bits, over the whole chip; after level 2 a region
//            holds at most 2^14 = kCandCap keys
//   compact  the keys of the crossing region gathered per row
//   resolve  (one workgroup per row) radix select over the gathered keys; a
//            top-p walk after top-k that crosses in a bin above the top-k
//            path asks for a second compact + resolve
// Only a top-p walk after a top-k wider than kCandCap can meet a region too
// crowded to gather; the single-workgroup rows kernel above finishes those
// rows. Every count is an integer, so the result does not depend on how the
// work is split.
// f(x, v) for x in [x0, x1): scalar head to 16-byte alignment, float4 body with
// kUnroll units per thread in flight, scalar tail.
template <typename F>
__device__ __forceinline__ void for_range(const float* __restrict__ row, int x0, int x1, F&& f) {
  const int nt = blockDim.x;
  const int lead = (int)(((16u - (uint32_t)(reinterpret_cast<uintptr_t>(row + x0) & 15u)) & 15u) >> 2);
  const int head = min(x1 - x0, lead);
  for (int i = threadIdx.x; i < head; i += nt) f(x0 + i, row[x0 + i]);
  const int b0 = x0 + head;
  const float4* body = reinterpret_cast<const float4*>(row + b0);
  const int nb = (x1 - b0) >> 2;
  for (int base = threadIdx.x; base < nb; base += nt * kUnroll) {
    float4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = body[min(base + u * nt, nb - 1)];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = base + u * nt;
      if (i < nb) {
        const int x = b0 + 4 * i;
        f(x, v[u].x);
        f(x + 1, v[u].y);
        f(x + 2, v[u].z);
        f(x + 3, v[u].w);
      }
    }
  }
  for (int x = b0 + 4 * nb + threadIdx.x; x < x1; x += nt) f(x, row[x]);
}

__device__ __forceinline__ const float* row_ptr(const float* p, const float* q, int64_t ps, int64_t qs, int K,
                                                int V, int r) {
  const int nrows = 2 * K + 1;
  const int e = r / nrows, rr = r % nrows;
  return rr <= K ? p + (int64_t)e * ps + (int64_t)rr * V : q + (int64_t)e * qs + (int64_t)(rr - K - 1) * V;
}

template <typename T>
__device__ T wg_sum(T v, T* lds /* blockDim/64 entries */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int off = 32; off > 0; off >>= 1) {
    if constexpr (sizeof(T) == 8) {
      const uint32_t lo = __shfl_xor((uint32_t)v, off), hi = __shfl_xor((uint32_t)((u64)v >> 32), off);
      v += (T)(((u64)hi << 32) | lo);
    } else {
      v += __shfl_xor(v, off);
    }
  }
  __syncthreads();
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  T t = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += lds[w];
  return t;
}

// A thread's run of consecutive elements in one histogram bin, added to the
// workgroup's LDS histogram in one atomic per run: rows whose keys crowd one
// bin (e.g. every zero probability) would otherwise serialise 64 lanes on one
// LDS address for every element.
struct BinRun {
  int bin = -1;
  uint32_t cnt = 0;
  u64 mass = 0;
  __device__ __forceinline__ void flush(uint32_t* c, u64* m) {
    if (cnt) {
      atomicAdd(&c[bin], cnt);
      if (mass) atomicAdd(&m[bin], mass);
    }
    cnt = 0;
    mass = 0;
  }
  __device__ __forceinline__ void add(int b, u64 w, uint32_t* c, u64* m) {
    if (b != bin) {
      flush(c, m);
      bin = b;
    }
    ++cnt;
    mass += w;
  }
};

__global__ __launch_bounds__(kCT) void rows_stats_kernel(const float* __restrict__ p, const float* __restrict__ q,
                                                         int64_t ps, int64_t qs, int K, int V, int C, float t_scale,
                                                         float2* __restrict__ stats, RowState* __restrict__ st,
                                                         uint32_t* __restrict__ hcnt, u64* __restrict__ hmass) {
  __shared__ float red[kCT / 64];
  const int c = blockIdx.x % C, r = blockIdx.x / C;
  // The clear of the row's level-0 histogram and select state, shared by the
  // row's C workgroups (the histogram kernel that follows adds into them).
  for (int b = c * kCT + threadIdx.x; b < kBins; b += C * kCT) {
    hcnt[(int64_t)r * kBins + b] = 0u;
    hmass[(int64_t)r * kBins + b] = 0ull;
  }
  if (c == 0 && threadIdx.x == 0) st[r] = RowState{};
  const float* src = row_ptr(p, q, ps, qs, K, V, r);
  const int x0 = c * kChunk, x1 = min(V, x0 + kChunk);
  float mx = -INFINITY, sm = 0.f;
  for_range(src, x0, x1, [&](int, float v) {
    const float a = scaled_logit(v, t_scale);
    if (a > mx) {
      sm = sm * exp2f(mx - a) + 1.f;
      mx = a;
    } else if (a > -INFINITY) {
      sm += exp2f(a - mx);
    }
  });
  const float cmx = block_reduce_max(mx, red);
  const float part = (mx == -INFINITY) ? 0.f : sm * exp2f(mx - cmx);
  const float csum = block_reduce_sum(part, red);
  if (threadIdx.x == 0) stats[(int64_t)r * C + c] = make_float2(cmx, csum);
}

// The softmax normaliser of row r from its chunk statistics: the row's largest
// scaled logit and 1 / (sum of exp2(a - largest)). Thread i takes chunks i,
// i + kCT, ..., then a fixed reduction tree, so every workgroup of the row gets
// the same values.
static_assert(VQ_MAX_VOCAB / kChunk <= kCT, "a row's chunk statistics fit one per thread");
__device__ __forceinline__ void row_normaliser(const float2* __restrict__ stats, int r, int C, float* redf,
                                               float& gmx, float& inv) {
  // One chunk per thread (C <= kCT), loaded once for both reductions.
  const int i = threadIdx.x;
  const float2 ld = stats[(int64_t)r * C + min(i, C - 1)];
  const float2 s2 = i < C ? ld : make_float2(-INFINITY, 0.f);
  gmx = block_reduce_max(s2.x, redf);
  const float part = (s2.x == -INFINITY) ? 0.f : s2.y * exp2f(s2.x - gmx);
  inv = 1.f / block_reduce_sum(part, redf);
}

__global__ __launch_bounds__(kCT) void rows_hist_kernel(
    const float* __restrict__ p, const float* __restrict__ q, int input_kind, int64_t ps, int64_t qs, int K, int V,
    int C, float t_scale, int use_hist, float* __restrict__ probs, const float2* __restrict__ stats,
    RowState* __restrict__ st, uint32_t* __restrict__ hcnt, u64* __restrict__ hmass) {
  __shared__ uint32_t cnt[kBins];
  __shared__ u64 mas[kBins];
  __shared__ u64 red64[kCT / 64];
  __shared__ float redf[kCT / 64];
  __shared__ int s_bad;
  const int c = blockIdx.x % C, r = blockIdx.x / C;
  const int tid = threadIdx.x;
  const int x0 = c * kChunk, x1 = min(V, x0 + kChunk);
  const float* src = row_ptr(p, q, ps, qs, K, V, r);
  float* dst = probs + (int64_t)r * V;
  if (tid == 0) s_bad = 0;
  float gmx = 0.f, inv = 0.f;
  if (input_kind == 1) row_normaliser(stats, r, C, redf, gmx, inv);
  if (use_hist) {
    for (int b = tid; b < kBins; b += kCT) {
      cnt[b] = 0u;
      mas[b] = 0ull;
    }
  }
  __syncthreads();
  u64 msum = 0;
  int bad = 0;
  BinRun run;
  auto visit = [&](int x, float pv) {
    if (!prob_ok(pv)) {
      bad = 1;
      return;
    }
    const u64 m = mass_of(pv);
    msum += m;
    if (use_hist) run.add((int)(key_of(pv, x, V) >> kTopShift), m, cnt, mas);
  };
  if (input_kind == 1) {
    for_range(src, x0, x1, [&](int x, float v) {
      const float pv = exp2f(scaled_logit(v, t_scale) - gmx) * inv;
      dst[x] = pv;
      visit(x, pv);
    });
  } else {
    for_range(src, x0, x1, visit);
  }
  if (use_hist) run.flush(cnt, mas);
  if (bad) s_bad = 1;
  const u64 tot = wg_sum<u64>(msum, red64);  // barriers inside
  if (tid == 0) {
    if (s_bad) atomicOr(&st[r].bad, 1u);
    if (tot) atomicAdd(&st[r].total, tot);
  }
  if (use_hist) {
    for (int b = tid; b < kBins; b += kCT) {
      if (cnt[b]) atomicAdd(&hcnt[(int64_t)r * kBins + b], cnt[b]);
      if (mas[b]) atomicAdd(&hmass[(int64_t)r * kBins + b], mas[b]);
    }
  }
}

// Walks a 4096-bin histogram from the top bin down (bins > `below` only when
// below >= 0): the bin where the running weight (count or mass) first reaches
// thr, its count, and the weight and mass of the bins above it; also the weight
// of every bin considered. bin = -1 if thr is not reached.
struct Crossing {
  int bin;
  uint32_t count;
  u64 above;
  u64 above_mass;
  u64 total;
};

__device__ Crossing find_bin(const uint32_t* hc, const u64* hm, bool by_mass, u64 thr, int below, u64* scan,
                             Crossing* out) {
  const int tid = threadIdx.x;  // 1024 threads, 4 bins each, descending
  u64 w[4], m[4];
  uint32_t cc[4];
  u64 lsum = 0, lmass = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = kBins - 1 - (4 * tid + i);
    const bool in = b > below;
    cc[i] = in ? hc[b] : 0u;
    m[i] = in ? hm[b] : 0ull;
    w[i] = by_mass ? m[i] : (u64)cc[i];
    lsum += w[i];
    lmass += m[i];
  }
  u64 tot, totm;
  const u64 excl = block_excl_scan<u64, kRowThreads>(lsum, scan, tot);
  const u64 exclm = block_excl_scan<u64, kRowThreads>(lmass, scan, totm);
  if (tid == 0) *out = Crossing{-1, 0u, 0ull, 0ull, tot};
  __syncthreads();
  if (excl < thr && thr <= excl + lsum) {
    u64 run = excl, runm = exclm;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (run + w[i] >= thr) {
        *out = Crossing{kBins - 1 - (4 * tid + i), cc[i], run, runm, tot};
        break;
      }
      run += w[i];
      runm += m[i];
    }
  }
  __syncthreads();
  const Crossing res = *out;
  __syncthreads();
  return res;
}

// Zeroes one row's histogram of a level (all threads of the workgroup).
__device__ __forceinline__ void clear_hist(uint32_t* hc, u64* hm) {
  for (int b = threadIdx.x; b < kBins; b += blockDim.x) {
    hc[b] = 0u;
    hm[b] = 0ull;
  }
}

__global__ __launch_bounds__(kRowThreads) void rows_find_kernel(int V, int top_k, uint32_t tp,
                                                                RowState* __restrict__ st,
                                                                uint32_t* __restrict__ hcnt, u64* __restrict__ hmass,
                                                                int64_t lvl_stride, RowMeta* __restrict__ meta) {
  __shared__ u64 scan[kRowThreads / 64 + 1];
  __shared__ Crossing cr;
  const int r = blockIdx.x;
  const RowState s0 = st[r];
  const bool use_k = top_k > 0 && top_k < V;
  const bool use_p = tp < (1u << 24);
  RowMeta out{};
  if (s0.bad || (!use_k && !use_p)) {
    out.z = s0.bad ? 0ull : s0.total;
    out.status = (s0.bad || s0.total == 0) ? 1 : 0;
    __syncthreads();
    if (threadIdx.x == 0) meta[r] = out;
    return;
  }
  u64 thr = (u64)top_k;
  if (!use_k) thr = (u64)(((u128)tp * s0.total + ((u128)1 << 24) - 1) >> 24);
  const Crossing c = find_bin(hcnt + (int64_t)r * kBins, hmass + (int64_t)r * kBins, !use_k, thr, -1, scan, &cr);
  if (thr == 0 || c.bin < 0) {  // nothing to keep
    out.status = 1;
    if (threadIdx.x == 0) meta[r] = out;
    return;
  }
  const bool crowded = c.count > (uint32_t)kCandCap;
  if (crowded)
    clear_hist(hcnt + lvl_stride + (int64_t)r * kBins, hmass + lvl_stride + (int64_t)r * kBins);
  if (threadIdx.x == 0) {
    RowState s = s0;
    s.prefix = (u64)c.bin;
    s.shift = kTopShift;
    s.above = c.above;
    s.above_mass = c.above_mass;
    s.thr = thr;
    s.cand_n = 0;
    s.phase = use_k ? 0 : 1;
    s.levels = 1;
    s.kbin[0] = c.bin;
    s.pending = crowded ? 0 : 1;
    s.refine = crowded ? 1 : 0;
    st[r] = s;
  }
}

// One more histogram level over a crowded region, spread over the chip like
// rows_hist: per (chunk, row) the next 12 key bits of the region's keys, merged
// into the row's level histogram with global atomics. Rows with nothing to
// refine at this level return at once.
__global__ __launch_bounds__(kCT) void rows_refine_hist_kernel(
    const float* __restrict__ p, const float* __restrict__ q, int input_kind, int64_t ps, int64_t qs, int K, int V,
    int C, const float* __restrict__ probs, const RowState* __restrict__ st, uint32_t* __restrict__ hcnt,
    u64* __restrict__ hmass, int64_t lvl_stride, int level) {
  __shared__ uint32_t cnt[kBins];
  __shared__ u64 mas[kBins];
  const int c = blockIdx.x % C, r = blockIdx.x / C;
  if (st[r].refine != level) return;
  const u64 prefix = st[r].prefix;
  const int shift = st[r].shift;
  const int sub = shift - kDigitBits;
  const float* row = input_kind == 1 ? probs + (int64_t)r * V : row_ptr(p, q, ps, qs, K, V, r);
  const int x0 = c * kChunk, x1 = min(V, x0 + kChunk);
  for (int b = threadIdx.x; b < kBins; b += kCT) {
    cnt[b] = 0u;
    mas[b] = 0ull;
  }
  __syncthreads();
  BinRun run;
  for_range(row, x0, x1, [&](int x, float v) {
    const u64 key = key_of(v, x, V);
    if ((key >> shift) != prefix) return;
    run.add((int)((key >> sub) & (u64)(kBins - 1)), mass_of(v), cnt, mas);
  });
  run.flush(cnt, mas);
  __syncthreads();
  uint32_t* hc = hcnt + (int64_t)level * lvl_stride + (int64_t)r * kBins;
  u64* hm = hmass + (int64_t)level * lvl_stride + (int64_t)r * kBins;
  for (int b = threadIdx.x; b < kBins; b += kCT) {
    if (cnt[b]) atomicAdd(&hc[b], cnt[b]);
    if (mas[b]) atomicAdd(&hm[b], mas[b]);
  }
}

// The crossing bin of a refined region (one workgroup per row at this level):
// the region narrows by 12 bits; gathered next if it holds at most kCandCap
// keys, else refined once more.
__global__ __launch_bounds__(kRowThreads) void rows_refine_find_kernel(RowState* __restrict__ st,
                                                                       uint32_t* __restrict__ hcnt,
                                                                       u64* __restrict__ hmass, int64_t lvl_stride,
                                                                       int level, RowMeta* __restrict__ meta) {
  __shared__ u64 scan[kRowThreads / 64 + 1];
  __shared__ Crossing cr;
  const int r = blockIdx.x;
  const RowState s0 = st[r];
  if (s0.refine != level) return;
  const Crossing c = find_bin(hcnt + (int64_t)level * lvl_stride + (int64_t)r * kBins,
                              hmass + (int64_t)level * lvl_stride + (int64_t)r * kBins, s0.phase == 1,
                              s0.thr - s0.above, -1, scan, &cr);
  // The region's keys weigh at least thr - above, so a crossing exists; a
  // region at the last level holds at most 2^14 <= kCandCap keys.
  const bool crowded = c.bin >= 0 && c.count > (uint32_t)kCandCap;
  if (crowded && level + 1 < kLevels)
    clear_hist(hcnt + (int64_t)(level + 1) * lvl_stride + (int64_t)r * kBins,
               hmass + (int64_t)(level + 1) * lvl_stride + (int64_t)r * kBins);
  if (threadIdx.x == 0) {
    RowState s = s0;
    if (c.bin < 0 || (crowded && level + 1 >= kLevels)) {  // not reached
      s.refine = 0;
      s.pending = 0;
      meta[r] = RowMeta{0ull, 0ull, 1, {0, 0, 0}};
      st[r] = s;
      return;
    }
    s.prefix = (s0.prefix << kDigitBits) | (u64)c.bin;
    s.shift = s0.shift - kDigitBits;
    s.above = s0.above + c.above;
    s.above_mass = s0.above_mass + c.above_mass;
    if (s0.phase == 0) {
      s.kbin[level] = c.bin;
      s.levels = level + 1;
    }
    s.refine = crowded ? level + 1 : 0;
    s.pending = crowded ? 0 : 1;
    st[r] = s;
  }
}

__global__ __launch_bounds__(kCT) void rows_compact_kernel(const float* __restrict__ p, const float* __restrict__ q,
                                                           int input_kind, int64_t ps, int64_t qs, int K, int V,
                                                           int C, const float* __restrict__ probs,
                                                           RowState* __restrict__ st, u64* __restrict__ cand) {
  __shared__ u64 keys[kStage];
  __shared__ uint32_t n_lds, base;
  const int c = blockIdx.x % C, r = blockIdx.x / C;
  if (!st[r].pending) return;
  const u64 prefix = st[r].prefix;
  const int shift = st[r].shift;
  const float* row = input_kind == 1 ? probs + (int64_t)r * V : row_ptr(p, q, ps, qs, K, V, r);
  const int x0 = c * kChunk, x1 = min(V, x0 + kChunk);
  // The chunk's keys of the region, kStage elements at a time, staged in LDS:
  // one LDS atomic per wave and element position (ballot of the matching
  // lanes), then one reservation in the row's gather buffer and a coalesced copy.
  const uint32_t lane = threadIdx.x & 63;
  for (int s0 = x0; s0 < x1; s0 += kStage) {
    if (threadIdx.x == 0) n_lds = 0u;
    __syncthreads();
    for_range(row, s0, min(x1, s0 + kStage), [&](int x, float v) {
      const u64 key = key_of(v, x, V);
      const bool hit = (key >> shift) == prefix;
      const u64 m = __ballot(hit);
      if (!m) return;
      const int lead = __ffsll((long long)m) - 1;
      uint32_t off = 0;
      if ((int)lane == lead) off = atomicAdd(&n_lds, (uint32_t)__popcll(m));
      off = __shfl(off, lead);
      if (hit) keys[off + __popcll(m & ((1ull << lane) - 1ull))] = key;
    });
    __syncthreads();
    const uint32_t n = n_lds;
    if (n) {
      if (threadIdx.x == 0) base = atomicAdd(&st[r].cand_n, n);
      __syncthreads();
      u64* dst = cand + (int64_t)r * kCandCap + base;
      for (uint32_t i = threadIdx.x; i < n; i += kCT) dst[i] = keys[i];
    }
    __syncthreads();  // keys and n_lds are reused by the next pass
  }
}

__device__ __forceinline__ float key_value(u64 key) { return __uint_as_float((uint32_t)(key >> 20)); }

// Radix select over gathered keys of one region ((key >> hi_shift) == prefix):
// the first key, walking down from the largest, at which the running weight
// (count or mass; only keys >= lo count) reaches thr, given the weight `above`
// of everything above the region. 8-bit digits from hi_shift down (the last
// one narrower); a level whose crossing digit holds one key ends the walk.
struct Sel {
  u64 key;
  u64 mass;
  u64 above;
};

__device__ Sel select_keys(const u64* __restrict__ keys, int n, u64 prefix, int hi_shift, u64 above, u64 thr,
                           bool by_mass, u64 lo, uint32_t* cnt, u64* mas, u64* scan, Sel* res, int* flag) {
  const int tid = threadIdx.x;
  for (;;) {
    const int bits = min(kCandBits, hi_shift);
    const int shift = hi_shift - bits;
    const int nb = 1 << bits;
    for (int b = tid; b < nb; b += kRowThreads) {
      cnt[b] = 0u;
      mas[b] = 0ull;
    }
    __syncthreads();
    for (int i = tid; i < n; i += kRowThreads) {
      const u64 key = keys[i];
      if (key < lo || (key >> hi_shift) != prefix) continue;
      const int d = (int)((key >> shift) & (u64)(nb - 1));
      atomicAdd(&cnt[d], 1u);
      if (by_mass) {
        const u64 m = mass_of(key_value(key));
        if (m) atomicAdd(&mas[d], m);
      }
    }
    __syncthreads();
    // Thread t < nb owns digit nb-1-t (descending).
    const int d = nb - 1 - tid;
    const uint32_t cd = (tid < nb) ? cnt[d] : 0u;
    const u64 wd = (tid < nb) ? (by_mass ? mas[d] : (u64)cd) : 0ull;
    u64 tot;
    const u64 excl = above + block_excl_scan<u64, kRowThreads>(wd, scan, tot);
    if (tid == 0) *flag = 0;
    __syncthreads();
    if (tid < nb && excl < thr && thr <= excl + wd) {
      *res = Sel{(prefix << bits) | (u64)d, cd, excl};  // mass field carries the digit's count here
      *flag = 1;
    }
    __syncthreads();
    const Sel s = *res;
    __syncthreads();
    prefix = s.key;
    above = s.above;
    hi_shift = shift;
    if (s.mass == 1 || shift == 0) {
      // One key left in the crossing digit: it is the answer.
      for (int i = tid; i < n; i += kRowThreads) {
        const u64 key = keys[i];
        if (key >= lo && (key >> hi_shift) == prefix) *res = Sel{key, mass_of(key_value(key)), above};
      }
      __syncthreads();
      const Sel out = *res;
      __syncthreads();
      return out;
    }
  }
}

__global__ __launch_bounds__(kRowThreads) void rows_resolve_kernel(int V, int top_k, uint32_t tp,
                                                                   RowState* __restrict__ st,
                                                                   uint32_t* __restrict__ hcnt,
                                                                   u64* __restrict__ hmass, int64_t lvl_stride,
                                                                   const u64* __restrict__ cand,
                                                                   RowMeta* __restrict__ meta) {
  __shared__ uint32_t cnt[1 << kCandBits];
  __shared__ u64 mas[1 << kCandBits];
  __shared__ u64 scan[kRowThreads / 64 + 1];
  __shared__ u64 red64[kRowThreads / 64];
  __shared__ Sel res;
  __shared__ Crossing cr;
  __shared__ int flag;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const RowState s0 = st[r];
  if (!s0.pending) return;
  __syncthreads();
  const u64* keys = cand + (int64_t)r * kCandCap;
  const int n = (int)s0.cand_n;
  const bool use_p = tp < (1u << 24);
  RowMeta out{};
  if (s0.phase == 1) {
    const Sel sel = select_keys(keys, n, s0.prefix, s0.shift, s0.above, s0.thr, true, 0ull, cnt, mas, scan, &res,
                                &flag);
    out.thresh = sel.key;
    out.z = sel.above + sel.mass;
    out.status = out.z == 0 ? 1 : 0;
    if (tid == 0) {
      meta[r] = out;
      st[r].pending = 0;
    }
    return;
  }
  // Top-k: the top_k-th key, then the kept mass Z_k (everything above the region
  // + the region's keys >= it).
  const Sel sk = select_keys(keys, n, s0.prefix, s0.shift, s0.above, s0.thr, false, 0ull, cnt, mas, scan, &res,
                             &flag);
  const u64 theta = sk.key;
  u64 m_in = 0;
  for (int i = tid; i < n; i += kRowThreads)
    if (keys[i] >= theta) m_in += mass_of(key_value(keys[i]));
  const u64 zk = s0.above_mass + wg_sum<u64>(m_in, red64);
  if (!use_p || zk == 0) {
    out.thresh = theta;
    out.z = zk;
    out.status = zk == 0 ? 1 : 0;
    if (tid == 0) {
      meta[r] = out;
      st[r].pending = 0;
    }
    return;
  }
  // Top-p over the kept set: walking down from the largest key, the mass-weighted
  // select with thr = ceil(tp * Z_k / 2^24) <= Z_k crosses at a key >= theta, so it
  // is the walk over the whole row. At each level of the top-k path, the bins
  // above its crossing bin come first.
  const u64 thr = (u64)(((u128)tp * zk + ((u128)1 << 24) - 1) >> 24);
  u64 run = 0, pre = 0;
  for (int L = 0; L < s0.levels; ++L) {
    const Crossing c = find_bin(hcnt + (int64_t)L * lvl_stride + (int64_t)r * kBins,
                                hmass + (int64_t)L * lvl_stride + (int64_t)r * kBins, true, thr - run, s0.kbin[L],
                                scan, &cr);
    if (c.bin >= 0) {
      // The walk crosses in a bin above the top-k path at this level (all of its
      // keys are kept by top-k, so it holds fewer than top_k keys): gather it next.
      if (tid == 0) {
        RowState s = s0;
        s.prefix = (pre << kDigitBits) | (u64)c.bin;
        s.shift = kTopShift - kDigitBits * L;
        s.above = run + c.above;
        s.thr = thr;
        s.cand_n = 0;
        if (c.count > (uint32_t)kCandCap) {
          s.phase = 3;
          s.pending = 0;
        } else {
          s.phase = 1;
          s.pending = 1;
        }
        st[r] = s;
      }
      return;
    }
    run += c.total;
    pre = (pre << kDigitBits) | (u64)s0.kbin[L];
  }
  // It crosses among the gathered keys kept by top-k.
  const Sel sp = select_keys(keys, n, s0.prefix, s0.shift, run, thr, true, theta, cnt, mas, scan, &res, &flag);
  out.thresh = sp.key;
  out.z = sp.above + sp.mass;
  out.status = out.z == 0 ? 1 : 0;
  if (tid == 0) {
    meta[r] = out;
    st[r].pending = 0;
  }
}

// ------------------------------------------- small top-k: per-chunk candidates
// For top_k <= kTopKMax, the row's top_k keys are among the union of the chunks'
// own top_k keys: a key that top_k keys of its own chunk outrank is outranked by
// top_k keys of the row. One workgroup per (chunk, row) selects its chunk's
// top_k keys into fixed slots of the row's gather buffer; one workgroup per row
// then selects the row's top_k keys from those slots and runs the top-p walk
// over them. Two launches replace the histogram levels, the compacts and the
// resolves, and a crowd of keys that agree in their high bits (every zero
// probability of a near one-hot row) costs one select level, not three
// chip-wide passes.
constexpr int kTopKMax = 64;
constexpr u64 kNoKey = ~0ull;  // an empty slot: above every 50-bit key, so in no region
constexpr int kSelJ = 16;      // keys per thread in the selects: 16 * kCT = kChunk, 16 * 1024 = kCandCap
constexpr int kFewKeys = 256;  // at most this many merge candidates are ranked directly
static_assert(kSelJ * kCT == kChunk && kSelJ * kRowThreads == kCandCap, "select capacities");
static_assert(kTopKMax <= 64, "the top-p walk over the kept keys takes one lane each");
static_assert((int64_t)kTopKMax * ((VQ_MAX_VOCAB + kChunk - 1) / kChunk) <= kCandCap,
              "every chunk's candidates fit one row's gather buffer");

struct TopRes {
  uint32_t digit, excl, cnt;
};

struct TopLds {
  uint32_t hist[256];
  u64 r_or[kRowThreads / 64];
  u64 r_and[kRowThreads / 64];
  uint32_t wsum[4];
  TopRes res[2];  // by level parity, so that a level needs no barrier before it writes its own
};

__device__ __forceinline__ u64 shfl_xor_u64(u64 v, int off) {
  const uint32_t lo = __shfl_xor((uint32_t)v, off), hi = __shfl_xor((uint32_t)(v >> 32), off);
  return ((u64)hi << 32) | lo;
}

__device__ __forceinline__ u64 shfl_u64(u64 v, int src_lane) {
  const uint32_t lo = __shfl((uint32_t)v, src_lane), hi = __shfl((uint32_t)(v >> 32), src_lane);
  return ((u64)hi << 32) | lo;
}

// A workgroup barrier that orders LDS accesses only: global stores still in
// flight (the probabilities the chunk pass writes) are not waited for.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Among the keys held kSelJ per thread in slots j < nj (kNoKey: empty), the
// bound T with exactly `need` keys >= T, for 1 <= need < number of keys. Radix
// select from the top over the keys still in the running (one bit per slot):
// each level takes the highest bit in which those keys differ (from their
// bitwise OR and AND), counts the digit of up to 8 bits from there down, and
// keeps the keys of the digit where the count from the top reaches `need`.
// Bits that every remaining key shares cost nothing, so a crowd of equal
// probabilities takes one level; keys are distinct, so the walk ends at a digit
// that holds exactly the keys still needed.
template <int NT>
__device__ u64 select_top(const u64 (&key)[kSelJ], int nj, uint32_t need, TopLds& s) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t alive = 0u;
#pragma unroll
  for (int j = 0; j < kSelJ; ++j)
    if (j < nj && key[j] != kNoKey) alive |= 1u << j;
  // Each level lowers the highest bit in which the remaining keys differ, and
  // keys are below 2^50: at most 50 levels.
  for (int level = 0; level < 64; ++level) {
    TopRes& res = s.res[level & 1];
    u64 o = 0ull, a = ~0ull;
#pragma unroll
    for (int j = 0; j < kSelJ; ++j) {
      if (j < nj && ((alive >> j) & 1u)) {
        o |= key[j];
        a &= key[j];
      }
    }
    // Over the wave, each 32-bit half on its own (the operations are bitwise).
    o = ((u64)or64_lanes((uint32_t)(o >> 32)) << 32) | or64_lanes((uint32_t)o);
    a = ((u64)and64_lanes((uint32_t)(a >> 32)) << 32) | and64_lanes((uint32_t)a);
    if (lane == 0) {
      s.r_or[wave] = o;
      s.r_and[wave] = a;
    }
    for (int b = tid; b < 256; b += NT) s.hist[b] = 0u;
    if (tid == 0) res = TopRes{0u, 0u, need};  // stands only if no digit crosses (never for distinct keys)
    lds_barrier();
    o = 0ull;
    a = ~0ull;
    for (int w = 0; w < NT / 64; ++w) {
      o |= s.r_or[w];
      a &= s.r_and[w];
    }
    if (o < a) return 0ull;  // no key left (not reached)
    const u64 diff = o ^ a;
    if (diff == 0ull) return a;  // one key left (not reached for need < count)
    const int h = 63 - __clzll((long long)diff);
    const int lo = h >= 7 ? h - 7 : 0;
    const uint32_t dmask = (2u << (h - lo)) - 1u;
    // Counts of the digit: a thread's run of keys in one digit is one LDS atomic
    // (a crowd that shares a digit would serialise on one address).
    uint32_t run_d = 0u, run_c = 0u;
#pragma unroll
    for (int j = 0; j < kSelJ; ++j) {
      if (j < nj && ((alive >> j) & 1u)) {
        const uint32_t d = (uint32_t)(key[j] >> lo) & dmask;
        if (run_c && d != run_d) {
          atomicAdd(&s.hist[run_d], run_c);
          run_c = 0u;
        }
        run_d = d;
        ++run_c;
      }
    }
    if (run_c) atomicAdd(&s.hist[run_d], run_c);
    lds_barrier();
    // Thread t <= dmask owns digit dmask - t (descending): a scan over the first
    // four waves (at most 256 digits).
    const int d = (int)dmask - tid;
    const uint32_t c = d >= 0 ? s.hist[d] : 0u;
    uint32_t inc = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o2 = __shfl_up(inc, off);
      if (lane >= off) inc += o2;
    }
    if (lane == 63 && wave < 4) s.wsum[wave] = inc;
    lds_barrier();
    uint32_t excl = inc - c;
    for (int w2 = 0; w2 < wave && w2 < 4; ++w2) excl += s.wsum[w2];
    if (d >= 0 && excl < need && need <= excl + c) res = TopRes{(uint32_t)d, excl, c};
    lds_barrier();
    const TopRes got = res;
    need -= got.excl;
    if (got.cnt == need) return ((a >> (h + 1)) << (h + 1)) | ((u64)got.digit << lo);
#pragma unroll
    for (int j = 0; j < kSelJ; ++j)
      if (j < nj && ((alive >> j) & 1u) && ((uint32_t)(key[j] >> lo) & dmask) != got.digit) alive &= ~(1u << j);
  }
  return 0ull;  // not reached
}

// Per (chunk, row): the probabilities (logits mode: written to probs), their
// validity, the chunk's top min(top_k, length) keys in slots [0, top_k) of
// cand[row * kCandCap + chunk * top_k] (kNoKey in the rest), and a bound T with
// exactly min(top_k, length) of the chunk's keys >= T (0 if it keeps them all).
__global__ __launch_bounds__(kCT) void rows_chunk_topk_kernel(
    const float* __restrict__ p, const float* __restrict__ q, int input_kind, int64_t ps, int64_t qs, int K, int V,
    int C, float t_scale, float* __restrict__ probs, const float2* __restrict__ stats, int top_k,
    u64* __restrict__ cand, uint32_t* __restrict__ badf, u64* __restrict__ bound) {
  __shared__ u64 keys[kChunk];
  __shared__ TopLds s;
  __shared__ float redf[kCT / 64];
  __shared__ uint32_t n_out, s_bad;
  const int c = blockIdx.x % C, r = blockIdx.x / C;
  const int tid = threadIdx.x;
  const int x0 = c * kChunk, x1 = min(V, x0 + kChunk), n = x1 - x0;
  const float* src = row_ptr(p, q, ps, qs, K, V, r);
  float* dst = probs + (int64_t)r * V;
  float gmx = 0.f, inv = 0.f;
  if (input_kind == 1) row_normaliser(stats, r, C, redf, gmx, inv);
  if (tid == 0) {
    n_out = 0u;
    s_bad = 0u;
  }
  lds_barrier();
  uint32_t bad = 0u;
  auto visit = [&](int x, float pv) {
    const bool ok = prob_ok(pv);
    bad |= ok ? 0u : 1u;
    // An invalid probability marks the row invalid; its key keeps only the id
    // part, so the keys stay distinct and below 2^50 whatever the input.
    keys[x - x0] = key_of(ok ? pv : 0.f, x, V);
  };
  if (input_kind == 1) {
    for_range(src, x0, x1, [&](int x, float v) {
      const float pv = exp2f(scaled_logit(v, t_scale) - gmx) * inv;
      dst[x] = pv;
      visit(x, pv);
    });
  } else {
    for_range(src, x0, x1, visit);
  }
  if (bad) atomicOr(&s_bad, 1u);
  lds_barrier();  // keys and s_bad complete; the probability stores drain meanwhile
  const uint32_t any_bad = s_bad;
  u64 kr[kSelJ];
#pragma unroll
  for (int j = 0; j < kSelJ; ++j) {
    const int i = j * kCT + tid;
    kr[j] = i < n ? keys[i] : kNoKey;
  }
  const uint32_t kk = (uint32_t)min(top_k, n);
  const u64 T = kk < (uint32_t)n ? select_top<kCT>(kr, kSelJ, kk, s) : 0ull;
  u64* out = cand + (int64_t)r * kCandCap + (int64_t)c * top_k;
#pragma unroll
  for (int j = 0; j < kSelJ; ++j) {
    if (kr[j] != kNoKey && kr[j] >= T) {
      const uint32_t slot = atomicAdd(&n_out, 1u);  // < kk: exactly kk keys are >= T
      if (slot < kk) out[slot] = kr[j];
    }
  }
  for (int i = (int)kk + tid; i < top_k; i += kCT) out[i] = kNoKey;
  if (tid == 0) {
    badf[(int64_t)r * C + c] = any_bad ? 1u : 0u;
    bound[(int64_t)r * C + c] = T;
  }
}

// Per row: the top_k keys of the row from the chunks' candidates, their mass
// Z_k, then top-p over them in descending order: the first key whose running
// mass reaches ceil(tp * Z_k / 2^24). The largest chunk bound L is a lower bound
// of the row's top_k-th key (its chunk holds top_k keys >= L), so candidates
// below L are dropped before the select (for a near one-hot row, every chunk's
// run of zero probabilities but the first).
__global__ __launch_bounds__(kRowThreads) void rows_topk_merge_kernel(int C, int top_k, uint32_t tp,
                                                                      const u64* __restrict__ cand,
                                                                      const uint32_t* __restrict__ badf,
                                                                      const u64* __restrict__ bound,
                                                                      RowMeta* __restrict__ meta) {
  __shared__ TopLds s;
  __shared__ u64 kept[kTopKMax];
  __shared__ u64 sorted[kTopKMax];
  __shared__ u64 few[kFewKeys];
  __shared__ u64 red[kRowThreads / 64];
  __shared__ uint32_t n_kept;
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int bad = 0;
  u64 lb = 0ull;
  for (int i = tid; i < C; i += kRowThreads) {
    bad |= badf[(int64_t)r * C + i] != 0u;
    lb = max(lb, bound[(int64_t)r * C + i]);
  }
  for (int off = 32; off > 0; off >>= 1) lb = max(lb, shfl_xor_u64(lb, off));
  if (lane == 0) red[wave] = lb;
  if (tid == 0) n_kept = 0u;
  if (__syncthreads_or(bad)) {
    if (tid == 0) meta[r] = RowMeta{0ull, 0ull, 1, {0, 0, 0}};
    return;
  }
  u64 L = 0ull;
  for (int w = 0; w < kRowThreads / 64; ++w) L = max(L, red[w]);
  const int n = C * top_k;
  const int nj = (n + kRowThreads - 1) / kRowThreads;  // slots in use per thread
  u64 kr[kSelJ];
  uint32_t live = 0u;
#pragma unroll
  for (int j = 0; j < kSelJ; ++j) {
    const int i = j * kRowThreads + tid;
    const u64 k = i < n ? cand[(int64_t)r * kCandCap + i] : kNoKey;
    kr[j] = (k != kNoKey && k >= L) ? k : kNoKey;  // only keys >= L can be kept
    live += kr[j] != kNoKey;
  }
  const uint32_t m = wg_sum<uint32_t>(live, reinterpret_cast<uint32_t*>(red));  // >= top_k
  int kc;
  if (m <= (uint32_t)kFewKeys) {
    // Few candidates (the usual case): a key's rank among them is its place
    // in descending order (keys are distinct), so the top_k come out sorted
    // without the digit-by-digit select.
#pragma unroll
    for (int j = 0; j < kSelJ; ++j) {
      if (j < nj && kr[j] != kNoKey) few[atomicAdd(&n_kept, 1u)] = kr[j];  // slots < m
    }
    __syncthreads();
    if (tid < (int)m) {
      const u64 mine = few[tid];
      uint32_t rank = 0;
      for (uint32_t i = 0; i < m; ++i) rank += few[i] > mine;
      if (rank < (uint32_t)top_k) sorted[rank] = mine;
    }
    kc = (int)min(m, (uint32_t)top_k);
  } else {
    const u64 T = select_top<kRowThreads>(kr, nj, (uint32_t)top_k, s);
#pragma unroll
    for (int j = 0; j < kSelJ; ++j) {
      if (j < nj && kr[j] != kNoKey && kr[j] >= T) {
        const uint32_t slot = atomicAdd(&n_kept, 1u);  // < top_k: exactly top_k keys are >= T
        if (slot < (uint32_t)top_k) kept[slot] = kr[j];
      }
    }
    __syncthreads();
    kc = min((int)n_kept, top_k);  // == top_k
    if (tid < kc) {
      const u64 mine = kept[tid];
      int rank = 0;
      for (int i = 0; i < kc; ++i) rank += kept[i] > mine;
      sorted[rank] = mine;
    }
  }
  __syncthreads();
  if (tid >= 64) return;
  if (kc == 0) {  // not reached: top_k >= 1 keys are present
    if (tid == 0) meta[r] = RowMeta{0ull, 0ull, 1, {0, 0, 0}};
    return;
  }
  const u64 key = lane < kc ? sorted[lane] : 0ull;
  const u64 ms = lane < kc ? mass_of(key_value(key)) : 0ull;
  u64 incl = ms;
  for (int off = 1; off < 64; off <<= 1) {
    const u64 o = shfl_up_u64(incl, off);
    if (lane >= off) incl += o;
  }
  const u64 zk = shfl_u64(incl, kc - 1);
  if (tp >= (1u << 24) || zk == 0) {
    // No top-p, or nothing kept: the threshold is the smallest kept key.
    if (lane == kc - 1) meta[r] = RowMeta{key, zk, zk == 0 ? 1 : 0, {0, 0, 0}};
    return;
  }
  const u64 thr = (u64)(((u128)tp * zk + ((u128)1 << 24) - 1) >> 24);  // 1 <= thr <= zk
  if (lane < kc && incl - ms < thr && thr <= incl) meta[r] = RowMeta{key, incl, 0, {0, 0, 0}};
}

// ------------------------------------------------------- chunked draw (entries)
// Per (chunk, entry): the accept tests (every workgroup of the entry repeats
// them: K pairs of loads), then the chunk's sums of the draw weights of the
// first rejected position j — the residual, or the kept target mass when all K
// drafts pass — and of the kept target mass of row j (used only if the
// residual is zero everywhere).
__global__ __launch_bounds__(kCT) void draw_sums_kernel(const float* __restrict__ probs_p,
                                                        const float* __restrict__ probs_q, int64_t pp_stride,
                                                        int64_t qq_stride, const RowMeta* __restrict__ meta,
                                                        int64_t meta_stride, const int32_t* __restrict__ draft,
                                                        const float* __restrict__ uniforms, int K, int V, int C,
                                                        u128* __restrict__ esum) {
  __shared__ u128 scan[kCT / 64 + 1];
  __shared__ int s_j, s_bad;
  const int c = blockIdx.x % C, b = blockIdx.x / C;
  const int tid = threadIdx.x;
  const RowMeta* mrow = meta + (int64_t)b * meta_stride;
  const float* P = probs_p + (int64_t)b * pp_stride;
  const float* Q = probs_q + (int64_t)b * qq_stride;
  if (tid < 64) {
    int bad;
    const int jj = entry_decide(P, Q, mrow, draft + (int64_t)b * K, uniforms + (int64_t)b * (K + 1), K, V, &bad);
    if (tid == 0) {
      s_j = jj;
      s_bad = bad;
    }
  }
  __syncthreads();
  if (s_bad) return;
  const int j = s_j;
  DrawRow d;
  d.P = P + (int64_t)j * V;
  d.mp = mrow[j];
  d.Q = j < K ? Q + (int64_t)j * V : nullptr;
  d.mq = j < K ? mrow[K + 1 + j] : RowMeta{};
  d.V = V;
  const int x0 = c * kChunk, x1 = min(V, x0 + kChunk);
  u128 wm = 0, wf = 0;
  if (d.Q) {
    // P and Q rows side by side: element x of both in the same step.
    const int lead = (int)(((16u - (uint32_t)(reinterpret_cast<uintptr_t>(d.P + x0) & 15u)) & 15u) >> 2);
    const bool qal = ((reinterpret_cast<uintptr_t>(d.Q + x0) ^ reinterpret_cast<uintptr_t>(d.P + x0)) & 15u) == 0;
    const int head = qal ? min(x1 - x0, lead) : x1 - x0;  // unaligned pair: all scalar
    for (int x = x0 + tid; x < x0 + head; x += kCT) {
      const float pv = d.P[x];
      wm += d.w(x, pv, d.Q[x]);
      wf += kept_mass_v(pv, x, V, d.mp);
    }
    const int b0 = x0 + head;
    const int nb = (x1 - b0) >> 2;
    const float4* P4 = reinterpret_cast<const float4*>(d.P + b0);
    const float4* Q4 = reinterpret_cast<const float4*>(d.Q + b0);
    for (int base = tid; base < nb; base += kCT * 4) {
      float4 pv[4], qv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = min(base + u * kCT, nb - 1);
        pv[u] = P4[i];
        qv[u] = Q4[i];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = base + u * kCT;
        if (i < nb) {
          const int x = b0 + 4 * i;
          wm += d.w(x, pv[u].x, qv[u].x) + d.w(x + 1, pv[u].y, qv[u].y) + d.w(x + 2, pv[u].z, qv[u].z) +
                d.w(x + 3, pv[u].w, qv[u].w);
          wf += (u128)(kept_mass_v(pv[u].x, x, V, d.mp) + kept_mass_v(pv[u].y, x + 1, V, d.mp)) +
                (u128)(kept_mass_v(pv[u].z, x + 2, V, d.mp) + kept_mass_v(pv[u].w, x + 3, V, d.mp));
        }
      }
    }
    for (int x = b0 + 4 * nb + tid; x < x1; x += kCT) {
      const float pv = d.P[x];
      wm += d.w(x, pv, d.Q[x]);
      wf += kept_mass_v(pv, x, V, d.mp);
    }
  } else {
    for_range(d.P, x0, x1, [&](int x, float v) { wm += kept_mass_v(v, x, V, d.mp); });
  }
  u128 tm, tf;
  block_excl_scan<u128, kCT>(wm, scan, tm);
  block_excl_scan<u128, kCT>(wf, scan, tf);
  if (tid == 0) {
    esum[((int64_t)b * C + c) * 2] = tm;
    esum[((int64_t)b * C + c) * 2 + 1] = tf;
  }
}

// Per entry: the draw weights' total from the chunk sums (in chunk order), the
// chunk that holds floor(mu * R / 2^24), and the token inside it (each thread
// sums 8 consecutive weights; a block scan finds the thread, which walks them).
__global__ __launch_bounds__(kRowThreads) void draw_pick_kernel(
    const float* __restrict__ probs_p, const float* __restrict__ probs_q, int64_t pp_stride, int64_t qq_stride,
    const RowMeta* __restrict__ meta, int64_t meta_stride, const int32_t* __restrict__ draft,
    const float* __restrict__ uniforms, int K, int V, int C, const u128* __restrict__ esum,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_n) {
  __shared__ u128 scan[kRowThreads / 64 + 1];
  __shared__ int s_j, s_bad, s_tok, s_c;
  __shared__ u128 s_before;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const RowMeta* mrow = meta + (int64_t)b * meta_stride;
  const float* P = probs_p + (int64_t)b * pp_stride;
  const float* Q = probs_q + (int64_t)b * qq_stride;
  const int32_t* dr = draft + (int64_t)b * K;
  const float* us = uniforms + (int64_t)b * (K + 1);
  // Every chunk's two sums go out with the accept tests (V <= 2^20, so C <= 256
  // chunks, one per thread).
  u128 w0 = 0, w1 = 0;
  if (tid < C) {
    w0 = esum[((int64_t)b * C + tid) * 2];
    w1 = esum[((int64_t)b * C + tid) * 2 + 1];
  }
  const float u_draw = us[K];
  if (tid < 64) {
    int bad;
    const int jj = entry_decide(P, Q, mrow, dr, us, K, V, &bad);
    if (tid == 0) {
      s_j = jj;
      s_bad = bad;
      s_tok = -1;
    }
  }
  __syncthreads();
  const int j = s_j;
  if (s_bad) {
    for (int i = tid; i <= K; i += kRowThreads) out_tokens[(int64_t)b * (K + 1) + i] = -1;
    if (tid == 0) out_n[b] = -1;
    return;
  }
  // Totals and chunk-order prefix sums of both weights; if the residual is zero
  // everywhere (p~_j == q~_j and the draft lay outside both supports) the draw
  // is from p~_j. The chunk that holds floor(mu * R / 2^24) is the one whose
  // prefix range contains it.
  u128 R0, R1;
  const u128 e0 = block_excl_scan<u128, kRowThreads>(w0, scan, R0);
  const u128 e1 = block_excl_scan<u128, kRowThreads>(w1, scan, R1);
  const int fb = R0 == 0 ? 1 : 0;
  const u128 R = fb ? R1 : R0;
  const u128 tau = scaled_draw(mu_of(u_draw), R);
  const u128 wc = fb ? w1 : w0, ec = fb ? e1 : e0;
  if (tid == 0) {
    s_c = C - 1;
    s_before = R;
  }
  __syncthreads();
  if (tid < C && ec <= tau && tau < ec + wc) {
    s_c = tid;
    s_before = ec;
  }
  __syncthreads();
  DrawRow d;
  d.P = P + (int64_t)j * V;
  d.mp = mrow[j];
  d.Q = (j < K && !fb) ? Q + (int64_t)j * V : nullptr;
  d.mq = j < K ? mrow[K + 1 + j] : RowMeta{};
  d.V = V;
  // Each thread takes kPer consecutive elements of the chunk (all loads at once;
  // indices clamped into the chunk, elements past a1 unused).
  constexpr int kPer = kChunk / kRowThreads;
  static_assert(kPer * kRowThreads == kChunk, "a chunk splits evenly over the threads");
  const int x0 = s_c * kChunk, x1 = min(V, x0 + kChunk);
  const int a0 = min(x1, x0 + tid * kPer), a1 = min(x1, a0 + kPer);
  float pv[kPer], qv[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int x = min(a0 + u, x1 - 1);
    pv[u] = d.P[x];
    qv[u] = d.Q ? d.Q[x] : 0.f;
  }
  u128 mine = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u)
    if (a0 + u < a1) mine += d.w(a0 + u, pv[u], qv[u]);
  u128 tot;
  const u128 excl = s_before + block_excl_scan<u128, kRowThreads>(mine, scan, tot);
  if (excl <= tau && tau < excl + mine) {
    u128 run = excl;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      if (a0 + u < a1) {
        run += d.w(a0 + u, pv[u], qv[u]);
        if (run > tau) {
          s_tok = a0 + u;
          break;
        }
      }
    }
  }
  __syncthreads();
  const int tok = s_tok;
  for (int i = tid; i <= K; i += kRowThreads) {
    int32_t t = -1;
    if (i < j) t = dr[i];
    else if (i == j) t = tok;
    out_tokens[(int64_t)b * (K + 1) + i] = t;
  }
  if (tid == 0) out_n[b] = j;
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
  DrawRow d;
  d.P = P + (int64_t)j * V;
  d.mp = meta[j];
  d.Q = j < K ? Q + (int64_t)j * V : nullptr;
  d.mq = j < K ? meta[K + 1 + j] : RowMeta{};
  d.V = V;
  const int per = (V + kEntryThreads - 1) / kEntryThreads;
  const int x0 = min(V, tid * per), x1 = min(V, x0 + per);
  u128 local = 0;
  for (int x = x0; x < x1; ++x) local += d.w(x, d.P[x], d.Q ? d.Q[x] : 0.f);
  u128 R;
  u128 excl = block_excl_scan<u128, kEntryThreads>(local, scan, R);
  if (d.Q && R == 0) {
    d.Q = nullptr;
    local = 0;
    for (int x = x0; x < x1; ++x) local += d.w(x, d.P[x], 0.f);
    excl = block_excl_scan<u128, kEntryThreads>(local, scan, R);
  }
  u128* out = table + (int64_t)j * V;
  u128 run = excl;
  for (int x = x0; x < x1; ++x) {
    run += d.w(x, d.P[x], d.Q ? d.Q[x] : 0.f);
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
    const u64 a = kept_mass(P + (int64_t)i * V, d, V, mp);
    const u64 c = kept_mass(Q + (int64_t)i * V, d, V, mq);
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

// The chunked stages are used while the rows (or entries) alone would leave
// most of the chip idle.
constexpr int kChunkedMaxRows = 1024;
constexpr int kChunkedMaxEntries = 64;

AcceptPlan accept_plan(int B, int K, int V, int input_kind, int64_t p_stride, int64_t q_stride) {
  AcceptPlan p{};
  p.shared = (p_stride == 0 && q_stride == 0);
  p.entries = p.shared ? 1 : B;
  p.rows_per_entry = 2 * K + 1;
  const int64_t R = (int64_t)p.entries * p.rows_per_entry;
  p.chunks = (V + kChunk - 1) / kChunk;
  p.chunked = R <= kChunkedMaxRows;
  p.draw_chunked = !p.shared && B <= kChunkedMaxEntries;
  p.meta_bytes = align_up((size_t)R * sizeof(RowMeta), 256);
  p.probs_bytes = input_kind == 1 ? align_up((size_t)R * V * sizeof(float), 256) : 0;
  p.table_bytes = p.shared ? align_up((size_t)(K + 1) * V * sizeof(u128), 256) : 0;
  if (p.chunked) {
    p.state_bytes = align_up((size_t)R * sizeof(RowState), 256);
    p.hist_bytes = align_up((size_t)kLevels * R * kBins * sizeof(uint32_t), 256) +
                   align_up((size_t)kLevels * R * kBins * sizeof(u64), 256);
    p.cand_bytes = align_up((size_t)R * kCandCap * sizeof(u64), 256);
    p.stats_bytes = input_kind == 1 ? align_up((size_t)R * p.chunks * sizeof(float2), 256) : 0;
  }
  if (p.draw_chunked) p.esum_bytes = align_up((size_t)B * p.chunks * 2 * sizeof(u128), 256);
  return p;
}

size_t accept_workspace_total(const AcceptPlan& p) {
  return p.meta_bytes + p.probs_bytes + p.table_bytes + p.state_bytes + p.hist_bytes + p.cand_bytes +
         p.stats_bytes + p.esum_bytes;
}

hipError_t accept_launch(const AcceptPlan& plan, const float* p, const float* q, int input_kind,
                         int64_t p_stride, int64_t q_stride, const int32_t* draft,
                         const float* uniforms, int B, int K, int V, float temperature, int top_k,
                         float top_p, int32_t* out_tokens, int32_t* out_n, float* probs_out,
                         void* workspace, hipStream_t stream) {
  // Workspace: per-row results, select state, histograms (cleared by the first
  // kernel of the call), gathered keys, chunk statistics, draw sums,
  // probabilities, shared-mode tables.
  char* ws = reinterpret_cast<char*>(workspace);
  RowMeta* meta = reinterpret_cast<RowMeta*>(ws);
  ws += plan.meta_bytes;
  RowState* st = reinterpret_cast<RowState*>(ws);
  ws += plan.state_bytes;
  uint32_t* hcnt = reinterpret_cast<uint32_t*>(ws);
  const int64_t R = (int64_t)plan.entries * plan.rows_per_entry;
  u64* hmass = reinterpret_cast<u64*>(ws + align_up((size_t)kLevels * R * kBins * sizeof(uint32_t), 256));
  const int64_t lvl_stride = R * kBins;  // one level's histograms of every row
  ws += plan.hist_bytes;
  u64* cand = reinterpret_cast<u64*>(ws);
  ws += plan.cand_bytes;
  float2* stats = reinterpret_cast<float2*>(ws);
  ws += plan.stats_bytes;
  u128* esum = reinterpret_cast<u128*>(ws);
  ws += plan.esum_bytes;
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
  const bool use_k = top_k > 0 && top_k < V;
  const bool use_p = tp < (1u << 24);
  const int C = plan.chunks;
  hipError_t e;
  if (plan.chunked && use_k && top_k <= kTopKMax) {
    // Small top-k: per-chunk candidates, then one select per row over them
    // (the per-chunk validity flags and bounds go where the histograms would).
    const unsigned cg = (unsigned)(C * R);
    if (input_kind == 1) {
      hipLaunchKernelGGL(rows_stats_kernel, dim3(cg), dim3(kCT), 0, stream, p, q, p_stride, q_stride, K, V, C,
                         t_scale, stats, st, hcnt, hmass);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(rows_chunk_topk_kernel, dim3(cg), dim3(kCT), 0, stream, p, q, input_kind, p_stride, q_stride,
                       K, V, C, t_scale, probs, stats, top_k, cand, hcnt, hmass);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(rows_topk_merge_kernel, dim3((unsigned)R), dim3(kRowThreads), 0, stream, C, top_k, tp, cand,
                       hcnt, hmass, meta);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else if (plan.chunked) {
    const unsigned cg = (unsigned)(C * R);
    if (input_kind == 1) {  // the statistics pass also clears the rows' state and level-0 histograms
      hipLaunchKernelGGL(rows_stats_kernel, dim3(cg), dim3(kCT), 0, stream, p, q, p_stride, q_stride, K, V, C,
                         t_scale, stats, st, hcnt, hmass);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    } else {
      hipLaunchKernelGGL(rows_clear_kernel, dim3((unsigned)R), dim3(256), 0, stream, st, hcnt, hmass);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(rows_hist_kernel, dim3(cg), dim3(kCT), 0, stream, p, q, input_kind, p_stride, q_stride, K, V,
                       C, t_scale, (int)(use_k || use_p), probs, stats, st, hcnt, hmass);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(rows_find_kernel, dim3((unsigned)R), dim3(kRowThreads), 0, stream, V, top_k, tp, st, hcnt,
                       hmass, lvl_stride, meta);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (use_k || use_p) {
      for (int level = 1; level < kLevels; ++level) {
        hipLaunchKernelGGL(rows_refine_hist_kernel, dim3(cg), dim3(kCT), 0, stream, p, q, input_kind, p_stride,
                           q_stride, K, V, C, probs, st, hcnt, hmass, lvl_stride, level);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(rows_refine_find_kernel, dim3((unsigned)R), dim3(kRowThreads), 0, stream, st, hcnt, hmass,
                           lvl_stride, level, meta);
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
      const int rounds = (use_k && use_p) ? 2 : 1;
      for (int round = 0; round < rounds; ++round) {
        hipLaunchKernelGGL(rows_compact_kernel, dim3(cg), dim3(kCT), 0, stream, p, q, input_kind, p_stride, q_stride,
                           K, V, C, probs, st, cand);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(rows_resolve_kernel, dim3((unsigned)R), dim3(kRowThreads), 0, stream, V, top_k, tp, st,
                           hcnt, hmass, lvl_stride, cand, meta);
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
      if (use_k && use_p && top_k > kCandCap) {
        // Top-p after a top-k wider than the gather buffer can cross in a bin
        // too crowded to gather; such rows are finished by the rows kernel.
        hipLaunchKernelGGL(accept_rows_kernel, dim3(plan.rows_per_entry, plan.entries), dim3(kRowThreads), 0,
                           stream, p, q, input_kind, p_stride, q_stride, K, V, t_scale, top_k, tp, probs, meta, st,
                           hcnt, hmass);
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
    }
  } else {
    hipLaunchKernelGGL(accept_rows_kernel, dim3(plan.rows_per_entry, plan.entries), dim3(kRowThreads), 0, stream, p,
                       q, input_kind, p_stride, q_stride, K, V, t_scale, top_k, tp, probs, meta, nullptr, nullptr,
                       nullptr);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
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
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(accept_trials_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, PP, QQ, meta, table,
                       draft, uniforms, B, K, V, out_tokens, out_n);
    return hipGetLastError();
  }
  if (plan.draw_chunked) {
    hipLaunchKernelGGL(draw_sums_kernel, dim3((unsigned)(C * B)), dim3(kCT), 0, stream, PP, QQ, pps, qqs, meta,
                       (int64_t)plan.rows_per_entry, draft, uniforms, K, V, C, esum);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(draw_pick_kernel, dim3(B), dim3(kRowThreads), 0, stream, PP, QQ, pps, qqs, meta,
                       (int64_t)plan.rows_per_entry, draft, uniforms, K, V, C, esum, out_tokens, out_n);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(accept_entry_kernel, dim3(B), dim3(kEntryThreads), 0, stream, PP, QQ, pps, qqs, meta,
                     (int64_t)plan.rows_per_entry, draft, uniforms, K, V, out_tokens, out_n);
  return hipGetLastError();
}

}  // namespace vq
