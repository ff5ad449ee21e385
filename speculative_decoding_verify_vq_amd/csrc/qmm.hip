// Skinny weight-only-quantized matmul for gfx950.
//
//   y[m, n] = sum_k x[m, k] * (s[n, g(k)] * q[n, k] + b[n, g(k)]),  g(k) = k / 64
//
// The verify pass runs M = K+1 <= 16 rows through one pass over the weights
// (page "The fastest way to run local LLMs on a Mac", section "Why native MTP
// doubles decode"); the stock small-M quantized matmul re-reads the weights per
// row and a small-M kernel shares them across up to 16 rows (page "Speculative
// decoding and MTP on Apple silicon", Facts). Here every weight byte is read from
// HBM once per call, whatever M is.
//
// Mapping onto CDNA4:
//   * A workgroup owns 128 output columns (rows n of W) and a range of groups
//     (64 inputs each); each of its 4 waves owns 32 of the columns.
//   * Codes stream in blocks of 128 bytes per row (4 groups of 4-bit codes, 2 of
//     8-bit): one block of a wave is 32 rows x 128 B, fetched by 4 dwordx4
//     instructions that each cover 8 whole 128-byte lines. Three blocks per
//     wave are in flight. An arrived block is written to a per-wave LDS buffer
//     (XOR-swizzled so writes and reads are bank-conflict free) and read back in
//     the B-operand layout of v_mfma_f32_32x32x16_bf16: lane n (of 32) holds
//     the codes of row n, lanes 0-31 the first half of the group's inputs and
//     lanes 32-63 the second half, so a group is a chain of four MFMAs.
//   * Codes become bf16 in registers. 4-bit: OR-ing a nibble into the mantissa
//     of 128.0 gives the exact bf16 value 128 + q, two per 32-bit word, and the
//     constant 128 is removed per group through the group sums of x. 8-bit:
//     v_cvt_f32_ubyte + a byte permute gives the exact bf16 q.
//   * x (zero-padded to MT = 8 or 16 rows) is staged in LDS once per workgroup,
//     in the element order of the unpack, with its per-group sums; the scales
//     and biases of the workgroup's rows and groups are preloaded into LDS too.
//   * The MFMA gives D_g = sum_{k in g} x*q' per group; scale and bias apply in
//     float32:
//         acc += s * D_g + (b - 128 s) * sum_{k in g} x     (4-bit)
//         acc += s * D_g +  b         * sum_{k in g} x     (8-bit)
//   * Parallelism beyond N/128 workgroups comes from splitting K across
//     workgroups; float32 partials go to the workspace and the last workgroup of
//     a column block (integer completion counter) adds them in split order, so
//     results are bit-identical run to run.
#include "vq_internal.h"

namespace vq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kTileN = 32;                // columns per wave
constexpr int kColsWG = kWaves * kTileN;  // columns per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kCG = 16;                   // max groups per workgroup (one LDS chunk of x)
constexpr int kXUnits = kCG * 8 + 1;      // 16-byte units per LDS row of x (+1 pad)
constexpr int kSBStride = kCG + 1;        // u32 (scale | bias << 16) per LDS row (+1 pad)
constexpr int kRowBytes = 128;            // bytes per row per pipeline block
constexpr int kLoads = 32 * kRowBytes / (64 * 16);  // dwordx4 per lane per block (= 4)
constexpr int kInFlight = 3;              // blocks in flight per wave
constexpr size_t kCounterBytes = 32768;   // completion counters (split-K only)
constexpr int kMaxCounters = (int)(kCounterBytes / sizeof(int));

// Codes of one pipeline block held by one lane (4 x 16 bytes).
struct Regs {
  u32x4 w[kLoads];
};

template <int BITS>
struct BlockCfg {
  static constexpr int GB = kRowBytes / (8 * BITS);  // groups per block: 4 (4-bit), 2 (8-bit)
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Eight nibbles -> eight bf16 values 128 + q, in the element order
// (q0, q4, q1, q5, q2, q6, q3, q7).
__device__ __forceinline__ bf16x8 unpack4(uint32_t w) {
  u32x4 t;
  t[0] = (w & 0x000F000Fu) | 0x43004300u;
  t[1] = ((w >> 4) & 0x000F000Fu) | 0x43004300u;
  t[2] = ((w >> 8) & 0x000F000Fu) | 0x43004300u;
  t[3] = ((w >> 12) & 0x000F000Fu) | 0x43004300u;
  return __builtin_bit_cast(bf16x8, t);
}

// Eight bytes (two words) -> eight bf16 values q, in natural order. A byte
// converts exactly to float (v_cvt_f32_ubyteN) and its float has at most 8
// significant bits, so the top half of the float is the exact bf16.
__device__ __forceinline__ uint32_t bytes_to_bf16x2(uint32_t w, int lo_byte) {
  const float a = (float)((w >> (8 * lo_byte)) & 0xFFu);
  const float b = (float)((w >> (8 * lo_byte + 8)) & 0xFFu);
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

__device__ __forceinline__ bf16x8 unpack8(uint32_t w0, uint32_t w1) {
  u32x4 t;
  t[0] = bytes_to_bf16x2(w0, 0);
  t[1] = bytes_to_bf16x2(w0, 2);
  t[2] = bytes_to_bf16x2(w1, 0);
  t[3] = bytes_to_bf16x2(w1, 2);
  return __builtin_bit_cast(bf16x8, t);
}

// 16-byte slot of (row r, chunk c) in a wave's block buffer: 32 rows x 8 chunks,
// chunk index XOR-ed with (r / 2) % 8 so that both the coalesced writes (8 rows
// x 8 chunks per instruction) and the operand reads (32 rows, same chunk) spread
// over all LDS banks.
__device__ __forceinline__ int tslot(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

template <int BITS, int MT, bool VEC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 8))) void qmm_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ wq,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases, int M, int N, int K,
    int splits, int groups_per_split, void* __restrict__ y, int64_t ldy, int y_f32,
    float* __restrict__ partial, int* __restrict__ counters) {
  constexpr int GB = BlockCfg<BITS>::GB;
  constexpr int kUseful = MT / 2;  // accumulator registers that hold rows < MT

  __shared__ u32x4 xl[MT * kXUnits];
  __shared__ float xsum[kCG][16];
  __shared__ uint32_t sbl[kColsWG * kSBStride];
  __shared__ u32x4 tl[kWaves][32 * 8];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int cb = blockIdx.x;
  const int split = blockIdx.y;
  const int G = K >> 6;
  const size_t row_bytes = (size_t)K * BITS / 8;
  const int g0 = split * groups_per_split;
  const int g1 = min(G, g0 + groups_per_split);
  const int ng = g1 - g0;
  const int nblk = (ng + GB - 1) / GB;
  const int n0 = cb * kColsWG;

  // ---- coalesced code loads: instruction j, lane l -> row 8j + l/8, chunk l%8
  const int lrow = lane >> 3;
  const int lchunk = lane & 7;
  const uint8_t* lptr[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int n = min(n0 + wave * kTileN + 8 * j + lrow, N - 1);
    lptr[j] = wq + (size_t)n * row_bytes;
  }
  // Byte offset of this lane's chunk in block bi (clamped inside [g0, g1)).
  auto chunk_off = [&](int bi) __attribute__((always_inline)) -> size_t {
    const int gchunk = g0 + bi * GB + (lchunk * 16) / (8 * BITS);
    const int gc = min(gchunk, g1 - 1);
    return (size_t)gc * (8 * BITS) + (lchunk * 16) % (8 * BITS);
  };
  auto issue = [&](Regs& R, int bi) __attribute__((always_inline)) {
    const size_t off = chunk_off(bi);
#pragma unroll
    for (int j = 0; j < kLoads; ++j) R.w[j] = *reinterpret_cast<const u32x4*>(lptr[j] + off);
  };

  // Three code blocks in flight per wave. Every block load is issued
  // unconditionally (block index clamped) and the block sequence is unrolled,
  // so the wait counts the compiler derives are exact.
  Regs R[kInFlight];

  // ---- stage x (element order of the unpack) with group sums, and scale|bias
  {
    constexpr int kIters = MT * kCG * 8 / kThreads;
    static_assert(kIters * kThreads == MT * kCG * 8, "staging loop must be uniform");
    u32x4 v[kIters];
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int t = tid + it * kThreads;
      const int m = t / (kCG * 8);
      const int c = t % (kCG * 8);
      const int gg = min(g0 + (c >> 3), g1 - 1);
      v[it] = *reinterpret_cast<const u32x4*>(x + (size_t)min(m, M - 1) * ldx + (size_t)gg * 64 + (c & 7) * 8);
    }
    if constexpr (VEC) {
      // 4 groups of scales and of biases per 8-byte unit; kColsWG rows x (kCG / 4) units.
      constexpr int kSBIters = kColsWG * (kCG / 4) / kThreads;
#pragma unroll
      for (int it = 0; it < kSBIters; ++it) {
        const int t = tid + it * kThreads;
        const int r = t / (kCG / 4);
        const int u = t % (kCG / 4);
        const int gl = 4 * u;
        const int glc = min(gl, (ng - 1) & ~3);  // clamped: the load stays inside the row
        const int n = min(n0 + r, N - 1);
        const uint2 sv = *reinterpret_cast<const uint2*>(scales + (size_t)n * G + g0 + glc);
        const uint2 bv = *reinterpret_cast<const uint2*>(biases + (size_t)n * G + g0 + glc);
        uint32_t* d = &sbl[r * kSBStride + gl];
        d[0] = (sv.x & 0xFFFFu) | (bv.x << 16);
        d[1] = (sv.x >> 16) | (bv.x & 0xFFFF0000u);
        d[2] = (sv.y & 0xFFFFu) | (bv.y << 16);
        d[3] = (sv.y >> 16) | (bv.y & 0xFFFF0000u);
      }
    } else {
      for (int t = tid; t < kColsWG * ng; t += kThreads) {
        const int r = t / ng, gl = t % ng;
        const int n = min(n0 + r, N - 1);
        sbl[r * kSBStride + gl] =
            (uint32_t)scales[(size_t)n * G + g0 + gl] | ((uint32_t)biases[(size_t)n * G + g0 + gl] << 16);
      }
    }
    // The first code blocks go out after the x, scale and bias loads, so that
    // waiting for those (in-order counter) leaves the code blocks in flight.
    issue(R[0], 0);
    issue(R[1], 1);
    issue(R[2], 2);
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int t = tid + it * kThreads;
      const int m = t / (kCG * 8);
      const int c = t % (kCG * 8);
      const int gg = g0 + (c >> 3);
      u32x4 w = (m < M && gg < g1) ? v[it] : u32x4{0, 0, 0, 0};
      float s8 = bf16_bits_to_f32(w[0] & 0xFFFFu) + bf16_bits_to_f32(w[0] >> 16) +
                 bf16_bits_to_f32(w[1] & 0xFFFFu) + bf16_bits_to_f32(w[1] >> 16) +
                 bf16_bits_to_f32(w[2] & 0xFFFFu) + bf16_bits_to_f32(w[2] >> 16) +
                 bf16_bits_to_f32(w[3] & 0xFFFFu) + bf16_bits_to_f32(w[3] >> 16);
      s8 += __shfl_xor(s8, 1);
      s8 += __shfl_xor(s8, 2);
      s8 += __shfl_xor(s8, 4);
      if ((c & 7) == 0) xsum[c >> 3][m] = s8;
      if (BITS == 4) {
        u32x4 o;
        o[0] = __builtin_amdgcn_perm(w[2], w[0], 0x05040100u);
        o[1] = __builtin_amdgcn_perm(w[2], w[0], 0x07060302u);
        o[2] = __builtin_amdgcn_perm(w[3], w[1], 0x05040100u);
        o[3] = __builtin_amdgcn_perm(w[3], w[1], 0x07060302u);
        w = o;
      }
      xl[m * kXUnits + c] = w;
    }
  }
  __syncthreads();

  float acc[kUseful];
#pragma unroll
  for (int r = 0; r < kUseful; ++r) acc[r] = 0.f;
  u32x4* tw = tl[wave];
  const uint32_t* sbrow = &sbl[(wave * kTileN + l32) * kSBStride];
  const bool a_live = l32 < MT;  // lanes whose A row is a real (possibly zero) x row

  // Consume block bi held in R: transpose through LDS, then 4 (or 2) groups.
  auto consume = [&](const Regs& R) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) tw[tslot(8 * j + lrow, lchunk)] = R.w[j];
  };
  auto compute = [&](int bi) __attribute__((always_inline)) {
#pragma unroll
    for (int jb = 0; jb < GB; ++jb) {
      const int gl = bi * GB + jb;  // group index within this workgroup's range
      if (gl >= ng) break;
      bf16x8 a[4];
      if (a_live) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int unit = (BITS == 4) ? gl * 8 + half * 4 + i : gl * 8 + (i >> 1) * 4 + half * 2 + (i & 1);
          a[i] = __builtin_bit_cast(bf16x8, xl[l32 * kXUnits + unit]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = bf16x8{};
      }
      u32x4 wv0, wv1;
      if (BITS == 4) {
        wv0 = tw[tslot(l32, 2 * jb + half)];
        wv1 = wv0;
      } else {
        wv0 = tw[tslot(l32, 4 * jb + half)];
        wv1 = tw[tslot(l32, 4 * jb + 2 + half)];
      }
      const uint32_t sbv = sbrow[gl];
      f32x16 d = {};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x8 bv;
        if (BITS == 4) {
          bv = unpack4(wv0[i]);
        } else {
          const u32x4 wh = (i >> 1) ? wv1 : wv0;
          bv = (i & 1) ? unpack8(wh[2], wh[3]) : unpack8(wh[0], wh[1]);
        }
        d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bv, d, 0, 0, 0);
      }
      const float s = bf16_bits_to_f32(sbv & 0xFFFFu);
      const float bb = bf16_bits_to_f32(sbv >> 16);
      const float c = (BITS == 4) ? __builtin_fmaf(-128.f, s, bb) : bb;
#pragma unroll
      for (int r = 0; r < kUseful; ++r) {
        const int m = 8 * (r >> 2) + 4 * half + (r & 3);
        acc[r] = __builtin_fmaf(s, d[r], __builtin_fmaf(c, xsum[gl][m], acc[r]));
      }
    }
  };

  constexpr int kMaxBlocks = kCG / GB;
#pragma unroll
  for (int b = 0; b < kMaxBlocks; ++b) {
    if (b >= nblk) break;
    consume(R[b % kInFlight]);
    if (b + kInFlight < kMaxBlocks && b + kInFlight < nblk) issue(R[b % kInFlight], b + kInFlight);
    compute(b);
  }

  // ------------------------------------------------------------------ epilogue
  const int n = n0 + wave * kTileN + l32;
  const bool n_ok = n < N;
  auto store = [&](int m, int col, float v) __attribute__((always_inline)) {
    if (y_f32)
      reinterpret_cast<float*>(y)[(size_t)m * ldy + col] = v;
    else
      reinterpret_cast<uint16_t*>(y)[(size_t)m * ldy + col] = f32_to_bf16_rne(v);
  };
  if (splits == 1) {
    if (n_ok) {
#pragma unroll
      for (int r = 0; r < kUseful; ++r) {
        const int m = 8 * (r >> 2) + 4 * half + (r & 3);
        if (m < M) store(m, n, acc[r]);
      }
    }
    return;
  }
  // Split-K completion without cache-wide fences. The partial sums are written
  // with agent-scope (L2 write-through) stores and read back with agent-scope
  // loads, and the counter is an agent-scope atomic; "s_waitcnt vmcnt(0)" before
  // the barrier makes every partial store of the workgroup complete before its
  // counter increment is issued. No store or load of this exchange goes through
  // a possibly stale cache line, so no L2 writeback or invalidation is needed
  // (which would evict the weight lines other waves are still streaming).
  float* part = partial + (size_t)split * M * N;
  if (n_ok) {
#pragma unroll
    for (int r = 0; r < kUseful; ++r) {
      const int m = 8 * (r >> 2) + 4 * half + (r & 3);
      if (m < M) __hip_atomic_store(&part[(size_t)m * N + n], acc[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(&counters[cb], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == splits - 1;
  __syncthreads();
  if (!s_last) return;
  for (int t = tid; t < M * kColsWG; t += kThreads) {
    const int m = t / kColsWG;
    const int col = cb * kColsWG + t % kColsWG;
    if (col >= N) continue;
    float v = 0.f;
    for (int sp = 0; sp < splits; ++sp)
      v += __hip_atomic_load(&partial[((size_t)sp * M + m) * N + col], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    store(m, col, v);
  }
  if (tid == 0) __hip_atomic_store(&counters[cb], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

QmmPlan qmm_plan(int bits, int M, int N, int K) {
  QmmPlan p{};
  p.mt = M <= 8 ? 8 : 16;
  p.cols_per_wg = kColsWG;
  p.n_blocks = (N + kColsWG - 1) / kColsWG;
  const int G = K / 64;
  const int GB = bits == 4 ? 4 : 2;
  // Enough workgroups for about two per compute unit, and at most kCG groups
  // per workgroup (one LDS chunk of x). Split boundaries fall on multiples of 4
  // groups (the scale/bias preload unit).
  int s = (2 * kNumCU + p.n_blocks - 1) / p.n_blocks;
  const int s_lds = (G + kCG - 1) / kCG;
  s = s < s_lds ? s_lds : s;
  s = s < 1 ? 1 : s;
  int gps = (G + s - 1) / s;
  gps = (gps + 2) / 4 * 4;  // nearest multiple of 4
  if (gps < 4) gps = 4;
  if (gps > kCG) gps = kCG;
  (void)GB;
  (void)kMaxCounters;  // n_blocks <= kMaxCounters is guaranteed by the N <= 2^20 limit of the ABI
  p.groups_per_split = gps;
  p.splits = (G + gps - 1) / gps;
  p.counter_bytes = p.splits > 1 ? kCounterBytes : 0;
  p.partial_bytes = p.splits > 1 ? align_up((size_t)p.splits * M * N * sizeof(float), 256) : 0;
  return p;
}

hipError_t qmm_launch(const QmmPlan& plan, const void* x, int64_t ldx, const void* wq,
                      const void* scales, const void* biases, int bits, int M, int N, int K,
                      void* y, int64_t ldy, int y_f32, void* workspace, hipStream_t stream) {
  int* counters = reinterpret_cast<int*>(workspace);
  float* partial = plan.splits > 1
                       ? reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + plan.counter_bytes)
                       : nullptr;
  dim3 grid(plan.n_blocks, plan.splits);
  dim3 block(kThreads);
  auto* xp = reinterpret_cast<const uint16_t*>(x);
  auto* wp = reinterpret_cast<const uint8_t*>(wq);
  auto* sp = reinterpret_cast<const uint16_t*>(scales);
  auto* bp = reinterpret_cast<const uint16_t*>(biases);
  // Vector (8-byte) scale/bias loads need 4-group alignment of every row and
  // split start; otherwise 2-byte loads.
  const int G = K / 64;
  const bool vec = (G % 4 == 0) && (plan.groups_per_split % 4 == 0) &&
                   (reinterpret_cast<uintptr_t>(scales) % 8 == 0) && (reinterpret_cast<uintptr_t>(biases) % 8 == 0);
#define VQ_QMM_LAUNCH(B, MTV, V)                                                                     \
  hipLaunchKernelGGL((qmm_kernel<B, MTV, V>), grid, block, 0, stream, xp, ldx, wp, sp, bp, M, N, K, \
                     plan.splits, plan.groups_per_split, y, ldy, y_f32, partial, counters)
#define VQ_QMM_MT(B, V) \
  if (plan.mt == 8) VQ_QMM_LAUNCH(B, 8, V); else VQ_QMM_LAUNCH(B, 16, V);
  if (bits == 4) {
    if (vec) { VQ_QMM_MT(4, true) } else { VQ_QMM_MT(4, false) }
  } else {
    if (vec) { VQ_QMM_MT(8, true) } else { VQ_QMM_MT(8, false) }
  }
#undef VQ_QMM_MT
#undef VQ_QMM_LAUNCH
  return hipGetLastError();
}

}  // namespace vq
