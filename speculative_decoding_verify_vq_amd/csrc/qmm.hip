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
//   * One wave owns a tile of 32 output columns. For each group of 64 inputs,
//     each lane issues one 16-byte load (4-bit) or two (8-bit) of its column's
//     packed codes: lanes 0-31 take the first half of the group, lanes 32-63 the
//     second, so the group is exactly one 32x32x16 MFMA chain of four.
//   * Codes are turned into bf16 in registers. 4-bit: OR-ing a nibble into the
//     mantissa of 128.0 gives the exact bf16 value 128 + q, two per 32-bit word
//     (v_and_or_b32), and the constant 128 is removed per group through the
//     group sums of x. 8-bit: v_cvt_f32_ubyte + a byte permute gives exact bf16 q.
//   * x rows live in LDS (staged per chunk of groups, zero-padded to MT rows) in
//     the element order that the register unpack produces; the per-group sums
//     of x are computed while staging.
//   * The MFMA produces D_g = sum_{k in g} x*q' per group; the group's affine
//     scale and bias are applied in float32:
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
constexpr size_t kCounterBytes = 16384;   // completion counters (split-K only)
constexpr int kMaxCounters = (int)(kCounterBytes / sizeof(int));

// Groups of x staged in LDS per chunk: 32 for up to 8 rows (32 KiB), 16 for 16 rows.
template <int MT>
struct ChunkCfg {
  static constexpr int CG = MT <= 8 ? 32 : 16;
  static constexpr int UNITS = CG * 8 + 1;  // 16-byte units per LDS row (+1 pad)
};

// Groups per pipeline block: 8 for 4-bit (one 16-byte load per lane per group),
// 4 for 8-bit (two loads per group) -> 8 KiB of codes per wave in flight.
template <int BITS>
struct BlockCfg {
  static constexpr int GB = BITS == 4 ? 8 : 4;
  static constexpr int LPG = BITS / 4;  // 16-byte code loads per lane per group
  static constexpr int NW = GB * LPG;   // code loads per block
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

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// One pipeline block: the codes of GB groups of this lane's column, and their
// scales and biases (bf16 bit patterns, GB of each).
template <int BITS>
struct Block {
  uint4 w[BlockCfg<BITS>::NW];
  uint32_t s[BlockCfg<BITS>::GB / 2];
  uint32_t b[BlockCfg<BITS>::GB / 2];
};

template <int BITS, int MT, bool VEC>
__global__ __launch_bounds__(kThreads) void qmm_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ wq,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases, int M, int N, int K,
    int splits, int groups_per_split, void* __restrict__ y, int64_t ldy, int y_f32,
    float* __restrict__ partial, int* __restrict__ counters) {
  using BC = BlockCfg<BITS>;
  using CC = ChunkCfg<MT>;
  constexpr int GB = BC::GB;
  constexpr int kUseful = MT / 2;  // accumulator registers that hold rows < MT

  __shared__ uint4 xl[MT * CC::UNITS];
  __shared__ float xsum[CC::CG][16];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;  // which half of each group's K range this lane loads
  const int cb = blockIdx.x;
  const int split = blockIdx.y;
  const int G = K >> 6;
  const int g0 = split * groups_per_split;
  const int g1 = min(G, g0 + groups_per_split);
  const int nblk = (g1 - g0 + GB - 1) / GB;

  const int n = cb * kColsWG + wave * kTileN + (lane & 31);
  const bool n_ok = n < N;
  const int nc = n_ok ? n : N - 1;  // clamped row for loads; results discarded
  const uint8_t* wrow = wq + (size_t)nc * (size_t)(K * BITS / 8) + half * 16;
  const uint16_t* srow = scales + (size_t)nc * G;
  const uint16_t* brow = biases + (size_t)nc * G;
  const int arow = (lane & 31) & (MT - 1);  // A-operand row; rows >= MT are never read back

  // Loads for block bi (clamped to the last block, so every load is in bounds
  // and issued unconditionally).
  auto load_block = [&](Block<BITS>& B, int bi) {
    const int gs = g0 + min(bi, nblk - 1) * GB;
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      const int g = min(gs + j, g1 - 1);
#pragma unroll
      for (int h = 0; h < BC::LPG; ++h)
        B.w[j * BC::LPG + h] = *reinterpret_cast<const uint4*>(wrow + (size_t)g * (8 * BITS) + h * 32);
    }
    if constexpr (VEC) {
      // gs is a multiple of GB and G % GB == 0, so the GB entries stay inside the row.
      if constexpr (GB == 8) {
        const uint4 sv = *reinterpret_cast<const uint4*>(srow + gs);
        const uint4 bv = *reinterpret_cast<const uint4*>(brow + gs);
        B.s[0] = sv.x; B.s[1] = sv.y; B.s[2] = sv.z; B.s[3] = sv.w;
        B.b[0] = bv.x; B.b[1] = bv.y; B.b[2] = bv.z; B.b[3] = bv.w;
      } else {
        const uint2 sv = *reinterpret_cast<const uint2*>(srow + gs);
        const uint2 bv = *reinterpret_cast<const uint2*>(brow + gs);
        B.s[0] = sv.x; B.s[1] = sv.y;
        B.b[0] = bv.x; B.b[1] = bv.y;
      }
    } else {
#pragma unroll
      for (int j = 0; j < GB / 2; ++j) {
        const int ga = min(gs + 2 * j, g1 - 1), gb2 = min(gs + 2 * j + 1, g1 - 1);
        B.s[j] = (uint32_t)srow[ga] | ((uint32_t)srow[gb2] << 16);
        B.b[j] = (uint32_t)brow[ga] | ((uint32_t)brow[gb2] << 16);
      }
    }
  };

  // Stage x[:, groups gc .. gc+CG) into LDS (element order of the unpack) and the
  // group sums. All loads of a thread are issued before any is consumed.
  auto stage = [&](int gc) {
    constexpr int kIters = MT * CC::CG * 8 / kThreads;
    static_assert(kIters * kThreads == MT * CC::CG * 8, "staging loop must be uniform");
    uint4 v[kIters];
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int t = tid + it * kThreads;
      const int m = t / (CC::CG * 8);
      const int c = t % (CC::CG * 8);
      const int gg = gc + (c >> 3);
      v[it] = make_uint4(0, 0, 0, 0);
      if (m < M && gg < g1)
        v[it] = *reinterpret_cast<const uint4*>(x + (size_t)m * ldx + (size_t)gg * 64 + (c & 7) * 8);
    }
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int t = tid + it * kThreads;
      const int m = t / (CC::CG * 8);
      const int c = t % (CC::CG * 8);
      uint4 w = v[it];
      float s8 = bf16_bits_to_f32(w.x & 0xFFFFu) + bf16_bits_to_f32(w.x >> 16) +
                 bf16_bits_to_f32(w.y & 0xFFFFu) + bf16_bits_to_f32(w.y >> 16) +
                 bf16_bits_to_f32(w.z & 0xFFFFu) + bf16_bits_to_f32(w.z >> 16) +
                 bf16_bits_to_f32(w.w & 0xFFFFu) + bf16_bits_to_f32(w.w >> 16);
      s8 += __shfl_xor(s8, 1);
      s8 += __shfl_xor(s8, 2);
      s8 += __shfl_xor(s8, 4);
      if ((c & 7) == 0) xsum[c >> 3][m] = s8;
      if (BITS == 4) {
        uint4 o;
        o.x = __builtin_amdgcn_perm(w.z, w.x, 0x05040100u);
        o.y = __builtin_amdgcn_perm(w.z, w.x, 0x07060302u);
        o.z = __builtin_amdgcn_perm(w.w, w.y, 0x05040100u);
        o.w = __builtin_amdgcn_perm(w.w, w.y, 0x07060302u);
        w = o;
      }
      xl[m * CC::UNITS + c] = w;
    }
  };

  float acc[kUseful];
#pragma unroll
  for (int r = 0; r < kUseful; ++r) acc[r] = 0.f;

  int chunk0 = g0;
  auto compute_block = [&](const Block<BITS>& B, int bi) {
    const int gs = g0 + bi * GB;
    if (gs != g0 && (gs - g0) % CC::CG == 0) {  // next x chunk (only for long K ranges)
      chunk0 = gs;
      __syncthreads();
      stage(chunk0);
      __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      const int g = gs + j;
      if (g >= g1) break;
      const int gl = g - chunk0;
      bf16x8 a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int unit = (BITS == 4) ? gl * 8 + half * 4 + i : gl * 8 + (i >> 1) * 4 + half * 2 + (i & 1);
        a[i] = __builtin_bit_cast(bf16x8, xl[arow * CC::UNITS + unit]);
      }
      f32x16 d = {};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x8 bv;
        if (BITS == 4) {
          bv = unpack4(word_of(B.w[j], i));
        } else {
          const uint4& wh = B.w[j * 2 + (i >> 1)];
          bv = (i & 1) ? unpack8(wh.z, wh.w) : unpack8(wh.x, wh.y);
        }
        d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bv, d, 0, 0, 0);
      }
      const float s = bf16_bits_to_f32((B.s[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
      const float bb = bf16_bits_to_f32((B.b[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
      const float c = (BITS == 4) ? __builtin_fmaf(-128.f, s, bb) : bb;
#pragma unroll
      for (int r = 0; r < kUseful; ++r) {
        const int m = 8 * (r >> 2) + 4 * half + (r & 3);
        acc[r] = __builtin_fmaf(s, d[r], __builtin_fmaf(c, xsum[gl][m], acc[r]));
      }
    }
  };

  Block<BITS> A, Bk;
  load_block(A, 0);
  stage(g0);
  __syncthreads();
  for (int bi = 0; bi < nblk; bi += 2) {
    load_block(Bk, bi + 1);
    compute_block(A, bi);
    if (bi + 1 >= nblk) break;
    load_block(A, bi + 2);
    compute_block(Bk, bi + 1);
  }

  // ------------------------------------------------------------------ epilogue
  auto store = [&](int m, int col, float v) {
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
  const int GB = bits == 4 ? 8 : 4;
  const int CG = p.mt <= 8 ? 32 : 16;
  // Enough workgroups for about two per compute unit, and a K range per
  // workgroup that fits one LDS chunk of x. Split boundaries fall on pipeline
  // blocks (multiples of GB groups).
  int s = (2 * kNumCU + p.n_blocks - 1) / p.n_blocks;
  const int s_lds = (G + CG - 1) / CG;
  s = s < s_lds ? s_lds : s;
  s = s < 1 ? 1 : s;
  int gps = (G + s - 1) / s;
  gps = (gps + GB / 2) / GB * GB;  // nearest multiple of GB
  if (gps < GB) gps = GB;
  if (gps > CG) gps = CG;
  if (p.n_blocks > kMaxCounters) gps = G;  // too many column blocks to count: no split
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
  const int G = K / 64;
  const int GB = bits == 4 ? 8 : 4;
  const size_t va = bits == 4 ? 16 : 8;
  const bool vec = (G % GB == 0) && (plan.groups_per_split % GB == 0) &&
                   (reinterpret_cast<uintptr_t>(scales) % va == 0) && (reinterpret_cast<uintptr_t>(biases) % va == 0);
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
