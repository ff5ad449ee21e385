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
//   * Parallelism beyond N/32 tiles comes from splitting K across workgroups;
//     float32 partials go to the workspace and the last workgroup of a column
//     block (integer completion counter) adds them in split order, so results
//     are bit-identical run to run.
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
constexpr int kChunkGroups = 16;          // groups of x staged in LDS at a time
constexpr int kRowUnits = kChunkGroups * 8 + 1;  // 16-byte units per LDS row (+1 pad)
constexpr size_t kCounterBytes = 4096;           // completion counters (split-K only)
static_assert(2 * kNumCU * sizeof(int) <= kCounterBytes, "counter region too small");

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

template <int BITS, int MT>
__global__ __launch_bounds__(kThreads) void qmm_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ wq,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases, int M, int N, int K,
    int splits, int groups_per_split, void* __restrict__ y, int64_t ldy, int y_f32,
    float* __restrict__ partial, int* __restrict__ counters) {
  constexpr int kLoads = BITS / 4;  // 16-byte loads per lane per group
  constexpr int PF = 4;             // groups prefetched ahead
  constexpr int kUseful = MT / 2;   // accumulator registers that hold rows < MT

  __shared__ uint4 xl[MT * kRowUnits];
  __shared__ float xsum[kChunkGroups][16];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;  // which half of the group's K range this lane loads
  const int cb = blockIdx.x;
  const int split = blockIdx.y;
  const int G = K >> 6;
  const int g0 = split * groups_per_split;
  const int g1 = min(G, g0 + groups_per_split);

  const int n = cb * kColsWG + wave * kTileN + (lane & 31);
  const bool n_ok = n < N;
  const int nc = n_ok ? n : N - 1;  // clamped row for loads; results discarded
  const uint8_t* wrow = wq + (size_t)nc * (size_t)(K * BITS / 8);
  const uint16_t* srow = scales + (size_t)nc * G;
  const uint16_t* brow = biases + (size_t)nc * G;
  const int arow = lane & 31;  // A-operand row (x row) of this lane

  float acc[kUseful];
#pragma unroll
  for (int r = 0; r < kUseful; ++r) acc[r] = 0.f;

  uint4 wb[PF][kLoads];
  uint32_t sb[PF];
  auto issue = [&](int slot, int g) {
    if (g < g1) {
#pragma unroll
      for (int h = 0; h < kLoads; ++h)
        wb[slot][h] = *reinterpret_cast<const uint4*>(wrow + (size_t)g * (8 * BITS) + h * 32 + half * 16);
      sb[slot] = (uint32_t)srow[g] | ((uint32_t)brow[g] << 16);
    }
  };
#pragma unroll
  for (int p = 0; p < PF; ++p) issue(p, g0 + p);

  int chunk0 = g0;
  for (int gb = g0; gb < g1; gb += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int g = gb + p;
      if (g >= g1) break;
      if (((g - g0) % kChunkGroups) == 0) {
        // Stage x[:, chunk] into LDS, permuted for the unpack order, plus group sums.
        chunk0 = g;
        __syncthreads();
        for (int t = tid; t < MT * kChunkGroups * 8; t += kThreads) {
          const int m = t / (kChunkGroups * 8);
          const int c = t % (kChunkGroups * 8);
          const int gg = chunk0 + (c >> 3);
          uint4 v = make_uint4(0, 0, 0, 0);
          if (m < M && gg < g1)
            v = *reinterpret_cast<const uint4*>(x + (size_t)m * ldx + (size_t)gg * 64 + (c & 7) * 8);
          float s8 = bf16_bits_to_f32(v.x & 0xFFFFu) + bf16_bits_to_f32(v.x >> 16) +
                     bf16_bits_to_f32(v.y & 0xFFFFu) + bf16_bits_to_f32(v.y >> 16) +
                     bf16_bits_to_f32(v.z & 0xFFFFu) + bf16_bits_to_f32(v.z >> 16) +
                     bf16_bits_to_f32(v.w & 0xFFFFu) + bf16_bits_to_f32(v.w >> 16);
          s8 += __shfl_xor(s8, 1);
          s8 += __shfl_xor(s8, 2);
          s8 += __shfl_xor(s8, 4);
          if ((c & 7) == 0) xsum[c >> 3][m] = s8;
          if (BITS == 4) {
            uint4 o;
            o.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
            o.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
            o.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
            o.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
            v = o;
          }
          xl[m * kRowUnits + c] = v;
        }
        __syncthreads();
      }

      const uint4 w0 = wb[p][0];
      uint4 w1 = w0;
      if (kLoads == 2) w1 = wb[p][kLoads - 1];
      const uint32_t sbv = sb[p];
      issue(p, g + PF);

      const int gl = g - chunk0;
      f32x16 d = {};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x8 b;
        int unit;  // 16-byte unit of x matching this MFMA's K slice
        if (BITS == 4) {
          const uint32_t wi = i == 0 ? w0.x : i == 1 ? w0.y : i == 2 ? w0.z : w0.w;
          b = unpack4(wi);
          unit = gl * 8 + half * 4 + i;
        } else {
          const uint4 wh = (i < 2) ? w0 : w1;
          const uint32_t lo = (i & 1) ? wh.z : wh.x;
          const uint32_t hi = (i & 1) ? wh.w : wh.y;
          b = unpack8(lo, hi);
          unit = gl * 8 + (i >> 1) * 4 + half * 2 + (i & 1);
        }
        bf16x8 a = {};
        if (arow < MT) a = __builtin_bit_cast(bf16x8, xl[arow * kRowUnits + unit]);
        d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, d, 0, 0, 0);
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
  float* part = partial + (size_t)split * M * N;
  if (n_ok) {
#pragma unroll
    for (int r = 0; r < kUseful; ++r) {
      const int m = 8 * (r >> 2) + 4 * half + (r & 3);
      if (m < M) part[(size_t)m * N + n] = acc[r];
    }
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = (atomicAdd(&counters[cb], 1) == splits - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  for (int t = tid; t < M * kColsWG; t += kThreads) {
    const int m = t / kColsWG;
    const int col = cb * kColsWG + t % kColsWG;
    if (col >= N) continue;
    float v = 0.f;
    for (int sp = 0; sp < splits; ++sp) v += __builtin_nontemporal_load(&partial[((size_t)sp * M + m) * N + col]);
    store(m, col, v);
  }
  if (tid == 0) counters[cb] = 0;
}

}  // namespace

QmmPlan qmm_plan(int bits, int M, int N, int K) {
  QmmPlan p{};
  p.mt = M <= 8 ? 8 : 16;
  p.cols_per_wg = kColsWG;
  p.n_blocks = (N + kColsWG - 1) / kColsWG;
  const int G = K / 64;
  // Aim for about two resident workgroups per compute unit, with at least four
  // groups of K per workgroup so that the prefetch pipeline fills.
  int s = (2 * kNumCU + p.n_blocks - 1) / p.n_blocks;
  s = s < 1 ? 1 : s;
  int max_s = G / 4 > 0 ? G / 4 : 1;
  s = s > max_s ? max_s : s;
  s = s > 64 ? 64 : s;
  const int gps = (G + s - 1) / s;
  p.groups_per_split = gps;
  p.splits = (G + gps - 1) / gps;
  // Split-K only happens when there are fewer than 2 * kNumCU column blocks, so
  // the counters always fit a fixed 4 KiB region at the start of the workspace:
  // calls of different shapes that share a workspace never see each other's
  // partial sums in their counter slots.
  p.counter_bytes = p.splits > 1 ? kCounterBytes : 0;
  p.partial_bytes = p.splits > 1 ? align_up((size_t)p.splits * M * N * sizeof(float), 256) : 0;
  (void)bits;
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
#define VQ_QMM_LAUNCH(B, MTV)                                                                     \
  hipLaunchKernelGGL((qmm_kernel<B, MTV>), grid, block, 0, stream, xp, ldx, wp, sp, bp, M, N, K, \
                     plan.splits, plan.groups_per_split, y, ldy, y_f32, partial, counters)
  if (bits == 4) {
    if (plan.mt == 8) VQ_QMM_LAUNCH(4, 8); else VQ_QMM_LAUNCH(4, 16);
  } else {
    if (plan.mt == 8) VQ_QMM_LAUNCH(8, 8); else VQ_QMM_LAUNCH(8, 16);
  }
#undef VQ_QMM_LAUNCH
  return hipGetLastError();
}

}  // namespace vq
