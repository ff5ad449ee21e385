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
//     instructions with the non-temporal hint (the weights are read once). Two
//     blocks per wave are in flight.
//   * Two weight layouts. Tiled (made once by the pack kernel below, the fast
//     path): for every 32-row tile and every block, the 32 x 128 B of codes in
//     the order in which the lanes of a wave take them as the B operand of
//     v_mfma_f32_32x32x16_bf16 (lane n%32 holds row n, lanes 0-31 the first
//     half of a group's inputs and lanes 32-63 the second), followed by the
//     block's scales and biases row by row: a block is one contiguous run of
//     4.5 KiB (4-bit), every fetch is a linear 1 KiB stretch, and the loaded
//     registers are the operands, so a group is a chain of four MFMAs with no
//     LDS round trip. As soon as a group's registers are consumed, the same
//     loads of the block two ahead are issued into them. Row-major (the plain
//     format: row n holds its codes, scales and biases are [N, K/64]): each
//     instruction covers 8 rows x 128 B, an arrived block is written to a
//     per-wave LDS buffer (XOR-swizzled, bank-conflict free) and read back in
//     the operand layout, and each lane fetches the scales and biases of its
//     own column.
//   * Codes become bf16 in registers. 4-bit: OR-ing a nibble into the mantissa
//     of 128.0 gives the exact bf16 value 128 + q, two per 32-bit word, and the
//     constant 128 is removed per group through the group sums of x. 8-bit:
//     v_cvt_f32_ubyte + a byte permute gives the exact bf16 q.
//   * x (zero-padded to MT = 4, 8 or 16 rows) is staged in LDS in chunks of 16
//     groups, in the element order of the unpack, with its per-group sums.
//     Optionally it is RMS-normalised on the way in (x * 1/sqrt(mean(x^2) +
//     eps), rounded to bf16), from per-row sums of squares that the producer of
//     x wrote. A workgroup whose range of groups spans several chunks loads the
//     next chunk into registers while it computes the current one.
//   * The MFMA gives D_g = sum_{k in g} x*q' per group; scale and bias apply in
//     float32:
//         acc += s * D_g + (b - 128 s) * sum_{k in g} x     (4-bit)
//         acc += s * D_g +  b         * sum_{k in g} x     (8-bit)
//   * Parallelism beyond N/128 workgroups comes from splitting K across
//     workgroups; float32 partials go to the workspace and the last workgroup of
//     a column block (integer completion counter) adds them in split order, so
//     results are bit-identical run to run. Partial-sum writes interleaved with
//     the weight stream cost read bandwidth far beyond their own size, so a wide
//     output (at least 512 column blocks) is not split at all: its workgroups
//     walk the whole of K.
//   * Epilogues: store (bf16 or float32); residual (y = bf16(r + bf16(acc)),
//     with per-row sums of squares of y per 128-column block for the next
//     RMSNorm); SwiGLU (rows packed as 64 gate rows then the 64 matching up
//     rows per 128-row block; y = bf16(silu(bf16(g)) * bf16(u)), N/2 columns).
#include <math.h>

#include <type_traits>

#include "lanes.h"
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
constexpr int kCG = 16;                   // groups per LDS chunk of x
constexpr int kRowBytes = 128;            // bytes per row per pipeline block
constexpr int kLoads = 32 * kRowBytes / (64 * 16);  // dwordx4 per lane per block (= 4)
constexpr size_t kCounterBytes = 32768;   // completion counters (split-K only)
constexpr int kPlanWGs = 2 * kNumCU;      // workgroups the split plan aims for

enum { kLayoutRow = 0, kLayoutRowScalar = 1, kLayoutTiled = 2 };

template <int BITS>
struct BlockCfg {
  static constexpr int GB = kRowBytes / (8 * BITS);            // groups per block: 4 (4-bit), 2 (8-bit)
  static constexpr int SB = BITS == 4 ? 16 : 8;                // tiled scale|bias bytes per row per block
  static constexpr int BYTES = 32 * kRowBytes + 32 * SB;       // tiled bytes per (tile, block)
  static constexpr int IN_FLIGHT = 2;                           // blocks in flight per wave
};

// Everything a launch needs; passed by value in the kernel arguments.
struct QmmArgs {
  const uint16_t* x;
  int64_t ldx;
  const float* x_ss;  // RMSNorm prologue: sums of squares [M][ss_parts]
  int ss_parts;
  float eps;
  const uint8_t* wq;  // row-major codes, or the tiled pack
  const uint16_t* scales;
  const uint16_t* biases;
  int M, N, K;
  int splits, groups_per_split;
  void* y;
  int64_t ldy;
  int y_f32;
  const uint16_t* res;  // residual epilogue
  int64_t ldr;
  float* y_ss;          // residual epilogue: sums of squares of y [M][ceil(N / 128)] (nullable)
  float* partial;
  int* counters;
};

// One pipeline block held by one lane: 4 x 16 bytes of codes and the scales
// and biases of the block's groups for the lane's own output column (4 bf16
// each for 4-bit, 2 for 8-bit).
struct Regs {
  u32x4 w[kLoads];
  uint32_t s[2], b[2];
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Two floats to bf16, rounded to nearest even, in one instruction
// (v_cvt_pk_bf16_f32); lo in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) { return (uint16_t)pack_bf16x2(f, 0.f); }

__device__ __forceinline__ float round_bf16(float f) { return bf16_bits_to_f32(f32_to_bf16_rne(f)); }

// Eight nibbles -> eight bf16 values 128 + q, in the element order
// (q0, q4, q1, q5, q2, q6, q3, q7).
__device__ __forceinline__ bf16x8 unpack4(uint32_t w, uint32_t m, uint32_t c) {
  u32x4 t;
  t[0] = (w & m) | c;
  t[1] = ((w >> 4) & m) | c;
  t[2] = ((w >> 8) & m) | c;
  t[3] = ((w >> 12) & m) | c;
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

// CHUNK: the workgroup's range of groups may exceed one LDS chunk of x (CG
// groups); the next chunk is then prefetched into registers while the current
// one is computed. Without it the range is at most CG groups. CG is kCG, or
// half of it for 16 rows with CHUNK, so that the prefetch registers are those
// of 8 rows and the occupancy stays.
template <int BITS, int MT, int LAYOUT, int EPI, bool NORM, bool CHUNK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 8))) void qmm_kernel(const QmmArgs a) {
  constexpr int GB = BlockCfg<BITS>::GB;
  constexpr int kInFlight = BlockCfg<BITS>::IN_FLIGHT;
  // Accumulator registers that hold rows < MT: with the 32x32 output layout,
  // register r of lane half h holds row 8*(r/4) + 4*h + r%4.
  constexpr int kUseful = MT <= 8 ? 4 : 8;
  constexpr int CG = (CHUNK && MT == 16) ? kCG / 2 : kCG;  // groups per LDS chunk of x
  constexpr int XU = CG * 8 + 1;                            // 16-byte units per LDS row of x (+1 pad)

  __shared__ u32x4 xl[MT * XU];
  __shared__ float xsum[CG][16];
  __shared__ u32x4 tl[LAYOUT == kLayoutTiled ? 1 : kWaves][32 * 8];
  __shared__ float red[kWaves][16];
  __shared__ float inv_rms[16];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int cb = blockIdx.x;
  const int split = blockIdx.y;
  const int M = a.M, N = a.N, K = a.K;
  const int G = K >> 6;                                                // groups of the matrix
  const int Gp = LAYOUT == kLayoutTiled ? (G + GB - 1) / GB * GB : G;  // groups of the layout
  const int g0 = split * a.groups_per_split;
  const int g1 = min(Gp, g0 + a.groups_per_split);
  const int ng = g1 - g0;
  const int nblk = (ng + GB - 1) / GB;
  const int n0 = cb * kColsWG;

  // ---- code and scale/bias addresses
  const int lrow = lane >> 3;
  const int lchunk = lane & 7;
  const uint8_t* lptr[kLoads];
  const uint8_t* tile_base = nullptr;
  const uint16_t* srow = nullptr;
  const uint16_t* brow = nullptr;
  if constexpr (LAYOUT == kLayoutTiled) {
    const int n_tiles = (N + 31) / 32;
    const int tile = min((n0 + wave * kTileN) / 32, n_tiles - 1);
    tile_base = a.wq + (size_t)tile * (Gp / GB) * BlockCfg<BITS>::BYTES;
  } else {
    const size_t row_bytes = (size_t)K * BITS / 8;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int n = min(n0 + wave * kTileN + 8 * j + lrow, N - 1);
      lptr[j] = a.wq + (size_t)n * row_bytes;
    }
    // Scale / bias rows of this lane's output column (lanes l and l+32 share one).
    const int ncol = min(n0 + wave * kTileN + l32, N - 1);
    srow = a.scales + (size_t)ncol * G;
    brow = a.biases + (size_t)ncol * G;
  }
  auto tiled_block = [&](int bi) __attribute__((always_inline)) -> const uint8_t* {
    // Block index clamped inside [g0, g1); one contiguous run per block.
    const int kb = min(g0 / GB + bi, (g1 - 1) / GB);
    return tile_base + (size_t)kb * BlockCfg<BITS>::BYTES;
  };
  auto issue_codes = [&](Regs& R, int bi, int j) __attribute__((always_inline)) {
    R.w[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(tiled_block(bi) + j * 1024 + lane * 16));
  };
  auto issue_sb = [&](Regs& R, int bi) __attribute__((always_inline)) {
    const uint8_t* blk = tiled_block(bi);
    if constexpr (BITS == 4) {
      const u32x4 sb = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(blk + 32 * kRowBytes + l32 * 16));
      R.s[0] = sb[0];
      R.s[1] = sb[1];
      R.b[0] = sb[2];
      R.b[1] = sb[3];
    } else {
      typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 sbv = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(blk + 32 * kRowBytes + l32 * 8));
      const uint2 sb = make_uint2(sbv[0], sbv[1]);
      R.s[0] = sb.x;
      R.b[0] = sb.y;
      R.s[1] = R.b[1] = 0u;
    }
  };
  auto issue = [&](Regs& R, int bi) __attribute__((always_inline)) {
    if constexpr (LAYOUT == kLayoutTiled) {
#pragma unroll
      for (int j = 0; j < kLoads; ++j) issue_codes(R, bi, j);
      issue_sb(R, bi);
    } else {
      // Byte offset of this lane's chunk (clamped inside [g0, g1)).
      const int gc = min(g0 + bi * GB + (lchunk * 16) / (8 * BITS), g1 - 1);
      const size_t off = (size_t)gc * (8 * BITS) + (lchunk * 16) % (8 * BITS);
#pragma unroll
      for (int j = 0; j < kLoads; ++j) R.w[j] = *reinterpret_cast<const u32x4*>(lptr[j] + off);
      if constexpr (LAYOUT == kLayoutRow) {
        // GB groups from a GB-aligned group index that stays inside [g0, g1).
        const int gq = min(g0 + bi * GB, g1 - GB);
        if constexpr (GB == 4) {
          const uint2 sv = *reinterpret_cast<const uint2*>(srow + gq);
          const uint2 bv = *reinterpret_cast<const uint2*>(brow + gq);
          R.s[0] = sv.x;
          R.s[1] = sv.y;
          R.b[0] = bv.x;
          R.b[1] = bv.y;
        } else {
          R.s[0] = *reinterpret_cast<const uint32_t*>(srow + gq);
          R.b[0] = *reinterpret_cast<const uint32_t*>(brow + gq);
          R.s[1] = R.b[1] = 0u;
        }
      } else {
        uint32_t sw[4], bw[4];
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
          const int gq = min(g0 + bi * GB + (jb < GB ? jb : 0), g1 - 1);
          sw[jb] = srow[gq];
          bw[jb] = brow[gq];
        }
        R.s[0] = sw[0] | (sw[1] << 16);
        R.s[1] = sw[2] | (sw[3] << 16);
        R.b[0] = bw[0] | (bw[1] << 16);
        R.b[1] = bw[2] | (bw[3] << 16);
      }
    }
  };

  // Code blocks in flight per wave. In the split variants every block load is
  // issued unconditionally (block index clamped into the range, so past its end
  // the loads re-read its last block) and the blocks of an x chunk are
  // unrolled, so the wait counts the compiler derives are exact: with a
  // conditional issue it cannot count the loads in flight at the next block and
  // waits for all of them, which leaves one block in flight instead of two. The
  // chunked variant issues only blocks inside the range, under tests known at
  // compile time except in a ragged last chunk.
  Regs R[kInFlight];

  // ---- x, staged in chunks of CG groups in the element order of the unpack,
  // with per-group sums. Chunk ch covers groups [g0 + ch*CG, g0 + (ch+1)*CG)
  // of this workgroup's range; the next chunk is loaded into registers while the
  // current one is computed, and written to LDS between two barriers.
  constexpr int kIters = MT * CG * 8 / kThreads;
  static_assert(kIters * kThreads == MT * CG * 8, "staging loop must be uniform");
  const int gx1 = min(g1, G);  // groups past G exist only as zero padding of the tiled layout
  u32x4 xv[kIters];
  static_assert(!CHUNK || LAYOUT == kLayoutTiled, "chunked ranges are planned for the tiled layout only");
  auto load_x = [&](int ch) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int t = tid + it * kThreads;
      const int m = t / (CG * 8);
      const int c = t % (CG * 8);
      const int gg = max(0, min(g0 + ch * CG + (c >> 3), gx1 - 1));
      xv[it] = *reinterpret_cast<const u32x4*>(a.x + (size_t)min(m, M - 1) * a.ldx + (size_t)gg * 64 + (c & 7) * 8);
    }
  };
  auto store_x = [&](int ch) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int t = tid + it * kThreads;
      const int m = t / (CG * 8);
      const int c = t % (CG * 8);
      const int gg = g0 + ch * CG + (c >> 3);
      u32x4 w = (m < M && gg < gx1) ? xv[it] : u32x4{0, 0, 0, 0};
      if constexpr (NORM) {
        if (m < M) {
          const float r = inv_rms[m];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            w[e] = pack_bf16x2(bf16_bits_to_f32(w[e] & 0xFFFFu) * r, bf16_bits_to_f32(w[e] >> 16) * r);
          }
        }
      }
      float s8 = bf16_bits_to_f32(w[0] & 0xFFFFu) + bf16_bits_to_f32(w[0] >> 16) +
                 bf16_bits_to_f32(w[1] & 0xFFFFu) + bf16_bits_to_f32(w[1] >> 16) +
                 bf16_bits_to_f32(w[2] & 0xFFFFu) + bf16_bits_to_f32(w[2] >> 16) +
                 bf16_bits_to_f32(w[3] & 0xFFFFu) + bf16_bits_to_f32(w[3] >> 16);
      s8 = sum8_lanes(s8);
      if ((c & 7) == 0) xsum[c >> 3][m] = s8;
      if (BITS == 4) {
        u32x4 o;
        o[0] = __builtin_amdgcn_perm(w[2], w[0], 0x05040100u);
        o[1] = __builtin_amdgcn_perm(w[2], w[0], 0x07060302u);
        o[2] = __builtin_amdgcn_perm(w[3], w[1], 0x05040100u);
        o[3] = __builtin_amdgcn_perm(w[3], w[1], 0x07060302u);
        w = o;
      }
      xl[m * XU + c] = w;
    }
  };
  load_x(0);
  // RMSNorm prologue: wave w reduces the sums of squares of rows w, w+4, ...
  // (4 parts per lane, butterfly order), loaded before the code blocks.
  float ssv[NORM ? 4 : 1][NORM ? 4 : 1];
  if constexpr (NORM) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = wave + kWaves * i;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int p = lane + 64 * u;
        ssv[i][u] = (m < M && p < a.ss_parts) ? a.x_ss[(size_t)m * a.ss_parts + p] : 0.f;
      }
    }
  }
  // x is waited for before the first code blocks go out: issued together, its
  // few lines would queue behind the burst of code requests of every
  // workgroup at the start of the kernel.
  __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
  for (int i = 0; i < kInFlight; ++i) issue(R[i], i);
  if constexpr (NORM) {
    // The four rows' wave sums (DPP and permlane steps, no LDS) run
    // interleaved: four independent chains.
    float t[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = sum64_lanes((ssv[i][0] + ssv[i][1]) + (ssv[i][2] + ssv[i][3]));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = wave + kWaves * i;
      if (lane == 0 && m < M) inv_rms[m] = 1.f / sqrtf(t[i] / (float)K + a.eps);
    }
    __syncthreads();
  }
  store_x(0);
  __syncthreads();

  float acc[kUseful];
#pragma unroll
  for (int r = 0; r < kUseful; ++r) acc[r] = 0.f;
  u32x4* tw = tl[LAYOUT == kLayoutTiled ? 0 : wave];
  uint32_t cur_s[2], cur_b[2];  // scales / biases of the block being computed
  uint32_t nib_mask = 0x000F000Fu, nib_bias = 0x43004300u;
  asm volatile("" : "+v"(nib_mask), "+v"(nib_bias));

  // Consume a block: keep its scales / biases; the row-major layouts transpose
  // the codes through LDS (the tiled layout already holds them in operand order).
  auto consume = [&](const Regs& R) __attribute__((always_inline)) {
    if constexpr (LAYOUT != kLayoutTiled) {
#pragma unroll
      for (int j = 0; j < kLoads; ++j) tw[tslot(8 * j + lrow, lchunk)] = R.w[j];
    }
    cur_s[0] = R.s[0];
    cur_s[1] = R.s[1];
    cur_b[0] = R.b[0];
    cur_b[1] = R.b[1];
  };
  // Compute block bi of this workgroup's range, block bc of its x chunk.
  // `tail`: the block may run past the range (a run-time test per group).
  auto compute = [&](Regs& R, int bi, int bc, bool more, bool tail) __attribute__((always_inline)) {
#pragma unroll
    for (int jb = 0; jb < GB; ++jb) {
      const int gl = bi * GB + jb;  // group index within this workgroup's range
      const int gx = bc * GB + jb;  // group index within the staged x chunk
      if (tail && gl >= ng) break;
      bf16x8 av[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int unit = (BITS == 4) ? gx * 8 + half * 4 + i : gx * 8 + (i >> 1) * 4 + half * 2 + (i & 1);
        av[i] = __builtin_bit_cast(bf16x8, xl[(l32 & (MT - 1)) * XU + unit]);
      }
      u32x4 wv0, wv1;
      if constexpr (LAYOUT == kLayoutTiled) {
        wv0 = R.w[BITS == 4 ? jb : 2 * jb];
        wv1 = R.w[BITS == 4 ? jb : 2 * jb + 1];
      } else if (BITS == 4) {
        wv0 = tw[tslot(l32, 2 * jb + half)];
        wv1 = wv0;
      } else {
        wv0 = tw[tslot(l32, 4 * jb + half)];
        wv1 = tw[tslot(l32, 4 * jb + 2 + half)];
      }
      f32x16 d = {};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x8 bv;
        if (BITS == 4) {
          bv = unpack4(wv0[i], nib_mask, nib_bias);
        } else {
          const u32x4 wh = (i >> 1) ? wv1 : wv0;
          bv = (i & 1) ? unpack8(wh[2], wh[3]) : unpack8(wh[0], wh[1]);
        }
        d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv, d, 0, 0, 0);
      }
      if constexpr (LAYOUT == kLayoutTiled) {
        // This group's code registers are free: fetch the same loads of block bi + kInFlight.
        if (more) {
          issue_codes(R, bi + kInFlight, BITS == 4 ? jb : 2 * jb);
          if (BITS == 8) issue_codes(R, bi + kInFlight, 2 * jb + 1);
        }
      }
      const uint32_t sw = cur_s[jb >> 1], bw = cur_b[jb >> 1];
      const float s = __uint_as_float((jb & 1) ? (sw & 0xFFFF0000u) : (sw << 16));
      const float bb = __uint_as_float((jb & 1) ? (bw & 0xFFFF0000u) : (bw << 16));
      const float c = (BITS == 4) ? __builtin_fmaf(-128.f, s, bb) : bb;
#pragma unroll
      for (int r = 0; r < kUseful; ++r) {
        const int m = 8 * (r >> 2) + 4 * half + (r & 3);
        acc[r] = __builtin_fmaf(s, d[r], __builtin_fmaf(c, xsum[gx][m], acc[r]));
      }
    }
  };

  constexpr int kBPC = CG / GB;  // blocks per x chunk
  static_assert(kBPC % kInFlight == 0, "the register ring must restart at every chunk");
  // The blocks of x chunk ch. KIND 0: a chunk followed by another one (every
  // next block is issued; the issues past the range of the split variants are
  // clamped re-reads, see the block ring above); 1: the last chunk of a walk,
  // full (the issues stop kInFlight blocks before its end, known at compile
  // time); 2: the last chunk, ragged (a run-time test). Issues under a
  // compile-time condition keep the compiler's wait counts exact; a run-time
  // test makes it wait for every load in flight.
  auto chunk_blocks = [&](int ch, auto kind) __attribute__((always_inline)) {
    constexpr int KIND = decltype(kind)::value;
#pragma unroll
    for (int bc = 0; bc < kBPC; ++bc) {
      const int b = ch * kBPC + bc;
      if (b >= nblk) break;
      Regs& Rb = R[bc % kInFlight];
      const bool more = KIND == 0 ? true : KIND == 1 ? bc + kInFlight < kBPC : b + kInFlight < nblk;
      consume(Rb);
      if constexpr (LAYOUT == kLayoutTiled) {
        if (more) issue_sb(Rb, b + kInFlight);
      } else {
        if (more) issue(Rb, b + kInFlight);
      }
      compute(Rb, b, bc, more, KIND == 2);
    }
  };
  if constexpr (CHUNK) {
    // A walk over the whole of K: the next chunk of x is loaded into registers
    // while this one is computed, and written to LDS between two barriers.
    const int nch = (ng + CG - 1) / CG;
    for (int ch = 0; ch + 1 < nch; ++ch) {
      load_x(ch + 1);
      chunk_blocks(ch, std::integral_constant<int, 0>{});
      __syncthreads();  // every wave is done with this chunk of x
      store_x(ch + 1);
      __syncthreads();
    }
    if (nblk - (nch - 1) * kBPC == kBPC)
      chunk_blocks(nch - 1, std::integral_constant<int, 1>{});
    else
      chunk_blocks(nch - 1, std::integral_constant<int, 2>{});
  } else {
#pragma unroll
    for (int bc = 0; bc < kBPC; ++bc) {
      if (bc >= nblk) break;
      Regs& Rb = R[bc % kInFlight];
      consume(Rb);
      if constexpr (LAYOUT == kLayoutTiled) {
        issue_sb(Rb, bc + kInFlight);
      } else {
        issue(Rb, bc + kInFlight);
      }
      compute(Rb, bc, bc, true, true);
    }
  }

  // ------------------------------------------------------------------ epilogue
  const int n = n0 + wave * kTileN + l32;
  const bool n_ok = n < N;
  const int n_cb = (N + kColsWG - 1) / kColsWG;
  uint16_t* yb = reinterpret_cast<uint16_t*>(a.y);
  auto store = [&](int m, int col, float v) __attribute__((always_inline)) {
    if (a.y_f32)
      reinterpret_cast<float*>(a.y)[(size_t)m * a.ldy + col] = v;
    else
      yb[(size_t)m * a.ldy + col] = f32_to_bf16_rne(v);
  };
  // Residual: y = bf16(r + bf16(v)); returns the stored value as float.
  auto residual = [&](int m, int col, float v) __attribute__((always_inline)) -> float {
    const float h = round_bf16(bf16_bits_to_f32(a.res[(size_t)m * a.ldr + col]) + round_bf16(v));
    yb[(size_t)m * a.ldy + col] = f32_to_bf16_rne(h);
    return h;
  };
  auto swiglu = [&](float g, float u) __attribute__((always_inline)) -> uint16_t {
    const float gb = round_bf16(g);
    return f32_to_bf16_rne(gb / (1.f + expf(-gb)) * round_bf16(u));
  };

  if (a.splits == 1) {
    if constexpr (EPI == kEpiStore) {
      if (n_ok) {
#pragma unroll
        for (int r = 0; r < kUseful; ++r) {
          const int m = 8 * (r >> 2) + 4 * half + (r & 3);
          if (m < M) store(m, n, acc[r]);
        }
      }
    } else if constexpr (EPI == kEpiResidual) {
      float sq[kUseful];
#pragma unroll
      for (int r = 0; r < kUseful; ++r) {
        const int m = 8 * (r >> 2) + 4 * half + (r & 3);
        sq[r] = 0.f;
        if (n_ok && m < M) {
          const float h = residual(m, n, acc[r]);
          sq[r] = h * h;
        }
      }
      if (a.y_ss) {
        // Sum over the wave's 32 columns (lanes of one half), then over the waves.
#pragma unroll
        for (int off = 16; off > 0; off >>= 1) {
#pragma unroll
          for (int r = 0; r < kUseful; ++r) sq[r] += __shfl_xor(sq[r], off);
        }
#pragma unroll
        for (int r = 0; r < kUseful; ++r)
          if (l32 == 0) red[wave][8 * (r >> 2) + 4 * half + (r & 3)] = sq[r];
        __syncthreads();
        if (tid < M) a.y_ss[(size_t)tid * n_cb + cb] = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
      }
    } else {
      // SwiGLU: waves 2, 3 hold the up rows of the gate rows of waves 0, 1.
      float* upl = reinterpret_cast<float*>(&tl[0][0]);  // 16 x 64 floats; the block buffers are free now
      __syncthreads();
      if (wave >= 2) {
#pragma unroll
        for (int r = 0; r < kUseful; ++r)
          upl[(8 * (r >> 2) + 4 * half + (r & 3)) * 64 + (wave - 2) * 32 + l32] = acc[r];
      }
      __syncthreads();
      const int col = cb * 64 + wave * 32 + l32;
      if (wave < 2 && col < N / 2) {
#pragma unroll
        for (int r = 0; r < kUseful; ++r) {
          const int m = 8 * (r >> 2) + 4 * half + (r & 3);
          if (m < M) yb[(size_t)m * a.ldy + col] = swiglu(acc[r], upl[m * 64 + wave * 32 + l32]);
        }
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
  float* part = a.partial + (size_t)split * M * N;
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
    s_last = __hip_atomic_fetch_add(&a.counters[cb], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.splits - 1;
  __syncthreads();
  if (!s_last) return;
  // Sum the partials in split order, kBatch splits x kVPT x kPair loads in
  // flight per thread (at most 36, 64 for 16 rows: each batch is a round trip,
  // and the 16-row variant reads twice the partials per split; a budget of 64
  // at 4 and 8 rows measured slower). Thread t, value i covers element
  // t + i * 256 of the block's [M][128] (store, residual) or of its [M][64]
  // gate/up column pairs (SwiGLU).
  constexpr int kCols = EPI == kEpiSwiGLU ? kColsWG / 2 : kColsWG;
  constexpr int kVPT = MT * kCols / kThreads;
  constexpr int kPair = EPI == kEpiSwiGLU ? 2 : 1;
  constexpr int kBatch = (MT == 16 ? 64 : 36) / (kVPT * kPair);
  float v[kVPT][kPair];
  size_t idx[kVPT];
  bool ok[kVPT];
#pragma unroll
  for (int i = 0; i < kVPT; ++i) {
    const int t = tid + i * kThreads;
    const int m = t / kCols;
    const int col = cb * kColsWG + t % kCols;
    ok[i] = m < M && col < N;
    idx[i] = (size_t)m * N + col;
#pragma unroll
    for (int h = 0; h < kPair; ++h) v[i][h] = 0.f;
  }
  // The residual rows go out with the first batch of partial loads. These
  // loads and the partial loads below are issued unconditionally (indices
  // clamped into the arrays, unused values discarded at the sum): a load under
  // a per-lane condition is followed by a full wait in the compiled code, which
  // turned the residual loads into one round trip each.
  uint32_t rv[EPI == kEpiResidual ? kVPT : 1];
  if constexpr (EPI == kEpiResidual) {
#pragma unroll
    for (int i = 0; i < kVPT; ++i) {
      const int t = tid + i * kThreads;
      const int m = min(t / kCols, M - 1);
      const int col = min(cb * kColsWG + t % kCols, N - 1);
      rv[i] = a.res[(size_t)m * a.ldr + col];
    }
  }
  const size_t sstride = (size_t)M * N;
  for (int sp = 0; sp < a.splits; sp += kBatch) {
    float pv[kBatch][kVPT][kPair];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const size_t su = (size_t)min(sp + u, a.splits - 1) * sstride;
#pragma unroll
      for (int i = 0; i < kVPT; ++i) {
#pragma unroll
        for (int h = 0; h < kPair; ++h)
          pv[u][i][h] = __hip_atomic_load(&a.partial[su + (ok[i] ? idx[i] + h * 64 : 0)], __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
#pragma unroll
      for (int i = 0; i < kVPT; ++i) {
#pragma unroll
        for (int h = 0; h < kPair; ++h) v[i][h] += (ok[i] && sp + u < a.splits) ? pv[u][i][h] : 0.f;
      }
    }
  }
  if constexpr (EPI == kEpiStore) {
#pragma unroll
    for (int i = 0; i < kVPT; ++i) {
      const int t = tid + i * kThreads;
      if (ok[i]) store(t / kCols, cb * kColsWG + t % kCols, v[i][0]);
    }
  } else if constexpr (EPI == kEpiResidual) {
    // Threads 0-127 of value i hold row 2i, threads 128-255 row 2i+1: each
    // wave sums half a row, then the two halves are added.
    float sq[kVPT];
#pragma unroll
    for (int i = 0; i < kVPT; ++i) {
      const int t = tid + i * kThreads;
      sq[i] = 0.f;
      if (ok[i]) {
        const int col = cb * kColsWG + t % kCols;
        const float h = round_bf16(bf16_bits_to_f32(rv[i]) + round_bf16(v[i][0]));
        yb[(size_t)(t / kCols) * a.ldy + col] = f32_to_bf16_rne(h);
        sq[i] = h * h;
      }
    }
    if (a.y_ss) {
#pragma unroll
      for (int i = 0; i < kVPT; ++i) sq[i] = sum64_lanes(sq[i]);
#pragma unroll
      for (int i = 0; i < kVPT; ++i)
        if (lane == 0) red[wave & 1][2 * i + (wave >> 1)] = sq[i];
    }
    if (a.y_ss) {
      __syncthreads();
      if (tid < M) a.y_ss[(size_t)tid * n_cb + cb] = red[0][tid] + red[1][tid];
    }
  } else {
#pragma unroll
    for (int i = 0; i < kVPT; ++i) {
      const int t = tid + i * kThreads;
      const int col = cb * (kColsWG / 2) + t % kCols;
      if (ok[i] && col < N / 2) yb[(size_t)(t / kCols) * a.ldy + col] = swiglu(v[i][0], v[i][1]);
    }
  }
  if (tid == 0) __hip_atomic_store(&a.counters[cb], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Tiled layout from the row-major one. Workgroup (tile t, block kb), thread u:
// 16-byte unit u of the block, the bytes 16 * (2 * (u / 64) + (u % 64) / 32) ..
// +15 of row 32t + (u % 64) % 32 (the operand that lane u % 64 of a wave takes
// with its (u / 64)-th load); threads 0-31 also write the scale|bias record of
// row 32t + u. Rows past N and groups past K are zero.
template <int BITS>
__global__ __launch_bounds__(256) void qmm_pack_kernel(const uint8_t* __restrict__ wq,
                                                       const uint16_t* __restrict__ scales,
                                                       const uint16_t* __restrict__ biases, int N, int K,
                                                       uint8_t* __restrict__ out) {
  constexpr int GB = BlockCfg<BITS>::GB;
  const int t = blockIdx.x;
  const int kb = blockIdx.y;
  const int KB = gridDim.y;
  const int G = K / 64;
  const size_t row_bytes = (size_t)K * BITS / 8;
  const int u = threadIdx.x;
  const int r = (u & 63) & 31, c = 2 * (u >> 6) + ((u & 63) >> 5);
  const int n = 32 * t + r;
  uint8_t* blk = out + ((size_t)t * KB + kb) * BlockCfg<BITS>::BYTES;
  const size_t src = (size_t)kb * kRowBytes + c * 16;
  u32x4 w = {0u, 0u, 0u, 0u};
  if (n < N && src < row_bytes) w = *reinterpret_cast<const u32x4*>(wq + (size_t)n * row_bytes + src);
  *reinterpret_cast<u32x4*>(blk + (size_t)u * 16) = w;
  if (u < 32) {
    const int nr = 32 * t + u;
    uint32_t sv[4] = {0u, 0u, 0u, 0u}, bv[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      const int g = kb * GB + j;
      if (nr < N && g < G) {
        sv[j] = scales[(size_t)nr * G + g];
        bv[j] = biases[(size_t)nr * G + g];
      }
    }
    if constexpr (BITS == 4) {
      u32x4 sb;
      sb[0] = sv[0] | (sv[1] << 16);
      sb[1] = sv[2] | (sv[3] << 16);
      sb[2] = bv[0] | (bv[1] << 16);
      sb[3] = bv[2] | (bv[3] << 16);
      *reinterpret_cast<u32x4*>(blk + 32 * kRowBytes + u * 16) = sb;
    } else {
      uint2 sb;
      sb.x = sv[0] | (sv[1] << 16);
      sb.y = bv[0] | (bv[1] << 16);
      *reinterpret_cast<uint2*>(blk + 32 * kRowBytes + u * 8) = sb;
    }
  }
}

// Per-row sums of squares of a bf16 matrix per 128-column block (the layout the
// residual epilogue writes), for the first RMSNorm of a chain.
__global__ __launch_bounds__(128) void row_sumsq_kernel(const uint16_t* __restrict__ x, int64_t ldx, int N,
                                                        float* __restrict__ out) {
  __shared__ float r2[2];
  const int cb = blockIdx.x, m = blockIdx.y;
  const int n_cb = gridDim.x;
  const int col = cb * kColsWG + threadIdx.x;
  float v = 0.f;
  if (col < N) {
    v = bf16_bits_to_f32(x[(size_t)m * ldx + col]);
    v = v * v;
  }
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  if ((threadIdx.x & 63) == 0) r2[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) out[(size_t)m * n_cb + cb] = r2[0] + r2[1];
}

}  // namespace

size_t qmm_pack_bytes(int bits, int N, int K) {
  const int GB = bits == 4 ? BlockCfg<4>::GB : BlockCfg<8>::GB;
  const size_t blk = bits == 4 ? BlockCfg<4>::BYTES : BlockCfg<8>::BYTES;
  const size_t tiles = (size_t)(N + 31) / 32;
  const size_t kbs = (size_t)(K / 64 + GB - 1) / GB;
  return tiles * kbs * blk;
}

hipError_t qmm_pack(const void* wq, const void* scales, const void* biases, int bits, int N, int K, void* out,
                    hipStream_t stream) {
  const int GB = bits == 4 ? BlockCfg<4>::GB : BlockCfg<8>::GB;
  dim3 grid((N + 31) / 32, (K / 64 + GB - 1) / GB);
  auto* w = reinterpret_cast<const uint8_t*>(wq);
  auto* s = reinterpret_cast<const uint16_t*>(scales);
  auto* b = reinterpret_cast<const uint16_t*>(biases);
  auto* o = reinterpret_cast<uint8_t*>(out);
  if (bits == 4)
    hipLaunchKernelGGL(qmm_pack_kernel<4>, grid, dim3(256), 0, stream, w, s, b, N, K, o);
  else
    hipLaunchKernelGGL(qmm_pack_kernel<8>, grid, dim3(256), 0, stream, w, s, b, N, K, o);
  return hipGetLastError();
}

hipError_t row_sumsq(const void* x, int64_t ldx, int M, int N, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(row_sumsq_kernel, dim3((N + kColsWG - 1) / kColsWG, M), dim3(128), 0, stream,
                     reinterpret_cast<const uint16_t*>(x), ldx, N, out);
  return hipGetLastError();
}

int qmm_sumsq_parts(int N) { return (N + kColsWG - 1) / kColsWG; }

QmmPlan qmm_plan(int bits, int M, int N, int K, bool tiled) {
  QmmPlan p{};
  p.mt = M <= 4 ? 4 : M <= 8 ? 8 : 16;
  p.cols_per_wg = kColsWG;
  p.n_blocks = (N + kColsWG - 1) / kColsWG;
  const int GB = bits == 4 ? 4 : 2;
  const int G = tiled ? (K / 64 + GB - 1) / GB * GB : K / 64;
  // About kPlanWGs workgroups. With at least that many column blocks (a wide
  // output such as the vocabulary projection) K is not split at all: every
  // split writes M x N float32 partial sums, and writes interleaved with the
  // weight stream cost read bandwidth out of proportion to their size. A
  // workgroup then walks the whole of K in LDS chunks of x (for 16 rows, chunks
  // of half as many groups, so that the prefetch registers do not cost
  // occupancy). Otherwise K is
  // split into ranges of at most one chunk (kCG groups), split boundaries on
  // multiples of 4 groups (the scale/bias vector unit and the tiled block).
  if (tiled && p.n_blocks >= kPlanWGs) {
    p.chunked = true;
    p.groups_per_split = G;
    p.splits = 1;
    p.counter_bytes = 0;
    p.partial_bytes = 0;
    return p;
  }
  int s = (kPlanWGs + p.n_blocks - 1) / p.n_blocks;
  const int s_lds = (G + kCG - 1) / kCG;
  s = s < s_lds ? s_lds : s;
  s = s < 1 ? 1 : s;
  int gps = (G + s - 1) / s;
  gps = (gps + 2) / 4 * 4;  // nearest multiple of 4
  if (gps < 4) gps = 4;
  // At least three blocks per range for long K (64 groups or more, the shapes
  // this was measured on): the ring issues two blocks up front and then one per
  // block consumed (clamped past the range), so a two-block range pays two
  // re-read blocks and gains nothing from the ring.
  if (gps < 3 * GB && G >= 64) gps = (3 * GB + 3) / 4 * 4;
  // Outputs of fewer than 64 column blocks (the 5120-wide o projection) split K
  // into full x chunks: the last workgroup of a column block sums fewer
  // partials, which outweighs the workgroups lost (o: 240 instead of 480).
  if (gps > kCG || (p.n_blocks < 64 && G > kCG)) gps = kCG;
  p.groups_per_split = gps;
  p.splits = (G + gps - 1) / gps;
  // n_blocks <= kCounterBytes / 4 follows from the N <= 2^20 limit of the ABI.
  p.counter_bytes = p.splits > 1 ? kCounterBytes : 0;
  p.partial_bytes = p.splits > 1 ? align_up((size_t)p.splits * M * N * sizeof(float), 256) : 0;
  return p;
}

hipError_t qmm_launch(const QmmPlan& plan, const QmmCall& c, hipStream_t stream) {
  QmmArgs a{};
  a.x = reinterpret_cast<const uint16_t*>(c.x);
  a.ldx = c.ldx;
  a.x_ss = c.x_ss;
  a.ss_parts = c.ss_parts;
  a.eps = c.eps;
  a.wq = reinterpret_cast<const uint8_t*>(c.wq);
  a.scales = reinterpret_cast<const uint16_t*>(c.scales);
  a.biases = reinterpret_cast<const uint16_t*>(c.biases);
  a.M = c.M;
  a.N = c.N;
  a.K = c.K;
  a.splits = plan.splits;
  a.groups_per_split = plan.groups_per_split;
  a.y = c.y;
  a.ldy = c.ldy;
  a.y_f32 = c.y_f32;
  a.res = reinterpret_cast<const uint16_t*>(c.res);
  a.ldr = c.ldr;
  a.y_ss = c.y_ss;
  a.counters = reinterpret_cast<int*>(c.workspace);
  a.partial = plan.splits > 1
                  ? reinterpret_cast<float*>(reinterpret_cast<char*>(c.workspace) + plan.counter_bytes)
                  : nullptr;
  dim3 grid(plan.n_blocks, plan.splits);
  dim3 block(kThreads);
  const int G = c.K / 64;
  int layout = kLayoutTiled;
  if (!c.tiled) {
    // Vector (8-byte) scale/bias loads need 4-group alignment of every row and
    // split start; otherwise 2-byte loads.
    const bool vec = (G % 4 == 0) && (plan.groups_per_split % 4 == 0) &&
                     (reinterpret_cast<uintptr_t>(c.scales) % 8 == 0) &&
                     (reinterpret_cast<uintptr_t>(c.biases) % 8 == 0);
    layout = vec ? kLayoutRow : kLayoutRowScalar;
  }
  const bool norm = c.x_ss != nullptr;
#define VQ_K(B, MT, L, E, NRM, CH) hipLaunchKernelGGL((qmm_kernel<B, MT, L, E, NRM, CH>), grid, block, 0, stream, a)
#define VQ_EPI_NORM_CH(B, MT, CH)                                      \
  switch (c.epilogue * 2 + (norm ? 1 : 0)) {                           \
    case 0: VQ_K(B, MT, kLayoutTiled, kEpiStore, false, CH); break;    \
    case 1: VQ_K(B, MT, kLayoutTiled, kEpiStore, true, CH); break;     \
    case 2: VQ_K(B, MT, kLayoutTiled, kEpiResidual, false, CH); break; \
    case 3: VQ_K(B, MT, kLayoutTiled, kEpiResidual, true, CH); break;  \
    case 4: VQ_K(B, MT, kLayoutTiled, kEpiSwiGLU, false, CH); break;   \
    default: VQ_K(B, MT, kLayoutTiled, kEpiSwiGLU, true, CH); break;   \
  }
#define VQ_EPI_NORM(B, MT)          \
  if (plan.chunked) {               \
    VQ_EPI_NORM_CH(B, MT, true)     \
  } else {                          \
    VQ_EPI_NORM_CH(B, MT, false)    \
  }
#define VQ_BITS(B)                                                      \
  if (layout == kLayoutRow) {                                           \
    if (plan.mt == 4) VQ_K(B, 4, kLayoutRow, kEpiStore, false, false);  \
    else if (plan.mt == 8) VQ_K(B, 8, kLayoutRow, kEpiStore, false, false); \
    else VQ_K(B, 16, kLayoutRow, kEpiStore, false, false);              \
  } else if (layout == kLayoutRowScalar) {                              \
    if (plan.mt == 4) VQ_K(B, 4, kLayoutRowScalar, kEpiStore, false, false); \
    else if (plan.mt == 8) VQ_K(B, 8, kLayoutRowScalar, kEpiStore, false, false); \
    else VQ_K(B, 16, kLayoutRowScalar, kEpiStore, false, false);        \
  } else if (plan.mt == 4) {                                            \
    VQ_EPI_NORM(B, 4)                                                   \
  } else if (plan.mt == 8) {                                            \
    VQ_EPI_NORM(B, 8)                                                   \
  } else {                                                              \
    VQ_EPI_NORM(B, 16)                                                  \
  }
  if (c.bits == 4) {
    VQ_BITS(4)
  } else {
    VQ_BITS(8)
  }
#undef VQ_BITS
#undef VQ_EPI_NORM
#undef VQ_EPI_NORM_CH
#undef VQ_K
  return hipGetLastError();
}

}  // namespace vq
