// Multi-row decode attention for gfx950.
//
// For query row i < M, query head h, KV head g = h / G (G = Hq / Hkv):
//   out[i, h] = sum_{j <= T-M+i} softmax_j(scale * <q[i,h], k[g,j]>) * v[g,j]
//
// Stock decode attention re-reads the KV cache once per query row; a
// multi-row kernel reads each KV tile once for all rows (page "Speculative
// decoding and MTP on Apple silicon", Facts). Here one workgroup owns one KV
// head and one contiguous range of keys; all M*G query rows that share the KV
// head are processed against each K/V tile while it sits in LDS, so every KV
// byte is read from HBM once per call.
//
// Per 32-key tile:
//   * the tile is loaded with coalesced 16-byte loads into registers two tiles
//     ahead, then written to LDS row-major (into the second of two K/V buffers
//     where they fit, so a tile costs one barrier, not two);
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q rows
//     from LDS, or from registers with a single row tile); in the output
//     layout each lane holds 16 keys of one query row, so the online-softmax
//     statistics of a row live in one lane pair;
//   * O^T += V^T P^T on the same MFMA: B = P (this lane's own probabilities,
//     rounded to bf16), A = V read from LDS along the key axis with transposed
//     reads, so the row rescaling stays lane-local.
// Waves split the query rows into tiles of 32 and, when there are few rows,
// the head dimension of O across waves (each of those waves recomputes the
// same S tile, which costs MFMA time the memory-bound kernel has to spare).
// With several key ranges per head, each range's output normalised by its own
// sum (bf16) and its (max, sum) statistics (float32) go to the workspace, and a
// combine kernel merges them.
//
// 8-bit KV cache (same page, Facts: KV-quantized caches used together with
// speculation): codes u8 [Hkv, T_cap, D] and one (bf16 scale, bf16 bias) word
// per 64 codes; a tile is fetched as 16-code units with their word and
// dequantized (s * q + b, rounded to bf16) while it is written to LDS, so
// everything after the staging is the bf16 path. The append quantizes rows per
// group: scale = (max - min) / 255 and code = rint((x - min) / scale), both in
// correctly rounded float32, bias = min.
//
// Several sequences in one call (same page, Facts: one verify pass for several
// streams): the grid gains a sequence dimension; sequence b owns query rows
// row_start[b] .. row_start[b+1]-1 and T_b = seq_len[b] keys of its own cache
// (batch stride in the cache). The per-sequence values come from device arrays
// and are clamped into the launch's bounds, so inconsistent arrays can only
// give wrong outputs, never an access outside the buffers.
//
// Tree verify (page "Speculative decoding and MTP on Apple silicon", Facts:
// tree-attention masks on the full-attention layers): with a mask, row i sees
// the committed keys j < T-M and the drafted key T-M+t iff t == i or bit t of
// mask[i] is set (bits at or above M are ignored); without one, bits 0..i
// (causal). Each lane keeps its row's bits, so the mask costs one compare per
// score.
#include <math.h>

#include "lanes.h"
#include "vq_internal.h"

namespace vq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

// gfx950 transposed LDS read of 4 x 16-bit values (ds_read_b64_tr_b16); the
// address must be 8-byte aligned.
__device__ __forceinline__ v4i16 ds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)((__attribute__((address_space(3))) uint16_t*)(p)));
}

constexpr int kThreads = 256;
constexpr int kTileKeys = 32;
// Sixteen zero bytes in global memory: read in place of a tree mask word when
// there is none, and of query rows past the last one.
__device__ __attribute__((aligned(16))) uint32_t kZero16[4] = {0u, 0u, 0u, 0u};
typedef const uint32_t __attribute__((address_space(1))) global_u32;
typedef const u32x4 __attribute__((address_space(1))) global_u32x4;
typedef const bf16x8 __attribute__((address_space(1))) global_bf16x8;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  // v_cvt_pk_bf16_f32: both values rounded to nearest even in one instruction.
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

template <int D, int RT, bool KV8 = false>
struct AttnCfg {
  static constexpr int DS0 = (RT == 1) ? 4 : (RT == 2) ? 2 : 1;
  static constexpr int DS = DS0 < D / 32 ? DS0 : D / 32;  // head-dim slices per row tile
  static constexpr int DW = D / DS;                         // head dims per wave
  static constexpr int DT = DW / 32;                        // 32-wide d tiles per wave
  static constexpr int LD = D + 8;                          // K and Q LDS row stride (elements)
  // V row stride: 16 dwords past a multiple of 64 banks. A transposed read
  // takes, per group of 16 lanes, 4 keys x 4 8-byte chunks (keys 16 banks
  // apart, so the 16 lanes hit distinct banks), and the two groups of a
  // 32-lane half, 16 head dims apart, fall into the other 8 banks of each key's
  // 16 (with 8 dwords past, the second group met the next key's banks).
  static constexpr int LDV = 128 * ((D - 16 + 127) / 128) + 32;
  static constexpr int UPK = KV8 ? D / 16 : D / 8;         // 16-byte units per key row
  static constexpr int UNITS = kTileKeys * UPK;             // 16-byte units per K (or V) tile
  static constexpr int PER_THREAD = (UNITS + kThreads - 1) / kThreads;
  // One row tile: every wave holds the whole of Q (D/4 registers per lane) as
  // the B operand of S, instead of reading it from LDS on every tile.
  static constexpr bool QREG = RT == 1;
  static constexpr int Q_LDS = QREG ? 1 : RT * 32 * LD;         // elements
  static constexpr int KV_LDS = kTileKeys * (LD + LDV);          // elements per K/V tile pair
  // Two K/V buffers (the next tile is written while the current one is read,
  // one barrier per tile) where they fit: two workgroups per compute unit
  // within 80 KB, or D = 256 with three or four row tiles (one per unit).
  static constexpr int LDS1 = 2 * (Q_LDS + KV_LDS);
  static constexpr int NBUF = (LDS1 + 2 * KV_LDS <= 80 * 1024 || (D >= 256 && RT >= 3)) ? 2 : 1;
};

// 16 codes and their (scale, bias) word -> 16 bf16 values s * q + b.
__device__ __forceinline__ void dequant16(const u32x4 w, uint32_t sb, u32x4& lo, u32x4& hi) {
  const float s = __uint_as_float(sb << 16);
  const float b = __uint_as_float(sb & 0xFFFF0000u);
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t word = w[i >> 1];
    const int sh = 16 * (i & 1);
    const float f0 = __builtin_fmaf(s, (float)((word >> sh) & 0xFFu), b);
    const float f1 = __builtin_fmaf(s, (float)((word >> (sh + 8)) & 0xFFu), b);
    o[i] = pack_bf16x2(f0, f1);
  }
  lo = u32x4{o[0], o[1], o[2], o[3]};
  hi = u32x4{o[4], o[5], o[6], o[7]};
}

// Rows M and keys T of sequence b, its first query row r0; returns false for an
// empty sequence. Without batch arrays: the launch's M and T.
__device__ __forceinline__ bool seq_bounds(const AttnBatch& bt, int b, int M_max, int T_max, int& M, int& T, int& r0) {
  M = M_max;
  T = T_max;
  r0 = 0;
  if (!bt.row_start) return true;
  r0 = min(max(bt.row_start[b], 0), bt.total_rows);
  const int r1 = min(max(bt.row_start[b + 1], r0), bt.total_rows);
  M = min(r1 - r0, M_max);
  T = min(max(bt.seq_len[b], M), T_max);
  return M > 0;
}

template <int D, int RT, bool KV8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu((D >= 256 && RT >= 3) ? 1 : 2, 8))) void attn_partial_kernel(
    const uint16_t* __restrict__ q, int64_t q_rs, const uint16_t* kc, const uint16_t* vc, int64_t kv_head_stride,
    int M_max, int Hq, int Hkv, int T_max, float scale_log2, int keys_per_split, int splits, uint16_t* __restrict__ out,
    int64_t out_rs, uint16_t* __restrict__ part_o, float* __restrict__ part_ml, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, int64_t new_rs, uint16_t* kc_w, uint16_t* vc_w,
    const uint32_t* __restrict__ tree, const uint32_t* __restrict__ ksb, const uint32_t* __restrict__ vsb,
    const AttnBatch bt, int rows_stride) {
  using C = AttnCfg<D, RT, KV8>;
  const int b = blockIdx.z;
  int M, T, row0;
  if (!seq_bounds(bt, b, M_max, T_max, M, T, row0)) return;
  {
    // Sequence b's rows, cache and outputs (cache offsets in elements of the cache's type).
    const size_t cb = (size_t)b * bt.kv_batch_stride;
    q += (size_t)row0 * q_rs;
    out += (size_t)row0 * out_rs;
    if constexpr (KV8) {
      kc = reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(kc) + cb);
      vc = reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(vc) + cb);
      ksb += cb / 64;
      vsb += cb / 64;
    } else {
      kc += cb;
      vc += cb;
      if (kc_w) {
        kc_w += cb;
        vc_w += cb;
      }
    }
    if (k_new) {
      k_new += (size_t)row0 * new_rs;
      v_new += (size_t)row0 * new_rs;
    }
    if (tree) tree += row0;
  }
  __shared__ uint16_t q_lds[C::Q_LDS];
  __shared__ uint16_t k_lds[C::NBUF][kTileKeys * C::LD];
  __shared__ uint16_t v_lds[C::NBUF][kTileKeys * C::LDV];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kq = lane >> 5;
  const int l32 = lane & 31;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int G = Hq / Hkv;
  const int rows = M * G;
  const int j0 = split * keys_per_split;
  const int j1 = min(T, j0 + keys_per_split);

  // This lane's row and its word of the tree mask, then the query rows of
  // this KV head (row i = position i / G, head kvh*G + i % G), all loaded
  // before the first K/V tiles are fetched and waited for only after those
  // fetches are issued, so the ramp is one memory round trip, not two. Every
  // load goes out unconditionally: a row past the last one, and the mask word
  // without a mask, come from a zero vector (the pointer is chosen, never
  // dereferenced out of range; code that chooses between a loaded value and
  // another waits for every load in flight first). The mask word is used only
  // in masked tiles.
  const int rt = wave / C::DS;
  const int row = rt * 32 + l32;  // this lane's query row (softmax owner)
  const bool row_ok = row < rows;
  const int mpos = row_ok ? row / G : 0;
  const uint32_t tword = *(tree ? (const global_u32*)(tree + mpos) : (const global_u32*)kZero16);
  constexpr int kQPT = C::QREG ? 1 : RT * 32 * (D / 8) / kThreads;
  static_assert(C::QREG || kQPT * kThreads == RT * 32 * (D / 8), "query staging must be uniform");
  bf16x8 qr[C::QREG ? D / 16 : 1];
  u32x4 qv[kQPT];
  if constexpr (C::QREG) {
    // Lane l: row l % 32, head dims 16c + 8(l / 32) .. +7 of step c (the B
    // operand layout of S).
    const uint16_t* qrow = q + (size_t)(row / G) * q_rs + ((size_t)kvh * G + row % G) * D + 8 * kq;
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      qr[c] = *(row_ok ? (const global_bf16x8*)(qrow + 16 * c) : (const global_bf16x8*)kZero16);
  } else {
#pragma unroll
    for (int e = 0; e < kQPT; ++e) {
      const int u = tid + e * kThreads;
      const int i = u / (D / 8), dc = u % (D / 8);
      const uint16_t* src = q + (size_t)(i / G) * q_rs + ((size_t)kvh * G + i % G) * D + dc * 8;
      qv[e] = *(i < rows ? (const global_u32x4*)src : (const global_u32x4*)kZero16);
    }
  }
  // Called right after the first two fetches, ahead of the barrier before the
  // first tile.
  auto q_to_lds = [&]() __attribute__((always_inline)) {
    if constexpr (!C::QREG) {
#pragma unroll
      for (int e = 0; e < kQPT; ++e) {
        const int u = tid + e * kThreads;
        const int i = u / (D / 8), dc = u % (D / 8);
        *reinterpret_cast<u32x4*>(&q_lds[i * C::LD + dc * 8]) = qv[e];
      }
    }
  };

  const uint16_t* kh = kc + (size_t)kvh * kv_head_stride;
  const uint16_t* vh = vc + (size_t)kvh * kv_head_stride;
  // Two K/V tiles in flight (register sets 0 and 1). The loads are issued
  // unconditionally (key clamped into the range, values past it masked later),
  // so the wait counts the compiler derives stay exact.
  struct KV {
    u32x4 k[C::PER_THREAD], v[C::PER_THREAD];
    uint32_t ks[KV8 ? C::PER_THREAD : 1], vs[KV8 ? C::PER_THREAD : 1];
  };
  KV r0, r1;
  // K/V tiles are read once per call: with one or two row tiles the loads carry
  // the non-temporal hint (8 rows at 128k: 116 -> 105-110 us per call, 8-bit KV
  // 112.5 -> 109 us, 4 rows at 16k 24.0 -> 23.5 us); with three or four row
  // tiles (16 rows, a 16-node tree) the plain loads measured the same or faster.
  auto ld16 = [](const void* p) __attribute__((always_inline)) -> u32x4 {
    if constexpr (RT <= 2)
      return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    else
      return *reinterpret_cast<const u32x4*>(p);
  };
  // Keys below lim_plain are read from the cache itself (not from the rows
  // being appended). A tile wholly below it is one contiguous run per K and
  // V: thread t's unit e is 16-byte unit t + e * kThreads of the run, so its
  // address is one add, not the per-key clamp and source test of the general
  // fetch (those were about a quarter of the tile loop's vector instructions).
  const int lim_plain = k_new ? min(j1, T - M) : j1;
  auto fetch = [&](KV& r, int t0) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < C::PER_THREAD; ++e) {
      if constexpr (KV8) {
        const int u = min(tid + e * kThreads, C::UNITS - 1);
        const int key = min(t0 + u / C::UPK, j1 - 1);
        const int dc = u % C::UPK;
        const size_t row = (size_t)kvh * kv_head_stride + (size_t)key * D;  // codes (bytes) before the row
        r.k[e] = ld16(reinterpret_cast<const uint8_t*>(kc) + row + dc * 16);
        r.v[e] = ld16(reinterpret_cast<const uint8_t*>(vc) + row + dc * 16);
        r.ks[e] = ksb[row / 64 + dc / 4];
        r.vs[e] = vsb[row / 64 + dc / 4];
        continue;
      }
      const int u = tid + e * kThreads;
      const int key = min(t0 + u / (D / 8), j1 - 1);
      const int dc = u % (D / 8);
      const uint16_t* ks = kh + (size_t)key * D;
      const uint16_t* vs = vh + (size_t)key * D;
      if (k_new && key >= T - M) {  // a row being appended: read it from its source
        ks = k_new + (size_t)(key - (T - M)) * new_rs + (size_t)kvh * D;
        vs = v_new + (size_t)(key - (T - M)) * new_rs + (size_t)kvh * D;
      }
      r.k[e] = ld16(ks + dc * 8);
      r.v[e] = ld16(vs + dc * 8);
    }
  };
  auto fetch_plain = [&](KV& r, int t0) __attribute__((always_inline)) {
    if constexpr (C::UNITS % kThreads != 0) {
      fetch(r, t0);  // a tile that does not split into whole units per thread
    } else if constexpr (KV8) {
      const size_t base = (size_t)kvh * kv_head_stride + (size_t)t0 * D;  // bytes of codes
      const uint8_t* kt = reinterpret_cast<const uint8_t*>(kc) + base;
      const uint8_t* vt = reinterpret_cast<const uint8_t*>(vc) + base;
#pragma unroll
      for (int e = 0; e < C::PER_THREAD; ++e) {
        const int u = tid + e * kThreads;
        r.k[e] = ld16(kt + (size_t)u * 16);
        r.v[e] = ld16(vt + (size_t)u * 16);
        r.ks[e] = ksb[base / 64 + u / 4];
        r.vs[e] = vsb[base / 64 + u / 4];
      }
    } else {
      const uint16_t* kt = kh + (size_t)t0 * D;
      const uint16_t* vt = vh + (size_t)t0 * D;
#pragma unroll
      for (int e = 0; e < C::PER_THREAD; ++e) {
        const int u = tid + e * kThreads;
        r.k[e] = ld16(kt + (size_t)u * 8);
        r.v[e] = ld16(vt + (size_t)u * 8);
      }
    }
  };
  // Write a fetched tile into K/V buffer `buf` (8-bit codes dequantized here).
  auto put = [&](const KV& r, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < C::PER_THREAD; ++e) {
      if constexpr (KV8) {
        const int u = tid + e * kThreads;
        if (C::UNITS % kThreads == 0 || u < C::UNITS) {  // a test only where the tile is not whole units per thread
          const int key = u / C::UPK;
          const int dc = u % C::UPK;
          u32x4 lo, hi;
          dequant16(r.k[e], r.ks[e], lo, hi);
          *reinterpret_cast<u32x4*>(&k_lds[buf][key * C::LD + dc * 16]) = lo;
          *reinterpret_cast<u32x4*>(&k_lds[buf][key * C::LD + dc * 16 + 8]) = hi;
          dequant16(r.v[e], r.vs[e], lo, hi);
          *reinterpret_cast<u32x4*>(&v_lds[buf][key * C::LDV + dc * 16]) = lo;
          *reinterpret_cast<u32x4*>(&v_lds[buf][key * C::LDV + dc * 16 + 8]) = hi;
        }
        continue;
      }
      const int u = tid + e * kThreads;
      const int key = u / (D / 8);
      const int dc = u % (D / 8);
      *reinterpret_cast<u32x4*>(&k_lds[buf][key * C::LD + dc * 8]) = r.k[e];
      *reinterpret_cast<u32x4*>(&v_lds[buf][key * C::LDV + dc * 8]) = r.v[e];
    }
  };
  // With one buffer: wait until every wave is done with the tile in it, write
  // the next one, wait until every wave can see it.
  auto stage = [&](const KV& r) __attribute__((always_inline)) {
    __syncthreads();
    put(r, 0);
    __syncthreads();
  };

  const int dpart = wave % C::DS;
  const bool active = wave < RT * C::DS;
  const bool causal = tree == nullptr;
  const int t_new = T - M;  // first drafted key

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[C::DT];
#pragma unroll
  for (int t = 0; t < C::DT; ++t) o[t] = f32x16{};

  auto tile = [&](int t0, int buf) __attribute__((always_inline)) {
    if (!active) return;

    // S^T[key][row] = sum_d K[key][d] Q[row][d]
    f32x16 s = {};
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&k_lds[buf][l32 * C::LD + 16 * i + 8 * kq]);
      bf16x8 b;
      if constexpr (C::QREG)
        b = qr[i];
      else
        b = *reinterpret_cast<const bf16x8*>(&q_lds[row * C::LD + 16 * i + 8 * kq]);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, s, 0, 0, 0);
    }
    // Scale and mask, for this lane's row (keys split between lanes l, l^32). A
    // tile wholly inside the committed keys of the range (all but the last one
    // or two of a call) needs no mask; the masked form is branch-free.
    float mx = -INFINITY;
    if (t0 + kTileKeys <= min(j1, t_new)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] *= scale_log2;
        mx = fmaxf(mx, s[r]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = t0 + 8 * (r >> 2) + 4 * kq + (r & 3);
        const int jr = j - t_new;
        // Drafted key T-M+t is seen by row position i if t == i, if bit t of
        // the row's mask word is set, or (without a mask) if t < i.
        const uint32_t vis = (uint32_t)(j < j1) & ((uint32_t)(jr < 0) | (uint32_t)(jr == mpos) |
                                                   (uint32_t)(causal & (jr < mpos)) | ((tword >> (jr & 31)) & 1u));
        s[r] = vis ? s[r] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, s[r]);
      }
    }
    {
      const LanePair p = xor32_pair(mx);  // the row's other 16 keys are in lane l ^ 32
      mx = fmaxf(p.a, p.b);
    }
    // Online softmax with a lazily moved reference: m_run changes only when some
    // row's maximum exceeds it by more than 8 (or at a row's first visible key),
    // so the probabilities exp2(s - m_run) stay below 2^8 and the rescale of O
    // (a pass through the accumulation registers) is skipped on most tiles.
    // O and the sum l use the same reference, so O / l is the same softmax.
    const bool rescale = __ballot(mx > m_run + 8.f) != 0ull;
    float alpha = 1.f;
    if (rescale) {
      const float m_new = fmaxf(m_run, mx);
      alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = __builtin_amdgcn_exp2f(s[r] - m_use);
      psum += s[r];
    }
    {
      const LanePair p = xor32_pair(psum);  // a + b == b + a: both lanes get the same sum
      psum = p.a + p.b;
    }
    l_run = l_run * alpha + psum;
    u32x4 pw0, pw1;
    pw0[0] = pack_bf16x2(s[0], s[1]);
    pw0[1] = pack_bf16x2(s[2], s[3]);
    pw0[2] = pack_bf16x2(s[4], s[5]);
    pw0[3] = pack_bf16x2(s[6], s[7]);
    pw1[0] = pack_bf16x2(s[8], s[9]);
    pw1[1] = pack_bf16x2(s[10], s[11]);
    pw1[2] = pack_bf16x2(s[12], s[13]);
    pw1[3] = pack_bf16x2(s[14], s[15]);
    const bf16x8 pb0 = __builtin_bit_cast(bf16x8, pw0);
    const bf16x8 pb1 = __builtin_bit_cast(bf16x8, pw1);

    // O^T[d][row] += sum_key V[key][d] P[row][key]. For MFMA c, element j of
    // this lane covers key 16c + 8*(j/4) + 4*kq + j%4, matching P's layout. The
    // A operand (V^T: lane = head dim, elements = keys) comes from two transposed
    // LDS reads: in each group of 16 lanes, lane s points at key kb + s/4 and
    // head dims d0 + 4*(s%4) .. +3, and lane i receives keys kb .. kb+3 of head
    // dim d0 + i.
    const int tg = lane & 15;
    const int dh = (lane >> 4) & 1;
#pragma unroll
    for (int t = 0; t < C::DT; ++t) {
      if (rescale) {
#pragma unroll
        for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
      }
      const int dcol = dpart * C::DW + t * 32 + 16 * dh + 4 * (tg & 3);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int kb = 16 * c + 4 * kq + (tg >> 2);
        const v4i16 lo = ds_read_tr16(&v_lds[buf][kb * C::LDV + dcol]);
        const v4i16 hi = ds_read_tr16(&v_lds[buf][(kb + 8) * C::LDV + dcol]);
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, c ? pb1 : pb0, o[t], 0, 0, 0);
      }
    }
  };
  static_assert(KV8 || C::UNITS % kThreads == 0, "every thread moves whole 16-byte units of a tile");
  // While enough whole tiles of plain cache rows remain, the fetches go out
  // unconditionally, so the compiler's wait counts stay exact and two tiles
  // stay in flight across each staging; a fetch under a run-time test makes it
  // wait for every load in flight. The last tiles (plus the one holding
  // appended rows) and short ranges take the tested loop.
  int t0 = j0;
  if constexpr (C::NBUF == 2) {
    // At the top of each pair: buffer 0 holds tile t0 (visible to all waves),
    // r1 tile t0 + 32 and r0 tile t0 + 64 (in flight). A buffer is rewritten
    // only after the barrier that follows the last reads of it.
    if (j0 + 5 * kTileKeys <= lim_plain) {
      fetch_plain(r0, j0);
      fetch_plain(r1, j0 + kTileKeys);
      q_to_lds();
      put(r0, 0);
      fetch_plain(r0, j0 + 2 * kTileKeys);
      __syncthreads();
      do {
        tile(t0, 0);
        put(r1, 1);
        fetch_plain(r1, t0 + 3 * kTileKeys);
        __syncthreads();
        tile(t0 + kTileKeys, 1);
        put(r0, 0);
        fetch_plain(r0, t0 + 4 * kTileKeys);
        __syncthreads();
        t0 += 2 * kTileKeys;
      } while (t0 + 5 * kTileKeys <= lim_plain);
    } else if (j0 < j1) {
      fetch(r0, j0);
      if (j0 + kTileKeys < j1) fetch(r1, j0 + kTileKeys);
      q_to_lds();
      put(r0, 0);
      if (j0 + 2 * kTileKeys < j1) fetch(r0, j0 + 2 * kTileKeys);
      __syncthreads();
    }
    while (t0 < j1) {
      tile(t0, 0);
      if (t0 + kTileKeys >= j1) break;
      put(r1, 1);
      if (t0 + 3 * kTileKeys < j1) fetch(r1, t0 + 3 * kTileKeys);
      __syncthreads();
      tile(t0 + kTileKeys, 1);
      if (t0 + 2 * kTileKeys >= j1) break;
      put(r0, 0);
      if (t0 + 4 * kTileKeys < j1) fetch(r0, t0 + 4 * kTileKeys);
      __syncthreads();
      t0 += 2 * kTileKeys;
    }
  } else {
    if (j0 + 4 * kTileKeys <= lim_plain) {
      fetch_plain(r0, j0);
      fetch_plain(r1, j0 + kTileKeys);
      q_to_lds();
      do {
        stage(r0);
        fetch_plain(r0, t0 + 2 * kTileKeys);
        tile(t0, 0);
        stage(r1);
        fetch_plain(r1, t0 + 3 * kTileKeys);
        tile(t0 + kTileKeys, 0);
        t0 += 2 * kTileKeys;
      } while (t0 + 4 * kTileKeys <= lim_plain);
    } else {
      if (j0 < j1) fetch(r0, j0);
      if (j0 + kTileKeys < j1) fetch(r1, j0 + kTileKeys);
      q_to_lds();
    }
    for (; t0 < j1; t0 += 2 * kTileKeys) {
      stage(r0);
      if (t0 + 2 * kTileKeys < j1) fetch(r0, t0 + 2 * kTileKeys);
      tile(t0, 0);
      if (t0 + kTileKeys < j1) {
        stage(r1);
        if (t0 + 3 * kTileKeys < j1) fetch(r1, t0 + 3 * kTileKeys);
        tile(t0 + kTileKeys, 0);
      }
    }
  }

  // Append: the rows T-M .. T-1 that fall in this key range are copied from
  // their source into the caches (every row is in exactly one range; the
  // tiles read those rows from the source, so the copy can come last).
  if (k_new) {
    const int a0 = max(j0, T - M), a1 = j1;
    for (int u = tid; u < (a1 - a0) * (D / 8); u += kThreads) {
      const int key = a0 + u / (D / 8);
      const int dc = u % (D / 8);
      const size_t src = (size_t)(key - (T - M)) * new_rs + (size_t)kvh * D + dc * 8;
      const size_t dst = (size_t)kvh * kv_head_stride + (size_t)key * D + dc * 8;
      *reinterpret_cast<u32x4*>(kc_w + dst) = *reinterpret_cast<const u32x4*>(k_new + src);
      *reinterpret_cast<u32x4*>(vc_w + dst) = *reinterpret_cast<const u32x4*>(v_new + src);
    }
  }
  if (!active || !row_ok) return;
  const int g = row % G;
  const int h = kvh * G + g;
  if (splits == 1) {
    const float inv = 1.f / l_run;
#pragma unroll
    for (int t = 0; t < C::DT; ++t) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d = dpart * C::DW + t * 32 + 8 * a4 + 4 * kq;
        uint2 w;
        w.x = pack_bf16x2(o[t][4 * a4] * inv, o[t][4 * a4 + 1] * inv);
        w.y = pack_bf16x2(o[t][4 * a4 + 2] * inv, o[t][4 * a4 + 3] * inv);
        *reinterpret_cast<uint2*>(out + (size_t)mpos * out_rs + (size_t)h * D + d) = w;
      }
    }
    return;
  }
  // The range's output normalised by its own sum, o / l (a convex combination
  // of value rows, so no larger than the largest of them), rounded to bf16;
  // the combine weighs it by l and the range maximum. A range with no visible
  // key (l = 0) stores zeros and gets weight 0.
  const size_t prow = (((size_t)split * gridDim.z + b) * Hkv + kvh) * rows_stride + row;
  uint16_t* po = part_o + prow * D;
  const float inv_l = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
  for (int t = 0; t < C::DT; ++t) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int d = dpart * C::DW + t * 32 + 8 * a4 + 4 * kq;
      uint2 w;
      w.x = pack_bf16x2(o[t][4 * a4] * inv_l, o[t][4 * a4 + 1] * inv_l);
      w.y = pack_bf16x2(o[t][4 * a4 + 2] * inv_l, o[t][4 * a4 + 3] * inv_l);
      *reinterpret_cast<uint2*>(po + d) = w;
    }
  }
  if (dpart == 0 && kq == 0) {
    float* pml = part_ml + prow * 2;
    pml[0] = m_run;
    pml[1] = l_run;
  }
}

// Merge the per-range partials of one (query row, KV head, 64 head dims): with
// range r's maximum m_r, sum l_r and normalised output o_r / l_r,
//   out = sum_r exp2(m_r - m) l_r (o_r / l_r) / sum_r exp2(m_r - m) l_r.
// 256 threads = 16 groups of 16 lanes; lane i of a group owns head dims
// 4i..4i+3 of the block's 64 and group g sums the ranges g, g+16, ...; the
// groups' sums are added in LDS in a fixed order (deterministic).
constexpr int kCombineGroups = 16;
constexpr int kMaxSplits = 1024;

__global__ __launch_bounds__(256) void attn_combine_kernel(
    const uint16_t* __restrict__ part_o, const float* __restrict__ part_ml, int M_max, int Hq, int Hkv, int D,
    int splits, uint16_t* __restrict__ out, int64_t out_rs, const AttnBatch bt, int rows_stride, int T_max) {
  __shared__ float w_lds[kMaxSplits];
  __shared__ float red[256 / 64];
  __shared__ float4 acc_lds[kCombineGroups][16];
  const int row = blockIdx.x;
  const int kvh = blockIdx.y;
  const int nd = D / 64;
  const int b = blockIdx.z / nd;
  const int d0 = (blockIdx.z % nd) * 64;
  const int tid = threadIdx.x;
  const int G = Hq / Hkv;
  int M, T, r0;
  if (!seq_bounds(bt, b, M_max, T_max, M, T, r0) || row >= M * G) return;
  out += (size_t)r0 * out_rs;
  const int nb = gridDim.z / nd;
  const size_t s_stride = (size_t)nb * Hkv * rows_stride;  // partial rows between consecutive ranges
  const size_t base = ((size_t)b * Hkv + kvh) * rows_stride + row;
  // The first batch of partial O rows (ranges grp, grp+16, ..., grp+112: all
  // of them up to 128 ranges) and the (max, sum) pairs go out together; the
  // weights need only the pairs.
  constexpr int kFirst = 8;
  const int grp = tid >> 4;
  const int d = d0 + 4 * (tid & 15);
  const uint16_t* po = part_o + base * D + d;
  // Four bf16 partial values (8 bytes) widened to float.
  auto load4 = [&](int sp) __attribute__((always_inline)) -> float4 {
    const uint2 w = *reinterpret_cast<const uint2*>(po + sp * s_stride * D);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u), __uint_as_float(w.y << 16),
                       __uint_as_float(w.y & 0xFFFF0000u));
  };
  // Every load of this first batch is issued (range index clamped, values past
  // the last range unused): a load under a per-lane condition is followed by a
  // full wait in the compiled code, which made the batch one round trip per load.
  float4 v0[kFirst];
#pragma unroll
  for (int u = 0; u < kFirst; ++u) v0[u] = load4(min(grp + u * kCombineGroups, splits - 1));
  constexpr int kMLPT = kMaxSplits / 256;
  float2 ml[kMLPT];
#pragma unroll
  for (int k = 0; k < kMLPT; ++k) {
    const int sp = tid + 256 * k;
    const float2 x = *reinterpret_cast<const float2*>(part_ml + ((size_t)min(sp, splits - 1) * s_stride + base) * 2);
    ml[k] = sp < splits ? x : make_float2(-INFINITY, 0.f);
  }
  // Range weights exp2(m_s - max) * l_s and the merged denominator (their sum).
  float mloc = -INFINITY;
#pragma unroll
  for (int k = 0; k < kMLPT; ++k) mloc = fmaxf(mloc, ml[k].x);
  mloc = max64_lanes(mloc);
  if ((tid & 63) == 0) red[tid >> 6] = mloc;
  __syncthreads();
  const float mmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float dloc = 0.f;
#pragma unroll
  for (int k = 0; k < kMLPT; ++k) {
    const int sp = tid + 256 * k;
    if (sp < splits) {
      const float w = ml[k].x == -INFINITY ? 0.f : exp2f(ml[k].x - mmax) * ml[k].y;
      w_lds[sp] = w;
      dloc += w;
    }
  }
  dloc = sum64_lanes(dloc);
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = dloc;
  __syncthreads();
  const float den = (red[0] + red[1]) + (red[2] + red[3]);
  // Weighted sum of the partial O rows, in range order per group.
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int u = 0; u < kFirst; ++u) {
    const int sp = grp + u * kCombineGroups;
    if (sp < splits) {
      const float w = w_lds[sp];
      acc.x += w * v0[u].x;
      acc.y += w * v0[u].y;
      acc.z += w * v0[u].z;
      acc.w += w * v0[u].w;
    }
  }
  int s = grp + kFirst * kCombineGroups;
  for (; s + 3 * kCombineGroups < splits; s += 4 * kCombineGroups) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = load4(s + u * kCombineGroups);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float w = w_lds[s + u * kCombineGroups];
      acc.x += w * v[u].x;
      acc.y += w * v[u].y;
      acc.z += w * v[u].z;
      acc.w += w * v[u].w;
    }
  }
  for (; s < splits; s += kCombineGroups) {
    const float4 v = load4(s);
    const float w = w_lds[s];
    acc.x += w * v.x;
    acc.y += w * v.y;
    acc.z += w * v.z;
    acc.w += w * v.w;
  }
  acc_lds[grp][tid & 15] = acc;
  __syncthreads();
  if (tid < 16) {
    float4 t = acc_lds[0][tid];
    for (int g2 = 1; g2 < kCombineGroups; ++g2) {
      const float4 u = acc_lds[g2][tid];
      t.x += u.x;
      t.y += u.y;
      t.z += u.z;
      t.w += u.w;
    }
    const float inv = 1.f / den;
    const int m = row / G;
    const int h = kvh * G + row % G;
    uint2 o2;
    o2.x = pack_bf16x2(t.x * inv, t.y * inv);
    o2.y = pack_bf16x2(t.z * inv, t.w * inv);
    *reinterpret_cast<uint2*>(out + (size_t)m * out_rs + (size_t)h * D + d0 + 4 * tid) = o2;
  }
}

}  // namespace

AttnPlan attn_plan(int M, int Hq, int Hkv, int D, int T, int B) {
  AttnPlan p{};
  p.rows = M * (Hq / Hkv);
  p.row_tiles = (p.rows + 31) / 32;
  // One round of resident workgroups, at least 128 keys per range. At D = 256
  // with three or four row tiles a lane needs about 380 registers, so one
  // workgroup fits per compute unit; otherwise two do.
  const int tiles = (T + kTileKeys - 1) / kTileKeys;
  // Below 64k keys one workgroup per compute unit also wins (fewer, longer ranges:
  // fewer partials to store and combine): 8k x 1 row 19.9 -> 18.0 us, 16k x 4
  // rows 26.0 -> 25.5 us, 32k x 8 rows 42.2 -> 41.2 us; at 128k two stay ahead.
  const int per_cu = ((D >= 256 && p.row_tiles >= 3) || T < 65536) ? 1 : 2;
  int s = (per_cu * kNumCU + Hkv * B - 1) / (Hkv * B);
  int max_s = (tiles + 3) / 4;
  s = s > max_s ? max_s : s;
  s = s < 1 ? 1 : s;
  const int tiles_per = (tiles + s - 1) / s;
  p.keys_per_split = tiles_per * kTileKeys;
  p.splits = (T + p.keys_per_split - 1) / p.keys_per_split;
  p.partial_bytes =
      p.splits > 1 ? align_up((size_t)p.splits * B * Hkv * p.rows * (D * sizeof(uint16_t) + 2 * sizeof(float)), 256)
                   : 0;
  return p;
}

hipError_t attn_launch(const AttnPlan& plan, const void* q, int64_t q_rs, const void* k, const void* v,
                       int64_t kv_head_stride, int M, int Hq, int Hkv, int D, int T, float scale,
                       void* out, int64_t out_rs, void* workspace, hipStream_t stream, const void* k_new,
                       const void* v_new, int64_t new_rs, const uint32_t* tree, const uint32_t* k_sb,
                       const uint32_t* v_sb, const AttnBatch* batch) {
  const AttnBatch bt = batch ? *batch : AttnBatch{nullptr, nullptr, 0, 0, 1};
  auto* kn = reinterpret_cast<const uint16_t*>(k_new);
  auto* vn = reinterpret_cast<const uint16_t*>(v_new);
  // With an append the caches are written (rows T-M .. T-1) as well as read.
  auto* kw = k_new ? const_cast<uint16_t*>(reinterpret_cast<const uint16_t*>(k)) : nullptr;
  auto* vw = k_new ? const_cast<uint16_t*>(reinterpret_cast<const uint16_t*>(v)) : nullptr;
  uint16_t* part_o = reinterpret_cast<uint16_t*>(workspace);
  float* part_ml = plan.splits > 1
                       ? reinterpret_cast<float*>(part_o + (size_t)plan.splits * bt.B * Hkv * plan.rows * D)
                       : nullptr;
  dim3 grid(plan.splits, Hkv, bt.B);
  auto* qp = reinterpret_cast<const uint16_t*>(q);
  auto* kp = reinterpret_cast<const uint16_t*>(k);
  auto* vp = reinterpret_cast<const uint16_t*>(v);
  auto* op = reinterpret_cast<uint16_t*>(out);
  const float sl2 = scale * kLog2e;
  const bool kv8 = k_sb != nullptr;
#define VQ_ATTN(DV, RTV)                                                                                     \
  if (kv8)                                                                                                   \
    hipLaunchKernelGGL((attn_partial_kernel<DV, RTV, true>), grid, dim3(kThreads), 0, stream, qp, q_rs, kp, vp, \
                       kv_head_stride, M, Hq, Hkv, T, sl2, plan.keys_per_split, plan.splits, op, out_rs, part_o,  \
                       part_ml, kn, vn, new_rs, kw, vw, tree, k_sb, v_sb, bt, plan.rows);                        \
  else                                                                                                       \
    hipLaunchKernelGGL((attn_partial_kernel<DV, RTV, false>), grid, dim3(kThreads), 0, stream, qp, q_rs, kp, vp, \
                       kv_head_stride, M, Hq, Hkv, T, sl2, plan.keys_per_split, plan.splits, op, out_rs, part_o,   \
                       part_ml, kn, vn, new_rs, kw, vw, tree, nullptr, nullptr, bt, plan.rows)
#define VQ_ATTN_RT(DV)                         \
  switch (plan.row_tiles) {                    \
    case 1: VQ_ATTN(DV, 1); break;             \
    case 2: VQ_ATTN(DV, 2); break;             \
    case 3: VQ_ATTN(DV, 3); break;             \
    default: VQ_ATTN(DV, 4); break;            \
  }
  if (D == 64) {
    VQ_ATTN_RT(64)
  } else if (D == 128) {
    VQ_ATTN_RT(128)
  } else {
    VQ_ATTN_RT(256)
  }
#undef VQ_ATTN_RT
#undef VQ_ATTN
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(plan.rows, Hkv, (D / 64) * bt.B), dim3(256), 0, stream,
                     part_o, part_ml, M, Hq, Hkv, D, plan.splits, op, out_rs, bt, plan.rows, T);
  return hipGetLastError();
}


namespace {

// One wave per (row m, KV head h, group g of 64): the keys, then the values.
__global__ __launch_bounds__(256) void kv8_append_kernel(const uint16_t* __restrict__ src, int64_t ld, int k_off,
                                                         int v_off, uint8_t* __restrict__ kq, uint32_t* __restrict__ ks,
                                                         uint8_t* __restrict__ vq, uint32_t* __restrict__ vs,
                                                         int64_t hs, int M, int Hkv, int D, int pos) {
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int groups = D / 64;
  if (w >= M * Hkv * groups) return;
  const int m = w / (Hkv * groups);
  const int h = (w / groups) % Hkv;
  const int g = w % groups;
  const size_t row = (size_t)h * hs + (size_t)(pos + m) * D;  // codes before the cache row
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    const uint16_t* x16 = src + (int64_t)m * ld + (kv ? v_off : k_off) + h * D + g * 64;
    const float x = __uint_as_float((uint32_t)x16[lane] << 16);
    float mn = x, mx = x;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      mn = fminf(mn, __shfl_xor(mn, off));
      mx = fmaxf(mx, __shfl_xor(mx, off));
    }
    const float scale = __fdiv_rn(__fsub_rn(mx, mn), 255.f);
    uint32_t code = 0;
    if (scale != 0.f) code = (uint32_t)fminf(fmaxf(rintf(__fdiv_rn(__fsub_rn(x, mn), scale)), 0.f), 255.f);
    (kv ? vq : kq)[row + g * 64 + lane] = (uint8_t)code;
    if (lane == 0) (kv ? vs : ks)[row / 64 + g] = (uint32_t)f32_to_bf16_rne(scale) | ((uint32_t)f32_to_bf16_rne(mn) << 16);
  }
}

}  // namespace

hipError_t kv8_append(const void* src, int64_t ld, int k_off, int v_off, void* k_codes, void* k_sb, void* v_codes,
                      void* v_sb, int64_t hs, int M, int Hkv, int D, int pos, hipStream_t stream) {
  const int waves = M * Hkv * (D / 64);
  hipLaunchKernelGGL(kv8_append_kernel, dim3((waves + 3) / 4), dim3(256), 0, stream,
                     reinterpret_cast<const uint16_t*>(src), ld, k_off, v_off, reinterpret_cast<uint8_t*>(k_codes),
                     reinterpret_cast<uint32_t*>(k_sb), reinterpret_cast<uint8_t*>(v_codes),
                     reinterpret_cast<uint32_t*>(v_sb), hs, M, Hkv, D, pos);
  return hipGetLastError();
}
}  // namespace vq
