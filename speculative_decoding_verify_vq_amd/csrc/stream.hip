// Streaming-read ceiling of the HBM, gfx950: the rate at which a plain kernel
// reads a large buffer with coalesced 16-byte loads. The verify pass is a
// memory-bandwidth problem (page "The fastest way to run local LLMs on a Mac",
// section "Decode is a memory-bandwidth problem"), so this rate, not the
// nominal 8 TB/s alone, is what the pass's kernels are compared with.
#include "vq_internal.h"

namespace vq {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 4;  // 16-byte loads in flight per thread

template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  return *p;
}

// Workgroup w reads 16 KiB blocks w, w + grid, w + 2 grid, ... (each thread
// four 16-byte units of a block, one block in flight per iteration) and folds
// them into one word that it stores, so no load can be dropped.
template <bool NT>
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                                     uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t block = (int64_t)kStreamThreads * kStreamUnroll;
  for (int64_t base = (int64_t)blockIdx.x * block + threadIdx.x; base < n16; base += (int64_t)gridDim.x * block) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const int64_t i = base + (int64_t)u * kStreamThreads;
      v[u] = i < n16 ? load16<NT>(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) sink[(int64_t)blockIdx.x * (kStreamThreads / 64) + (threadIdx.x >> 6)] = acc;
}

}  // namespace

hipError_t stream_read_launch(const void* src, size_t bytes, bool nontemporal, int workgroups, uint32_t* sink,
                              hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  const u32x4* p = reinterpret_cast<const u32x4*>(src);
  if (nontemporal)
    hipLaunchKernelGGL(stream_read_kernel<true>, dim3(workgroups), dim3(kStreamThreads), 0, stream, p, n16, sink);
  else
    hipLaunchKernelGGL(stream_read_kernel<false>, dim3(workgroups), dim3(kStreamThreads), 0, stream, p, n16, sink);
  return hipGetLastError();
}

}  // namespace vq
