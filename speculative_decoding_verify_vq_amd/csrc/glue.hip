// Element-wise kernels of the dense verify stack (RMSNorm, SwiGLU, residual
// add, KV append). bf16 in and out, float32 arithmetic, RNE stores.
#include <math.h>

#include "vq_internal.h"

namespace vq {
namespace {

__device__ __forceinline__ float bf(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t to_bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                      uint16_t* __restrict__ y, int64_t ldy, int N,
                                                      float eps) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  const uint16_t* xr = x + (int64_t)m * ldx;
  float ss = 0.f;
  for (int i = threadIdx.x; i < N; i += 256) {
    const float v = bf(xr[i]);
    ss += v * v;
  }
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float r = 1.f / sqrtf(tot / (float)N + eps);
  uint16_t* yr = y + (int64_t)m * ldy;
  for (int i = threadIdx.x; i < N; i += 256) yr[i] = to_bf(bf(xr[i]) * r);
}

__global__ __launch_bounds__(256) void add_kernel(const uint16_t* a, const uint16_t* b, uint16_t* y,
                                                  int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    y[i] = to_bf(bf(a[i]) + bf(b[i]));
}

__global__ __launch_bounds__(256) void silu_mul_kernel(const uint16_t* __restrict__ gu, int64_t ldgu,
                                                       uint16_t* __restrict__ y, int64_t ldy, int I) {
  const int m = blockIdx.y;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < I; i += gridDim.x * 256) {
    const float g = bf(gu[(int64_t)m * ldgu + i]);
    const float u = bf(gu[(int64_t)m * ldgu + I + i]);
    y[(int64_t)m * ldy + i] = to_bf(g / (1.f + expf(-g)) * u);
  }
}

__global__ __launch_bounds__(256) void kv_append_kernel(const uint16_t* __restrict__ src, int64_t ld,
                                                        int k_off, int v_off, uint16_t* __restrict__ kc,
                                                        uint16_t* __restrict__ vc, int64_t hs, int M,
                                                        int Hkv, int D, int pos) {
  const int units = D / 8;
  const int total = M * Hkv * units;
  for (int t = blockIdx.x * 256 + threadIdx.x; t < total; t += gridDim.x * 256) {
    const int m = t / (Hkv * units);
    const int h = (t / units) % Hkv;
    const int u = t % units;
    const uint16_t* s = src + (int64_t)m * ld;
    *reinterpret_cast<uint4*>(kc + h * hs + (int64_t)(pos + m) * D + u * 8) =
        *reinterpret_cast<const uint4*>(s + k_off + h * D + u * 8);
    *reinterpret_cast<uint4*>(vc + h * hs + (int64_t)(pos + m) * D + u * 8) =
        *reinterpret_cast<const uint4*>(s + v_off + h * D + u * 8);
  }
}

}  // namespace

hipError_t glue_rmsnorm(const void* x, int64_t ldx, void* y, int64_t ldy, int M, int N, float eps,
                        hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(M), dim3(256), 0, s, (const uint16_t*)x, ldx, (uint16_t*)y, ldy, N,
                     eps);
  return hipGetLastError();
}

hipError_t glue_add(const void* a, const void* b, void* y, int64_t n, hipStream_t s) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(add_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const uint16_t*)a, (const uint16_t*)b,
                     (uint16_t*)y, n);
  return hipGetLastError();
}

hipError_t glue_silu_mul(const void* gu, int64_t ldgu, void* y, int64_t ldy, int M, int I, hipStream_t s) {
  int bx = (I + 255) / 256;
  if (bx > 1024) bx = 1024;
  hipLaunchKernelGGL(silu_mul_kernel, dim3(bx, M), dim3(256), 0, s, (const uint16_t*)gu, ldgu, (uint16_t*)y,
                     ldy, I);
  return hipGetLastError();
}

hipError_t glue_kv_append(const void* src, int64_t ld, int k_off, int v_off, void* kc, void* vc, int64_t hs,
                          int M, int Hkv, int D, int pos, hipStream_t s) {
  const int total = M * Hkv * (D / 8);
  int blocks = (total + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(kv_append_kernel, dim3(blocks), dim3(256), 0, s, (const uint16_t*)src, ld, k_off, v_off,
                     (uint16_t*)kc, (uint16_t*)vc, hs, M, Hkv, D, pos);
  return hipGetLastError();
}

}  // namespace vq
