// Host side of the C ABI: argument validation, workspace sizing, dispatch and
// error reporting. Every check runs before any HIP call, so an invalid call
// returns VQ_ERR_INVALID_ARG without touching the device.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "vq.h"
#include "vq_bench.h"
#include "vq_glue.h"
#include "vq_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  snprintf(g_err, sizeof(g_err), "%s: %s", what, hipGetErrorString(e));
  return VQ_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Per-device result of the architecture check: 0 unknown, 1 gfx950, 2 other.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

int check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(VQ_ERR_UNSUPPORTED_DEVICE, "device index %d out of range", dev);
  int st = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(st, std::memory_order_relaxed);
    if (st == 2) return fail(VQ_ERR_UNSUPPORTED_DEVICE, "device %d is %s; this library is built for gfx950 only", dev,
                             prop.gcnArchName);
  }
  if (st == 2) return fail(VQ_ERR_UNSUPPORTED_DEVICE, "device %d is not gfx950", dev);
  return VQ_OK;
}

int check_workspace(void* ws, size_t have, size_t need) {
  if (need == 0) return VQ_OK;
  if (ws == nullptr) return fail(VQ_ERR_INVALID_ARG, "workspace is NULL but %zu bytes are needed", need);
  if (!aligned(ws, 256)) return fail(VQ_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (have < need) return fail(VQ_ERR_INVALID_ARG, "workspace has %zu bytes, %zu needed", have, need);
  return VQ_OK;
}

bool qmm_shape_ok(int bits, int group_size, int M, int N, int K) {
  return (bits == 4 || bits == 8) && group_size == 64 && M >= 1 && M <= VQ_MAX_ROWS && N >= 1 && K >= 64 &&
         K % 64 == 0 && N <= (1 << 20) && K <= (1 << 24);
}

bool attn_shape_ok(int M, int Hq, int Hkv, int D, int T) {
  return M >= 1 && M <= VQ_MAX_ROWS && Hkv >= 1 && Hkv <= 65535 && Hq >= Hkv && Hq % Hkv == 0 &&
         (Hq / Hkv) * M <= 128 && (D == 64 || D == 128 || D == 256) && T >= M && T <= (1 << 26);
}

bool accept_shape_ok(int B, int K, int V, int input_kind, int64_t ps, int64_t qs) {
  if (B < 1 || K < 0 || K > VQ_MAX_DRAFTS || V < 2 || V > VQ_MAX_VOCAB) return false;
  if (input_kind != VQ_PROBS && input_kind != VQ_LOGITS) return false;
  if (ps < 0 || qs < 0) return false;
  if (ps != 0 && ps < (int64_t)(K + 1) * V) return false;
  if (qs != 0 && qs < (int64_t)K * V) return false;
  const bool shared = ps == 0 && qs == 0;
  if (!shared && B > 65535) return false;
  return true;
}

}  // namespace

extern "C" {

const char* vq_status_string(int status) {
  switch (status) {
    case VQ_OK: return "ok";
    case VQ_ERR_INVALID_ARG: return "invalid argument";
    case VQ_ERR_HIP: return "HIP runtime error";
    case VQ_ERR_UNSUPPORTED_DEVICE: return "unsupported device";
    default: return "unknown status";
  }
}

const char* vq_last_error(void) { return g_err; }

const char* vq_version(void) { return "0.1.0"; }

// ------------------------------------------------------------------ QMM
size_t vq_skinny_qmm_workspace(int bits, int group_size, int M, int N, int K) {
  if (!qmm_shape_ok(bits, group_size, M, N, K)) return 0;
  const vq::QmmPlan p = vq::qmm_plan(bits, M, N, K, false);
  return p.counter_bytes + p.partial_bytes;
}

}  // extern "C"

namespace {

// The argument checks of the row-major skinny QMM (fn names the entry point).
int qmm_rowmajor_args(const char* fn, const void* x, int64_t ldx, const void* wq, const void* scales,
                      const void* biases, int bits, int group_size, int M, int N, int K, const void* y, int64_t ldy,
                      int y_dtype) {
  if (!x || !wq || !scales || !biases || !y) return fail(VQ_ERR_INVALID_ARG, "%s: NULL data pointer", fn);
  if (bits != 4 && bits != 8) return fail(VQ_ERR_INVALID_ARG, "%s: bits must be 4 or 8 (got %d)", fn, bits);
  if (group_size != 64) return fail(VQ_ERR_INVALID_ARG, "%s: group_size must be 64 (got %d)", fn, group_size);
  if (M < 1 || M > VQ_MAX_ROWS) return fail(VQ_ERR_INVALID_ARG, "%s: M must be in [1, 16] (got %d)", fn, M);
  if (!qmm_shape_ok(bits, group_size, M, N, K))
    return fail(VQ_ERR_INVALID_ARG, "%s: unsupported shape N=%d K=%d (K a positive multiple of 64)", fn, N, K);
  if (ldx < K || ldx % 8 != 0) return fail(VQ_ERR_INVALID_ARG, "%s: ldx must be >= K and a multiple of 8", fn);
  if (ldy < N) return fail(VQ_ERR_INVALID_ARG, "%s: ldy must be >= N", fn);
  if (y_dtype != VQ_BF16 && y_dtype != VQ_F32) return fail(VQ_ERR_INVALID_ARG, "%s: bad y_dtype %d", fn, y_dtype);
  if (!aligned(x, 16) || !aligned(wq, 16)) return fail(VQ_ERR_INVALID_ARG, "%s: x and wq must be 16-byte aligned", fn);
  if (!aligned(scales, 2) || !aligned(biases, 2) || !aligned(y, y_dtype == VQ_F32 ? 4 : 2))
    return fail(VQ_ERR_INVALID_ARG, "%s: misaligned scales, biases or y", fn);
  return VQ_OK;
}

vq::QmmCall qmm_rowmajor_call(const void* x, int64_t ldx, const void* wq, const void* scales, const void* biases,
                              int bits, int M, int N, int K, void* y, int64_t ldy, int y_dtype, void* workspace) {
  vq::QmmCall c{};
  c.x = x;
  c.ldx = ldx;
  c.wq = wq;
  c.scales = scales;
  c.biases = biases;
  c.tiled = false;
  c.bits = bits;
  c.M = M;
  c.N = N;
  c.K = K;
  c.epilogue = vq::kEpiStore;
  c.y = y;
  c.ldy = ldy;
  c.y_f32 = y_dtype == VQ_F32;
  c.workspace = workspace;
  return c;
}

}  // namespace

extern "C" {

int vq_skinny_qmm(const void* x, int64_t ldx, const void* wq, const void* scales, const void* biases, int bits,
                  int group_size, int M, int N, int K, void* y, int64_t ldy, int y_dtype, void* workspace,
                  size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  int rc = qmm_rowmajor_args("vq_skinny_qmm", x, ldx, wq, scales, biases, bits, group_size, M, N, K, y, ldy, y_dtype);
  if (rc) return rc;
  const vq::QmmPlan plan = vq::qmm_plan(bits, M, N, K, false);
  if ((rc = check_workspace(workspace, workspace_bytes, plan.counter_bytes + plan.partial_bytes))) return rc;
  if ((rc = check_device())) return rc;
  const vq::QmmCall c = qmm_rowmajor_call(x, ldx, wq, scales, biases, bits, M, N, K, y, ldy, y_dtype, workspace);
  hipError_t e = vq::qmm_launch(plan, c, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? VQ_OK : hip_fail(e, "vq_skinny_qmm launch");
}

}  // extern "C"

// ------------------------------------------------- the entry point without allocation
// The library's own scratch for vq_skinny_qmm_noalloc: one copy per GPU, held
// from the library's load until the process ends. In host code `scratch` only
// names the symbol; its device address on the current GPU is looked up once
// per device with hipGetSymbolAddress and used from then on.
static __device__ __align__(256) unsigned char scratch[VQ_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each GPU (null until looked up)

int scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(VQ_ERR_UNSUPPORTED_DEVICE, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(VQ_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return VQ_OK;
}

// Zeroes n 32-bit words (a fill kernel rather than a memset node, so that the
// call can be captured into a graph).
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* __restrict__ p, uint32_t n) {
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < n; i += gridDim.x * 256u) p[i] = 0u;
}

}  // namespace

extern "C" {

int vq_skinny_qmm_noalloc(const void* x, int64_t ldx, const void* wq, const void* scales, const void* biases,
                          int bits, int group_size, int M, int N, int K, void* y, int64_t ldy, int y_dtype,
                          void* stream) {
  g_err[0] = 0;
  int rc = qmm_rowmajor_args("vq_skinny_qmm_noalloc", x, ldx, wq, scales, biases, bits, group_size, M, N, K, y, ldy,
                             y_dtype);
  if (rc) return rc;
  const vq::QmmPlan plan = vq::qmm_plan(bits, M, N, K, false);
  const size_t need = plan.counter_bytes + plan.partial_bytes;
  if (need > VQ_NOALLOC_SCRATCH_BYTES)
    return fail(VQ_ERR_INVALID_ARG,
                "vq_skinny_qmm_noalloc: M=%d N=%d K=%d needs %zu bytes of scratch, more than the library's %zu "
                "(use vq_skinny_qmm with a workspace)", M, N, K, need, (size_t)VQ_NOALLOC_SCRATCH_BYTES);
  if ((rc = check_device())) return rc;
  void* ws = nullptr;
  if ((rc = scratch_of_current_device(&ws))) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (plan.counter_bytes) {
    // The completion counters start at zero on every call, whatever the last
    // call on this GPU left behind.
    const uint32_t words = (uint32_t)(plan.counter_bytes / 4);
    hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, s,
                       reinterpret_cast<uint32_t*>(ws), words);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "vq_skinny_qmm_noalloc clear");
  }
  const vq::QmmCall c = qmm_rowmajor_call(x, ldx, wq, scales, biases, bits, M, N, K, y, ldy, y_dtype, ws);
  hipError_t e = vq::qmm_launch(plan, c, s);
  return e == hipSuccess ? VQ_OK : hip_fail(e, "vq_skinny_qmm_noalloc launch");
}

size_t vq_qmm_pack_bytes(int bits, int group_size, int N, int K) {
  if (!qmm_shape_ok(bits, group_size, 1, N, K)) return 0;
  return vq::qmm_pack_bytes(bits, N, K);
}

int vq_qmm_pack(const void* wq, const void* scales, const void* biases, int bits, int group_size, int N, int K,
                void* packed, size_t packed_bytes, void* stream) {
  g_err[0] = 0;
  if (!wq || !scales || !biases || !packed) return fail(VQ_ERR_INVALID_ARG, "vq_qmm_pack: NULL pointer");
  if (!qmm_shape_ok(bits, group_size, 1, N, K))
    return fail(VQ_ERR_INVALID_ARG, "vq_qmm_pack: unsupported bits=%d group_size=%d N=%d K=%d", bits, group_size, N, K);
  if (!aligned(wq, 16) || !aligned(packed, 16) || !aligned(scales, 2) || !aligned(biases, 2))
    return fail(VQ_ERR_INVALID_ARG, "vq_qmm_pack: wq and packed must be 16-byte aligned");
  const size_t need = vq::qmm_pack_bytes(bits, N, K);
  if (packed_bytes < need) return fail(VQ_ERR_INVALID_ARG, "vq_qmm_pack: packed has %zu bytes, %zu needed", packed_bytes, need);
  int rc = check_device();
  if (rc) return rc;
  hipError_t e = vq::qmm_pack(wq, scales, biases, bits, N, K, packed, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? VQ_OK : hip_fail(e, "vq_qmm_pack launch");
}

size_t vq_qmm_packed_workspace(int bits, int group_size, int M, int N, int K) {
  if (!qmm_shape_ok(bits, group_size, M, N, K)) return 0;
  const vq::QmmPlan p = vq::qmm_plan(bits, M, N, K, true);
  return p.counter_bytes + p.partial_bytes;
}

int vq_sumsq_parts(int N) { return N >= 1 ? vq::qmm_sumsq_parts(N) : 0; }

int vq_qmm_packed(const void* x, int64_t ldx, const float* x_sumsq, int x_sumsq_parts, float eps, const void* packed,
                  int bits, int group_size, int M, int N, int K, int epilogue, const void* residual, int64_t ldr,
                  void* y, int64_t ldy, int y_dtype, float* y_sumsq, void* workspace, size_t workspace_bytes,
                  void* stream) {
  g_err[0] = 0;
  if (!x || !packed || !y) return fail(VQ_ERR_INVALID_ARG, "vq_qmm_packed: NULL data pointer");
  if (!qmm_shape_ok(bits, group_size, M, N, K))
    return fail(VQ_ERR_INVALID_ARG, "vq_qmm_packed: unsupported bits=%d group_size=%d M=%d N=%d K=%d", bits,
                group_size, M, N, K);
  if (ldx < K || ldx % 8 != 0) return fail(VQ_ERR_INVALID_ARG, "vq_qmm_packed: ldx must be >= K and a multiple of 8");
  if (!aligned(x, 16) || !aligned(packed, 16))
    return fail(VQ_ERR_INVALID_ARG, "vq_qmm_packed: x and packed must be 16-byte aligned");
  if (x_sumsq) {
    if (x_sumsq_parts < 1 || x_sumsq_parts > 256)
      return fail(VQ_ERR_INVALID_ARG, "vq_qmm_packed: x_sumsq_parts must be in [1, 256] (got %d)", x_sumsq_parts);
    if (!(eps >= 0.f) || !isfinite(eps)) return fail(VQ_ERR_INVALID_ARG, "vq_qmm_packed: eps must be finite and >= 0");
    if (!aligned(x_sumsq, 4)) return fail(VQ_ERR_INVALID_ARG, "vq_qmm_packed: misaligned x_sumsq");
  }
  if (y_sumsq && epilogue != VQ_EPI_RESIDUAL)
    return fail(VQ_ERR_INVALID_ARG, "vq_qmm_packed: y_sumsq is produced by the residual epilogue only");
  if (y_sumsq && !aligned(y_sumsq, 4)) return fail(VQ_ERR_INVALID_ARG, "vq_qmm_packed: misaligned y_sumsq");
  switch (epilogue) {
    case VQ_EPI_STORE:
      if (y_dtype != VQ_BF16 && y_dtype != VQ_F32) return fail(VQ_ERR_INVALID_ARG, "vq_qmm_packed: bad y_dtype %d", y_dtype);
      if (ldy < N) return fail(VQ_ERR_INVALID_ARG, "vq_qmm_packed: ldy must be >= N");
      break;
    case VQ_EPI_RESIDUAL:
      if (y_dtype != VQ_BF16) return fail(VQ_ERR_INVALID_ARG, "vq_qmm_packed: the residual epilogue writes bf16");
      if (!residual) return fail(VQ_ERR_INVALID_ARG, "vq_qmm_packed: residual is NULL");
      if (ldy < N || ldr < N) return fail(VQ_ERR_INVALID_ARG, "vq_qmm_packed: ldy and ldr must be >= N");
      if (residual == y && ldr != ldy)
        return fail(VQ_ERR_INVALID_ARG, "vq_qmm_packed: an in-place residual needs ldr == ldy");
      if (!aligned(residual, 2)) return fail(VQ_ERR_INVALID_ARG, "vq_qmm_packed: misaligned residual");
      break;
    case VQ_EPI_SWIGLU:
      if (y_dtype != VQ_BF16) return fail(VQ_ERR_INVALID_ARG, "vq_qmm_packed: the SwiGLU epilogue writes bf16");
      if (N % 128 != 0) return fail(VQ_ERR_INVALID_ARG, "vq_qmm_packed: SwiGLU needs N a multiple of 128 (got %d)", N);
      if (ldy < N / 2) return fail(VQ_ERR_INVALID_ARG, "vq_qmm_packed: ldy must be >= N / 2");
      break;
    default:
      return fail(VQ_ERR_INVALID_ARG, "vq_qmm_packed: unknown epilogue %d", epilogue);
  }
  if (!aligned(y, y_dtype == VQ_F32 ? 4 : 2)) return fail(VQ_ERR_INVALID_ARG, "vq_qmm_packed: misaligned y");
  const vq::QmmPlan plan = vq::qmm_plan(bits, M, N, K, true);
  int rc = check_workspace(workspace, workspace_bytes, plan.counter_bytes + plan.partial_bytes);
  if (rc) return rc;
  if ((rc = check_device())) return rc;
  vq::QmmCall c{};
  c.x = x;
  c.ldx = ldx;
  c.x_ss = x_sumsq;
  c.ss_parts = x_sumsq ? x_sumsq_parts : 0;
  c.eps = eps;
  c.wq = packed;
  c.tiled = true;
  c.bits = bits;
  c.M = M;
  c.N = N;
  c.K = K;
  c.epilogue = epilogue;
  c.res = residual;
  c.ldr = ldr;
  c.y = y;
  c.ldy = ldy;
  c.y_f32 = y_dtype == VQ_F32;
  c.y_ss = y_sumsq;
  c.workspace = workspace;
  hipError_t e = vq::qmm_launch(plan, c, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? VQ_OK : hip_fail(e, "vq_qmm_packed launch");
}

// ------------------------------------------------------------ attention
size_t vq_multirow_attn_workspace(int M, int Hq, int Hkv, int D, int T) {
  if (!attn_shape_ok(M, Hq, Hkv, D, T)) return 0;
  return vq::attn_plan(M, Hq, Hkv, D, T).partial_bytes;
}

namespace {

// Checks shared by the attention entry points; `who` names the call.
int attn_checks(const char* who, const void* q, int64_t q_row_stride, const void* k_cache, const void* v_cache,
                int64_t kv_head_stride, int M, int Hq, int Hkv, int D, int T, float scale, const void* out,
                int64_t out_row_stride) {
  if (!q || !k_cache || !v_cache || !out) return fail(VQ_ERR_INVALID_ARG, "%s: NULL data pointer", who);
  if (!attn_shape_ok(M, Hq, Hkv, D, T))
    return fail(VQ_ERR_INVALID_ARG,
                "%s: unsupported shape M=%d Hq=%d Hkv=%d D=%d T=%d (M in [1,16], Hq %% Hkv == 0, "
                "M*Hq/Hkv <= 128, D in {64,128,256}, T >= M)",
                who, M, Hq, Hkv, D, T);
  if (kv_head_stride < (int64_t)T * D || kv_head_stride % 8 != 0)
    return fail(VQ_ERR_INVALID_ARG, "%s: kv_head_stride must be >= T*D and a multiple of 8", who);
  if (q_row_stride < (int64_t)Hq * D || q_row_stride % 8 != 0 || out_row_stride < (int64_t)Hq * D ||
      out_row_stride % 8 != 0)
    return fail(VQ_ERR_INVALID_ARG, "%s: row strides must be >= Hq*D and multiples of 8", who);
  if (!isfinite(scale)) return fail(VQ_ERR_INVALID_ARG, "%s: scale must be finite", who);
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
    return fail(VQ_ERR_INVALID_ARG, "%s: q, caches and out must be 16-byte aligned", who);
  return VQ_OK;
}

int append_checks(const char* who, const void* k_new, const void* v_new, int64_t new_row_stride, int Hkv, int D) {
  if (!k_new || !v_new) return fail(VQ_ERR_INVALID_ARG, "%s: NULL k_new or v_new", who);
  if (new_row_stride < (int64_t)Hkv * D || new_row_stride % 8 != 0)
    return fail(VQ_ERR_INVALID_ARG, "%s: new_row_stride must be >= Hkv*D and a multiple of 8", who);
  if (!aligned(k_new, 16) || !aligned(v_new, 16))
    return fail(VQ_ERR_INVALID_ARG, "%s: k_new and v_new must be 16-byte aligned", who);
  return VQ_OK;
}

int attn_run(const char* who, const void* q, int64_t q_row_stride, const void* k_new, const void* v_new,
             int64_t new_row_stride, const void* k_cache, const void* v_cache, int64_t kv_head_stride, int M, int Hq,
             int Hkv, int D, int T, float scale, const uint32_t* tree_mask, void* out, int64_t out_row_stride,
             void* workspace, size_t workspace_bytes, void* stream) {
  const vq::AttnPlan plan = vq::attn_plan(M, Hq, Hkv, D, T);
  int rc = check_workspace(workspace, workspace_bytes, plan.partial_bytes);
  if (rc) return rc;
  if ((rc = check_device())) return rc;
  hipError_t e = vq::attn_launch(plan, q, q_row_stride, k_cache, v_cache, kv_head_stride, M, Hq, Hkv, D, T, scale,
                                 out, out_row_stride, workspace, reinterpret_cast<hipStream_t>(stream), k_new, v_new,
                                 new_row_stride, tree_mask);
  return e == hipSuccess ? VQ_OK : hip_fail(e, who);
}

}  // namespace

int vq_multirow_attn(const void* q, int64_t q_row_stride, const void* k_cache, const void* v_cache,
                     int64_t kv_head_stride, int M, int Hq, int Hkv, int D, int T, float scale, void* out,
                     int64_t out_row_stride, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  const char* who = "vq_multirow_attn";
  int rc = attn_checks(who, q, q_row_stride, k_cache, v_cache, kv_head_stride, M, Hq, Hkv, D, T, scale, out,
                       out_row_stride);
  if (rc) return rc;
  return attn_run(who, q, q_row_stride, nullptr, nullptr, 0, k_cache, v_cache, kv_head_stride, M, Hq, Hkv, D, T,
                  scale, nullptr, out, out_row_stride, workspace, workspace_bytes, stream);
}

int vq_multirow_attn_append(const void* q, int64_t q_row_stride, const void* k_new, const void* v_new,
                            int64_t new_row_stride, void* k_cache, void* v_cache, int64_t kv_head_stride, int M,
                            int Hq, int Hkv, int D, int T, float scale, void* out, int64_t out_row_stride,
                            void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  const char* who = "vq_multirow_attn_append";
  int rc = append_checks(who, k_new, v_new, new_row_stride, Hkv, D);
  if (!rc)
    rc = attn_checks(who, q, q_row_stride, k_cache, v_cache, kv_head_stride, M, Hq, Hkv, D, T, scale, out,
                     out_row_stride);
  if (rc) return rc;
  return attn_run(who, q, q_row_stride, k_new, v_new, new_row_stride, k_cache, v_cache, kv_head_stride, M, Hq, Hkv,
                  D, T, scale, nullptr, out, out_row_stride, workspace, workspace_bytes, stream);
}

int vq_multirow_attn_tree(const void* q, int64_t q_row_stride, const void* k_new, const void* v_new,
                          int64_t new_row_stride, void* k_cache, void* v_cache, int64_t kv_head_stride, int M,
                          int Hq, int Hkv, int D, int T, float scale, const uint32_t* tree_mask, void* out,
                          int64_t out_row_stride, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  const char* who = "vq_multirow_attn_tree";
  if (!tree_mask) return fail(VQ_ERR_INVALID_ARG, "%s: tree_mask is NULL", who);
  if (!aligned(tree_mask, 4)) return fail(VQ_ERR_INVALID_ARG, "%s: misaligned tree_mask", who);
  int rc = VQ_OK;
  if (k_new || v_new) rc = append_checks(who, k_new, v_new, new_row_stride, Hkv, D);
  if (!rc)
    rc = attn_checks(who, q, q_row_stride, k_cache, v_cache, kv_head_stride, M, Hq, Hkv, D, T, scale, out,
                     out_row_stride);
  if (rc) return rc;
  return attn_run(who, q, q_row_stride, k_new, v_new, new_row_stride, k_cache, v_cache, kv_head_stride, M, Hq, Hkv,
                  D, T, scale, tree_mask, out, out_row_stride, workspace, workspace_bytes, stream);
}

size_t vq_multirow_attn_batched_workspace(int B, int max_rows, int Hq, int Hkv, int D, int max_T) {
  if (B < 1 || B > VQ_MAX_SEQS || !attn_shape_ok(max_rows, Hq, Hkv, D, max_T)) return 0;
  return vq::attn_plan(max_rows, Hq, Hkv, D, max_T, B).partial_bytes;
}

int vq_multirow_attn_batched(const void* q, int64_t q_row_stride, const int32_t* row_start, const int32_t* seq_len,
                             int B, int total_rows, int max_rows, int max_T, const void* k_new, const void* v_new,
                             int64_t new_row_stride, void* k_cache, void* v_cache, int64_t kv_batch_stride,
                             int64_t kv_head_stride, int Hq, int Hkv, int D, float scale, const uint32_t* tree_mask,
                             void* out, int64_t out_row_stride, void* workspace, size_t workspace_bytes,
                             void* stream) {
  g_err[0] = 0;
  const char* who = "vq_multirow_attn_batched";
  if (!row_start || !seq_len) return fail(VQ_ERR_INVALID_ARG, "%s: NULL row_start or seq_len", who);
  if (!aligned(row_start, 4) || !aligned(seq_len, 4) || (tree_mask && !aligned(tree_mask, 4)))
    return fail(VQ_ERR_INVALID_ARG, "%s: misaligned row_start, seq_len or tree_mask", who);
  if (B < 1 || B > VQ_MAX_SEQS || total_rows < 1 || total_rows > 65535)
    return fail(VQ_ERR_INVALID_ARG, "%s: B must be in [1, %d] and total_rows in [1, 65535] (B=%d total_rows=%d)", who,
                VQ_MAX_SEQS, B, total_rows);
  int rc = VQ_OK;
  if (k_new || v_new) rc = append_checks(who, k_new, v_new, new_row_stride, Hkv, D);
  if (!rc)
    rc = attn_checks(who, q, q_row_stride, k_cache, v_cache, kv_head_stride, max_rows, Hq, Hkv, D, max_T, scale, out,
                     out_row_stride);
  if (rc) return rc;
  if (kv_batch_stride < (int64_t)Hkv * kv_head_stride || kv_batch_stride % 8 != 0)
    return fail(VQ_ERR_INVALID_ARG, "%s: kv_batch_stride must be >= Hkv * kv_head_stride and a multiple of 8", who);
  const vq::AttnPlan plan = vq::attn_plan(max_rows, Hq, Hkv, D, max_T, B);
  if ((rc = check_workspace(workspace, workspace_bytes, plan.partial_bytes))) return rc;
  if ((rc = check_device())) return rc;
  const vq::AttnBatch bt{row_start, seq_len, kv_batch_stride, total_rows, B};
  hipError_t e = vq::attn_launch(plan, q, q_row_stride, k_cache, v_cache, kv_head_stride, max_rows, Hq, Hkv, D,
                                 max_T, scale, out, out_row_stride, workspace, reinterpret_cast<hipStream_t>(stream),
                                 k_new, v_new, new_row_stride, tree_mask, nullptr, nullptr, &bt);
  return e == hipSuccess ? VQ_OK : hip_fail(e, who);
}

int vq_multirow_attn_int8(const void* q, int64_t q_row_stride, const void* k_codes, const void* k_sb,
                          const void* v_codes, const void* v_sb, int64_t kv_head_stride, int M, int Hq, int Hkv,
                          int D, int T, float scale, const uint32_t* tree_mask, void* out, int64_t out_row_stride,
                          void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  const char* who = "vq_multirow_attn_int8";
  if (!k_sb || !v_sb) return fail(VQ_ERR_INVALID_ARG, "%s: NULL k_sb or v_sb", who);
  if (!aligned(k_sb, 4) || !aligned(v_sb, 4) || (tree_mask && !aligned(tree_mask, 4)))
    return fail(VQ_ERR_INVALID_ARG, "%s: misaligned k_sb, v_sb or tree_mask", who);
  int rc = attn_checks(who, q, q_row_stride, k_codes, v_codes, kv_head_stride, M, Hq, Hkv, D, T, scale, out,
                       out_row_stride);
  if (rc) return rc;
  if (kv_head_stride % D != 0)
    return fail(VQ_ERR_INVALID_ARG, "%s: kv_head_stride must be a multiple of D (T_cap * D)", who);
  const vq::AttnPlan plan = vq::attn_plan(M, Hq, Hkv, D, T);
  if ((rc = check_workspace(workspace, workspace_bytes, plan.partial_bytes))) return rc;
  if ((rc = check_device())) return rc;
  hipError_t e = vq::attn_launch(plan, q, q_row_stride, k_codes, v_codes, kv_head_stride, M, Hq, Hkv, D, T, scale,
                                 out, out_row_stride, workspace, reinterpret_cast<hipStream_t>(stream), nullptr,
                                 nullptr, 0, tree_mask, reinterpret_cast<const uint32_t*>(k_sb),
                                 reinterpret_cast<const uint32_t*>(v_sb));
  return e == hipSuccess ? VQ_OK : hip_fail(e, who);
}

int vq_kv8_append(const void* src, int64_t ld_src, int k_off, int v_off, void* k_codes, void* k_sb, void* v_codes,
                  void* v_sb, int64_t kv_head_stride, int M, int Hkv, int D, int pos, void* stream) {
  g_err[0] = 0;
  const char* who = "vq_kv8_append";
  if (!src || !k_codes || !k_sb || !v_codes || !v_sb) return fail(VQ_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if (M < 1 || M > VQ_MAX_ROWS || Hkv < 1 || (D != 64 && D != 128 && D != 256) || pos < 0)
    return fail(VQ_ERR_INVALID_ARG, "%s: unsupported M=%d Hkv=%d D=%d pos=%d", who, M, Hkv, D, pos);
  if (k_off < 0 || v_off < 0 || ld_src < (int64_t)(k_off > v_off ? k_off : v_off) + (int64_t)Hkv * D)
    return fail(VQ_ERR_INVALID_ARG, "%s: k_off, v_off and ld_src must hold Hkv*D values per row", who);
  if (kv_head_stride < (int64_t)(pos + M) * D || kv_head_stride % D != 0)
    return fail(VQ_ERR_INVALID_ARG, "%s: kv_head_stride must be a multiple of D and hold pos + M rows", who);
  if (!aligned(src, 2) || !aligned(k_sb, 4) || !aligned(v_sb, 4))
    return fail(VQ_ERR_INVALID_ARG, "%s: misaligned src, k_sb or v_sb", who);
  int rc;
  if ((rc = check_device())) return rc;
  hipError_t e = vq::kv8_append(src, ld_src, k_off, v_off, k_codes, k_sb, v_codes, v_sb, kv_head_stride, M, Hkv, D,
                                pos, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? VQ_OK : hip_fail(e, who);
}

// ----------------------------------------------------------- acceptance
size_t vq_spec_accept_workspace(int B, int K, int V, int input_kind, int64_t p_batch_stride,
                                int64_t q_batch_stride) {
  if (!accept_shape_ok(B, K, V, input_kind, p_batch_stride, q_batch_stride)) return 0;
  const vq::AcceptPlan p = vq::accept_plan(B, K, V, input_kind, p_batch_stride, q_batch_stride);
  return vq::accept_workspace_total(p);
}

int vq_spec_accept(const float* p, const float* q, int input_kind, int64_t p_batch_stride, int64_t q_batch_stride,
                   const int32_t* draft, const float* uniforms, int B, int K, int V, float temperature, int top_k,
                   float top_p, int32_t* out_tokens, int32_t* out_n_accepted, float* probs_out, void* workspace,
                   size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  if (!p || !uniforms || !out_tokens || !out_n_accepted)
    return fail(VQ_ERR_INVALID_ARG, "vq_spec_accept: NULL data pointer");
  if (K > 0 && (!q || !draft)) return fail(VQ_ERR_INVALID_ARG, "vq_spec_accept: q and draft are required for K > 0");
  if (!accept_shape_ok(B, K, V, input_kind, p_batch_stride, q_batch_stride))
    return fail(VQ_ERR_INVALID_ARG,
                "vq_spec_accept: unsupported arguments B=%d K=%d V=%d kind=%d strides=(%lld,%lld) (B >= 1, "
                "K in [0,15], V in [2, 2^20], strides 0 or >= the rows of one entry, B <= 65535 unless both "
                "strides are 0)",
                B, K, V, input_kind, (long long)p_batch_stride, (long long)q_batch_stride);
  if (top_k < 0) return fail(VQ_ERR_INVALID_ARG, "vq_spec_accept: top_k must be >= 0");
  if (!(top_p > 0.f && top_p <= 1.f)) return fail(VQ_ERR_INVALID_ARG, "vq_spec_accept: top_p must be in (0, 1]");
  if (input_kind == VQ_LOGITS && !(temperature > 0.f && isfinite(temperature)))
    return fail(VQ_ERR_INVALID_ARG, "vq_spec_accept: temperature must be finite and > 0 for logits");
  if (!aligned(p, 4) || (q && !aligned(q, 4)) || (draft && !aligned(draft, 4)) || !aligned(uniforms, 4) ||
      !aligned(out_tokens, 4) || !aligned(out_n_accepted, 4) || (probs_out && !aligned(probs_out, 4)))
    return fail(VQ_ERR_INVALID_ARG, "vq_spec_accept: misaligned pointer");
  const vq::AcceptPlan plan = vq::accept_plan(B, K, V, input_kind, p_batch_stride, q_batch_stride);
  int rc = check_workspace(workspace, workspace_bytes, vq::accept_workspace_total(plan));
  if (rc) return rc;
  if ((rc = check_device())) return rc;
  hipError_t e = vq::accept_launch(plan, p, q, input_kind, p_batch_stride, q_batch_stride, draft, uniforms, B, K, V,
                                   temperature, top_k, top_p, out_tokens, out_n_accepted, probs_out, workspace,
                                   reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? VQ_OK : hip_fail(e, "vq_spec_accept launch");
}

// ----------------------------------------------------------------- glue
int vq_rmsnorm_bf16(const void* x, int64_t ldx, void* y, int64_t ldy, int M, int N, float eps, void* stream) {
  g_err[0] = 0;
  if (!x || !y || M < 1 || N < 1 || N > 65536 || ldx < N || ldy < N || !(eps >= 0.f) || !aligned(x, 2) ||
      !aligned(y, 2))
    return fail(VQ_ERR_INVALID_ARG, "vq_rmsnorm_bf16: invalid arguments");
  int rc = check_device();
  if (rc) return rc;
  hipError_t e = vq::glue_rmsnorm(x, ldx, y, ldy, M, N, eps, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? VQ_OK : hip_fail(e, "vq_rmsnorm_bf16 launch");
}

int vq_row_sumsq_bf16(const void* x, int64_t ldx, int M, int N, float* out, void* stream) {
  g_err[0] = 0;
  if (!x || !out || M < 1 || M > 65535 || N < 1 || N > (1 << 20) || ldx < N || !aligned(x, 2) || !aligned(out, 4))
    return fail(VQ_ERR_INVALID_ARG, "vq_row_sumsq_bf16: invalid arguments");
  int rc = check_device();
  if (rc) return rc;
  hipError_t e = vq::row_sumsq(x, ldx, M, N, out, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? VQ_OK : hip_fail(e, "vq_row_sumsq_bf16 launch");
}

int vq_add_bf16(const void* a, const void* b, void* y, int64_t n, void* stream) {
  g_err[0] = 0;
  if (!a || !b || !y || n < 0 || !aligned(a, 2) || !aligned(b, 2) || !aligned(y, 2))
    return fail(VQ_ERR_INVALID_ARG, "vq_add_bf16: invalid arguments");
  if (n == 0) return VQ_OK;
  int rc = check_device();
  if (rc) return rc;
  hipError_t e = vq::glue_add(a, b, y, n, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? VQ_OK : hip_fail(e, "vq_add_bf16 launch");
}

int vq_silu_mul_bf16(const void* gu, int64_t ldgu, void* y, int64_t ldy, int M, int I, void* stream) {
  g_err[0] = 0;
  if (!gu || !y || M < 1 || M > 65535 || I < 1 || ldgu < 2 * (int64_t)I || ldy < I || !aligned(gu, 2) ||
      !aligned(y, 2))
    return fail(VQ_ERR_INVALID_ARG, "vq_silu_mul_bf16: invalid arguments");
  int rc = check_device();
  if (rc) return rc;
  hipError_t e = vq::glue_silu_mul(gu, ldgu, y, ldy, M, I, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? VQ_OK : hip_fail(e, "vq_silu_mul_bf16 launch");
}

int vq_kv_append_bf16(const void* src, int64_t ld_src, int k_off, int v_off, void* k_cache, void* v_cache,
                      int64_t kv_head_stride, int M, int Hkv, int D, int pos, void* stream) {
  g_err[0] = 0;
  if (!src || !k_cache || !v_cache || M < 1 || Hkv < 1 || D < 8 || D % 8 || k_off < 0 || v_off < 0 ||
      k_off % 8 || v_off % 8 || ld_src % 8 || ld_src < (int64_t)k_off + (int64_t)Hkv * D ||
      ld_src < (int64_t)v_off + (int64_t)Hkv * D || pos < 0 || kv_head_stride % 8 ||
      kv_head_stride < (int64_t)(pos + M) * D || !aligned(src, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(VQ_ERR_INVALID_ARG, "vq_kv_append_bf16: invalid arguments");
  int rc = check_device();
  if (rc) return rc;
  hipError_t e = vq::glue_kv_append(src, ld_src, k_off, v_off, k_cache, v_cache, kv_head_stride, M, Hkv, D, pos,
                                    reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? VQ_OK : hip_fail(e, "vq_kv_append_bf16 launch");
}

// ------------------------------------------------------ streaming-read ceiling
int vq_stream_read(const void* src, size_t bytes, int nontemporal, int workgroups, uint32_t* sink, void* stream) {
  g_err[0] = 0;
  if (!src || !sink) return fail(VQ_ERR_INVALID_ARG, "vq_stream_read: NULL pointer");
  if (bytes == 0 || bytes % 16 != 0) return fail(VQ_ERR_INVALID_ARG, "vq_stream_read: bytes must be a positive multiple of 16");
  if (!aligned(src, 16) || !aligned(sink, 4)) return fail(VQ_ERR_INVALID_ARG, "vq_stream_read: misaligned src or sink");
  if (nontemporal != 0 && nontemporal != 1) return fail(VQ_ERR_INVALID_ARG, "vq_stream_read: nontemporal must be 0 or 1");
  if (workgroups < 1 || workgroups > (1 << 20))
    return fail(VQ_ERR_INVALID_ARG, "vq_stream_read: workgroups must be in [1, 2^20] (got %d)", workgroups);
  int rc = check_device();
  if (rc) return rc;
  hipError_t e = vq::stream_read_launch(src, bytes, nontemporal == 1, workgroups, sink,
                                        reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? VQ_OK : hip_fail(e, "vq_stream_read launch");
}

}  // extern "C"
