// lli8_int8_linear_noalloc: the forward with every workspace buffer in a
// fixed device array of the library, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  It enqueues exactly what
// lli8_int8_linear enqueues, with the workspace carved from that array.
#include <stdio.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/lli8.h"
#include "lli8_internal.h"

// One copy per GPU, allocated with the code object when the library is first
// used on that GPU and held until the process ends; zero at load.
static __device__ __align__(256) unsigned char scratch[LLI8_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch`, per device

// The array's device address on the current device.  In host code the name
// `scratch` is only a host-side stand-in; kernels must be given this address.
lli8_status_t scratch_address(void** out) {
  char msg[256];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    snprintf(msg, sizeof msg, "hipGetDevice: %s", hipGetErrorString(e));
    return lli8::set_error(LLI8_ERR_HIP, msg);
  }
  if (dev < 0 || dev >= kMaxDevices) {
    snprintf(msg, sizeof msg, "device %d beyond the %d the library tracks", dev, kMaxDevices);
    return lli8::set_error(LLI8_ERR_UNSUPPORTED, msg);
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      snprintf(msg, sizeof msg, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
      return lli8::set_error(LLI8_ERR_HIP, msg);
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LLI8_OK;
}

}  // namespace

extern "C" {

size_t lli8_noalloc_scratch_bytes(void) { return LLI8_NOALLOC_SCRATCH_BYTES; }

lli8_status_t lli8_int8_linear_noalloc(const void* X, int64_t T, int64_t K, int64_t N, lli8_dtype_t dtype,
                                       const int8_t* CB, const float* SCB, const void* bias, float threshold,
                                       void* out, void* stream) {
  lli8_status_t st = lli8::check_linear_args(X, T, K, N, dtype, CB, SCB, bias, threshold, out);
  if (st != LLI8_OK) return st;
  const size_t need = lli8_workspace_bytes(T, K, N, dtype);
  if (need > LLI8_NOALLOC_SCRATCH_BYTES) {
    char msg[256];
    snprintf(msg, sizeof msg,
             "T=%lld K=%lld N=%lld needs %zu bytes of workspace, above the fixed %zu of the no-allocation "
             "entry point (use lli8_int8_linear with a caller workspace)",
             (long long)T, (long long)K, (long long)N, need, (size_t)LLI8_NOALLOC_SCRATCH_BYTES);
    return lli8::set_error(LLI8_ERR_UNSUPPORTED, msg);
  }
  void* base = nullptr;
  st = scratch_address(&base);
  if (st != LLI8_OK) return st;
  lli8_workspace_t ws;
  st = lli8_workspace_carve(base, LLI8_NOALLOC_SCRATCH_BYTES, T, K, N, dtype, &ws);
  if (st != LLI8_OK) return st;
  return lli8_int8_linear(X, T, K, N, dtype, CB, SCB, bias, threshold, out, &ws, stream);
}

}  // extern "C"
