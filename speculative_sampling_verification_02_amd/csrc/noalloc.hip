// spec_verify_noalloc: spec_verify for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation).  The verification's scratch -- the fused path's
// exchange slots or the multi-pass path's statistics -- lives in one
// file-scope device array instead of a caller-provided workspace.
//
// The array's name is only a host-side stand-in in host code.  Its device
// address is looked up once per device, with that device current, through
// hipGetSymbolAddress, and only that address is handed to kernels.  The array
// is zero-filled on the first call on each device; every call that completes
// leaves the part it used zero again, as the workspace contract of spec_verify
// requires.

#include <hip/hip_runtime.h>

#include <mutex>

#include "specverify.h"
#include "verify_internal.hpp"

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;  // per device, held until the process ends
constexpr int kMaxDevices = 64;
constexpr int kFillThreads = 256;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct DeviceScratch {
  void* ptr = nullptr;  // device address of `scratch` on that device
  bool zeroed = false;
};
DeviceScratch g_dev[kMaxDevices];
std::mutex g_mutex;

// Zeroes `words` 16-byte words (a kernel, not a memset, so it can be captured
// into a graph and replayed).
__global__ __launch_bounds__(kFillThreads) void fill_zero(uint4* p, size_t words) {
  for (size_t i = (size_t)blockIdx.x * kFillThreads + threadIdx.x; i < words; i += (size_t)gridDim.x * kFillThreads)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

hipError_t zero_scratch(void* ptr, hipStream_t s) {
  static_assert(kScratchBytes % 16 == 0, "whole words");
  const size_t words = kScratchBytes / 16;
  fill_zero<<<dim3(1024), dim3(kFillThreads), 0, s>>>(static_cast<uint4*>(ptr), words);
  return hipGetLastError();
}

// The current device's scratch address, looked up (and zero-filled on
// `s`) on the first call on that device.
hipError_t device_scratch(hipStream_t s, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  DeviceScratch& d = g_dev[dev];
  if (!d.ptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    d.ptr = p;
  }
  if (!d.zeroed) {
    e = zero_scratch(d.ptr, s);
    if (e != hipSuccess) return e;
    d.zeroed = true;
  }
  *out = d.ptr;
  return hipSuccess;
}

int map_hip(hipError_t e) {
  if (e == hipSuccess) return SPEC_OK;
  return e == hipErrorNotSupported ? SPEC_EUNSUPPORTED : SPEC_EHIP;
}

}  // namespace

extern "C" {

size_t spec_verify_noalloc_limit(void) { return kScratchBytes; }

int spec_verify_noalloc(const void* target_logits, const void* draft_logits, int dtype,
                        const int32_t* draft_tokens, const float* uniforms, int B, int gamma, int V,
                        float temperature, int32_t* n_accepted, int32_t* next_token, float* alpha,
                        float* p_draft, float* q_draft, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the argument checks of spec_verify, before anything is queued
  const int st = specv::verify_check(target_logits, draft_logits, dtype, draft_tokens, uniforms, B, gamma, V,
                                     temperature, n_accepted, next_token);
  if (st != SPEC_OK) return st;
  if (B > 0 && specv::verify_scratch_bytes(B, gamma, V) > kScratchBytes) return SPEC_ENOSPACE;
  void* ws = nullptr;
  const hipError_t e = device_scratch(s, &ws);
  if (e != hipSuccess) return map_hip(e);
  if (B == 0) return map_hip(zero_scratch(ws, s));  // B == 0 clears the scratch
  return specv::verify_in_scratch(target_logits, draft_logits, dtype, draft_tokens, uniforms, B, gamma, V,
                                  temperature, n_accepted, next_token, alpha, p_draft, q_draft, ws,
                                  kScratchBytes, s);
}

}  // extern "C"
