// A plain streaming read of a device buffer: the HBM read rate this device
// sustains, measured beside the verification kernels for context.

#include <hip/hip_runtime.h>

#include "common.hpp"
#include "specverify.h"

namespace specv {
namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;  // 16-byte loads in flight per thread per step

// Every 16-byte vector is read once (grid-stride, four loads in flight per
// thread); the XOR of the words is written per workgroup so the reads stay.
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4* p, size_t n, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * kReadThreads;
  size_t i = (size_t)blockIdx.x * kReadThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kReadUnroll - 1) * stride < n; i += kReadUnroll * stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = load_stream(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) {
    const u32x4 v = load_stream(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red[kReadThreads / kWave];
  for (int off = kWave / 2; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < kReadThreads / kWave; ++w) r ^= red[w];
    sink[blockIdx.x] = r;
  }
}

}  // namespace
}  // namespace specv

extern "C" int spec_stream_read(const void* buffer, size_t bytes, uint32_t* sink, int blocks, void* stream) {
  if (!buffer || !sink || blocks < 1 || bytes % 16 || (reinterpret_cast<uintptr_t>(buffer) & 15u)) return SPEC_EINVAL;
  if (bytes == 0) return SPEC_OK;
  specv::stream_read_kernel<<<dim3(blocks), dim3(specv::kReadThreads), 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const specv::u32x4*>(buffer), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}
