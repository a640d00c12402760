// Device helpers for the gfx950 verification kernels: element loads for
// fp32 / bf16 logit rows, wave64 and workgroup reductions, and a workgroup
// exclusive scan.  All reductions combine in a fixed order, so results are
// bit-reproducible run to run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specv {

constexpr int kWave = 64;

// 16 bytes as four 32-bit words (a native clang vector, so it can be used
// with the nontemporal load builtin).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------ element types

struct F32 {
  using storage = float;
  static constexpr int kVec = 4;  // elements per 16-byte load
  __device__ static inline float at(const storage* p, size_t j) { return p[j]; }
  // Unpack one 16-byte vector into kVec floats.
  __device__ static inline void unpack(const u32x4& v, float* out) {
    out[0] = __uint_as_float(v.x);
    out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z);
    out[3] = __uint_as_float(v.w);
  }
};

struct BF16 {
  using storage = uint16_t;
  static constexpr int kVec = 8;
  __device__ static inline float at(const storage* p, size_t j) {
    return __uint_as_float(static_cast<uint32_t>(p[j]) << 16);
  }
  // bf16 -> fp32 is exact: the 16 stored bits are the high half of the fp32 word.
  __device__ static inline void unpack(const u32x4& v, float* out) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      out[2 * k] = __uint_as_float(w[k] << 16);
      out[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  }
};

// Streaming 16-byte load that does not need to stay in cache.
__device__ inline u32x4 load_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------ wave reductions

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ inline double wave_sum(double v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// (value, index) with "greater value wins, lower index breaks ties".
struct ArgMax {
  float v;
  int i;
};

__device__ inline ArgMax argmax_better(ArgMax a, ArgMax b) {
  // IEEE comparison: -0.0 == +0.0, so signed zeros tie and the lower index wins.
  if (b.v > a.v || (b.v == a.v && b.i < a.i)) return b;
  return a;
}

__device__ inline ArgMax wave_argmax(ArgMax a) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    ArgMax b{__shfl_xor(a.v, o, kWave), __shfl_xor(a.i, o, kWave)};
    a = argmax_better(a, b);
  }
  return a;
}

// Inclusive scan across the wave in lane order.
__device__ inline float wave_inclusive_scan(float v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    float t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

// ------------------------------------------------------- workgroup reductions
// `lds` must hold at least kMaxWaves entries; the call contains barriers and
// must be reached by every thread of the workgroup.

constexpr int kMaxWaves = 16;

__device__ inline float block_max(float v, float* lds) {
  const int wid = threadIdx.x / kWave, nw = blockDim.x / kWave;
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) lds[wid] = v;
  __syncthreads();
  float r = lds[0];
  for (int w = 1; w < nw; ++w) r = fmaxf(r, lds[w]);
  return r;
}

__device__ inline float block_sum(float v, float* lds) {
  const int wid = threadIdx.x / kWave, nw = blockDim.x / kWave;
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) lds[wid] = v;
  __syncthreads();
  float r = lds[0];
  for (int w = 1; w < nw; ++w) r += lds[w];
  return r;
}

__device__ inline ArgMax block_argmax(ArgMax a, float* ldsv, int* ldsi) {
  const int wid = threadIdx.x / kWave, nw = blockDim.x / kWave;
  a = wave_argmax(a);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) {
    ldsv[wid] = a.v;
    ldsi[wid] = a.i;
  }
  __syncthreads();
  ArgMax r{ldsv[0], ldsi[0]};
  for (int w = 1; w < nw; ++w) r = argmax_better(r, ArgMax{ldsv[w], ldsi[w]});
  return r;
}

// Scan of one value per thread in thread order.  Returns the exclusive prefix
// in *excl and the inclusive prefix as the result; the inclusive prefix of
// thread t is bit-identical to the exclusive prefix of thread t+1, so the
// ranges [excl, incl) partition [0, total) without gaps.  *total gets the sum.
__device__ inline float block_scan(float v, float* lds, float* excl, float* total) {
  const int wid = threadIdx.x / kWave, nw = blockDim.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const float inc = wave_inclusive_scan(v);
  float prev = __shfl_up(inc, 1, kWave);
  if (lane == 0) prev = 0.f;
  __syncthreads();
  if (lane == kWave - 1) lds[wid] = inc;
  __syncthreads();
  float before = 0.f;
  for (int w = 0; w < wid; ++w) before += lds[w];
  float all = before;
  for (int w = wid; w < nw; ++w) all += lds[w];
  *total = all;
  *excl = (lane == 0) ? before : before + prev;
  return before + inc;
}

}  // namespace specv
