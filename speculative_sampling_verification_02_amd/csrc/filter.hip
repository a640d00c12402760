// Top-k / top-p keep thresholds of logit rows for gfx950.
//
// The verification runs on p and q as the sampling method adjusted them ([FI]
// "The loop: draft, verify in one pass, keep a prefix": top-k and nucleus
// sampling zero the tail and renormalise, and the method treats the adjusted
// distributions as p and q), with the same settings for both models ([NZ] "5.
// Sampling and evaluation").  Each filter keeps the tokens whose logit is at
// least a per-row threshold tau, ties included:
//   top-k: tau_k = the k-th largest logit;
//   top-p: tau_p = the largest logit threshold whose kept set (among the top-k
//          survivors) holds at least top_p of their softmax(l / T) mass;
// and the row keeps logit >= max(tau_k, tau_p).  The verification kernels then
// read a dropped logit as -inf.
//
// One workgroup per row finds each threshold by a radix select over the
// logits' order-preserving bit keys, 8 bits per pass from the top: per pass,
// a histogram of the next byte of the keys that share the bytes already
// chosen (counts for top-k, softmax mass for top-p), then a scan from the top
// bin picks the byte.  bf16 keys are 16 bits (2 passes per filter), fp32 keys
// 32 bits (4 passes).  Mass is accumulated in 64-bit fixed point (2^-40 of the
// row maximum's weight), so the sums, and therefore the thresholds, do not
// depend on the order of the atomic additions.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "common.hpp"
#include "specverify.h"
#include "verify_internal.hpp"

namespace specv {
namespace {

constexpr int kFThreads = 512;
constexpr double kMassScale = 1099511627776.0;  // 2^40

struct FilterArgs {
  const void* target;  // [B][gamma+1][V]
  const void* draft;   // [B][gamma][V]
  int nt;              // target rows B (gamma + 1); rows past nt are draft rows
  int V;
  float k;             // log2(e) / T
  int top_k;           // active when 0 < top_k < V
  float top_p;         // active when top_p < 1
  float* thr;          // [rows] out: keep threshold (-inf: keep all)
};

// Order-preserving unsigned key of a finite or -inf logit (-0 as +0), in the
// top KB bits of the dtype's width.
template <int KB>
__device__ inline uint32_t key_of(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return k >> (32 - KB);
}
template <int KB>
__device__ inline float value_of(uint32_t key) {
  const uint32_t k = key << (32 - KB);
  // a bf16 key's low 16 bits are zero for a positive value and all ones for a
  // negative one (they came from the widened value's zero bits)
  const uint32_t full = KB == 32 ? k : ((k & 0x80000000u) ? k : (k | 0x0000ffffu));
  const uint32_t u = (full & 0x80000000u) ? (full & 0x7fffffffu) : ~full;
  return __uint_as_float(u);
}

template <class E>
__global__ __launch_bounds__(kFThreads) void row_threshold_kernel(FilterArgs f) {
  constexpr int KB = std::is_same<E, BF16>::value ? 16 : 32;
  constexpr int kPasses = KB / 8;
  __shared__ uint32_t cnt[256];
  __shared__ unsigned long long msum[256];
  __shared__ float red_f[kFThreads / kWave];
  __shared__ uint32_t prefix_s, need_s;
  __shared__ unsigned long long above_s;
  __shared__ double target_s;
  const int tid = threadIdx.x;
  const int r = blockIdx.x;
  const auto* row = r < f.nt ? static_cast<const typename E::storage*>(f.target) + (size_t)r * f.V
                             : static_cast<const typename E::storage*>(f.draft) + (size_t)(r - f.nt) * f.V;
  auto for_each = [&](auto fn) {
    for (int j0 = tid * E::kVec; j0 < f.V; j0 += kFThreads * E::kVec) {
      float t[E::kVec];
      E::unpack(load_stream(row + j0), t);
#pragma unroll
      for (int e = 0; e < E::kVec; ++e) fn(t[e]);
    }
  };
  const bool use_k = f.top_k > 0 && f.top_k < f.V;
  const bool use_p = f.top_p < 1.f;

  // ---- top-k: the key of the k-th largest logit
  uint32_t tau_k = 0;  // the smallest key: keep all
  if (use_k) {
    if (tid == 0) {
      prefix_s = 0;
      need_s = (uint32_t)f.top_k;  // rank from the top among the keys that share the prefix
    }
    for (int pass = 0; pass < kPasses; ++pass) {
      const int shift = KB - 8 * (pass + 1);
      const uint32_t mask = pass == 0 ? 0u : (~0u << (shift + 8)) & (KB == 32 ? ~0u : 0xffffu);
      for (int b = tid; b < 256; b += kFThreads) cnt[b] = 0;
      __syncthreads();
      const uint32_t prefix = prefix_s;
      for_each([&](float x) {
        const uint32_t key = key_of<KB>(x);
        if ((key & mask) == prefix) atomicAdd(&cnt[(key >> shift) & 0xffu], 1u);
      });
      __syncthreads();
      if (tid == 0) {
        const uint32_t need = need_s;
        uint32_t acc = 0;
        for (int b = 255; b >= 0; --b) {
          if (acc + cnt[b] >= need) {
            need_s = need - acc;
            prefix_s = prefix | ((uint32_t)b << shift);
            break;
          }
          acc += cnt[b];
        }
      }
      __syncthreads();
    }
    tau_k = prefix_s;
  }

  // ---- top-p: the largest key whose upper set holds top_p of the survivors' mass
  uint32_t tau_p = 0;
  if (use_p) {
    // the row maximum, for weights exp2((l - m) k) in (0, 1]
    float m = -INFINITY;
    for_each([&](float x) { m = fmaxf(m, x); });
    m = wave_max(m);
    if ((tid & (kWave - 1)) == 0) red_f[tid / kWave] = m;
    __syncthreads();
    m = red_f[0];
    for (int w = 1; w < kFThreads / kWave; ++w) m = fmaxf(m, red_f[w]);
    if (tid == 0) {
      prefix_s = 0;
      above_s = 0;
    }
    for (int pass = 0; pass < kPasses; ++pass) {
      const int shift = KB - 8 * (pass + 1);
      const uint32_t mask = pass == 0 ? 0u : (~0u << (shift + 8)) & (KB == 32 ? ~0u : 0xffffu);
      for (int b = tid; b < 256; b += kFThreads) msum[b] = 0;
      __syncthreads();
      const uint32_t prefix = prefix_s;
      for_each([&](float x) {
        const uint32_t key = key_of<KB>(x);
        if (key >= tau_k && (key & mask) == prefix && x != -INFINITY) {
          const float w = __builtin_amdgcn_exp2f((x - m) * f.k);
          atomicAdd(&msum[(key >> shift) & 0xffu], (unsigned long long)((double)w * kMassScale + 0.5));
        }
      });
      __syncthreads();
      if (tid == 0) {
        if (pass == 0) {
          unsigned long long total = 0;
          for (int b = 0; b < 256; ++b) total += msum[b];
          target_s = (double)f.top_p * (double)total;
        }
        unsigned long long acc = above_s;
        for (int b = 255; b >= 0; --b) {
          if ((double)(acc + msum[b]) >= target_s) {
            above_s = acc;
            prefix_s = prefix | ((uint32_t)b << shift);
            break;
          }
          acc += msum[b];
        }
      }
      __syncthreads();
    }
    tau_p = prefix_s;
  }
  if (tid == 0) f.thr[r] = (use_k || use_p) ? value_of<KB>(max(tau_k, tau_p)) : -INFINITY;
}

__global__ void fill_zero_kernel(float* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

}  // namespace

hipError_t filter_thresholds(const VerifyArgs& a, int top_k, float top_p, float* thr, hipStream_t s) {
  FilterArgs f{a.target, a.draft, a.B * (a.gamma + 1), a.V, a.k, top_k, top_p, thr};
  const int rows = a.B * (2 * a.gamma + 1);
  if (rows == 0) return hipSuccess;
  if (a.dtype == SPEC_BF16)
    row_threshold_kernel<BF16><<<dim3(rows), dim3(kFThreads), 0, s>>>(f);
  else
    row_threshold_kernel<F32><<<dim3(rows), dim3(kFThreads), 0, s>>>(f);
  return hipGetLastError();
}

hipError_t filter_clear(float* thr, int rows, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  fill_zero_kernel<<<dim3((rows + 255) / 256), dim3(256), 0, s>>>(thr, rows);
  return hipGetLastError();
}

}  // namespace specv
