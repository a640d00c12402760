// Multi-pass verification path for gfx950.
//
// Three launches on one stream:
//   K1 row_stats     per (row, chunk of kChunk tokens): the chunk maximum m_c and
//                    S_c = sum exp2((l - m_c) k), or the chunk argmax at T = 0.
//   K2 pair_overlap  per (draft position, chunk): the two rows' global
//                    normalisers from K1's partials, then the chunk's share of
//                    alpha = sum min(p, q) and of the residual mass sum max(0, p - q).
//   K3 finish        per sequence: ratio tests, accepted prefix, alpha totals,
//                    then the inverse-CDF sample.  It locates the chunk that
//                    holds the sample from the chunk masses and scans only that chunk.
//
// Each logit is read by K1 and again by K2 (the overlap needs both rows'
// normalisers before any element can be compared), and one chunk per sequence
// is read by K3.  The fused path reads every logit once.
//
// Page abbreviations: [FI] intuitivepapers.ai "Fast Inference from Transformers
// via Speculative Decoding"; [SD] nonconvexcard "Speculative Decoding".

#include <math.h>

#include "common.hpp"
#include "specverify.h"
#include "verify_internal.hpp"

namespace specv {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 8192;  // tokens per chunk; a multiple of 256 * 8

__host__ __device__ inline int num_chunks(int V) { return (V + kChunk - 1) / kChunk; }

// Row numbering shared by K1..K3: target rows first, then draft rows.
__device__ inline size_t target_row(int b, int i, int gamma) { return (size_t)b * (gamma + 1) + i; }
__device__ inline size_t draft_row(int b, int i, int gamma, int B) {
  return (size_t)B * (gamma + 1) + (size_t)b * gamma + i;
}

template <class E>
__device__ inline const typename E::storage* row_ptr(const VerifyArgs& a, size_t row) {
  const size_t nt = (size_t)a.B * (a.gamma + 1);
  if (row < nt) return static_cast<const typename E::storage*>(a.target) + row * (size_t)a.V;
  return static_cast<const typename E::storage*>(a.draft) + (row - nt) * (size_t)a.V;
}

// Visit the elements [lo, hi) of a row owned by this thread, in a fixed order:
// vector steps of kThreads * kVec tokens, thread t taking the t-th vector.
// `VEC` requires a 16-byte aligned row base and V a multiple of kVec.
template <class E, bool VEC, class F>
__device__ inline void for_chunk(const typename E::storage* row, int lo, int hi, F&& f) {
  if constexpr (VEC) {
    constexpr int step = kThreads * E::kVec;
    for (int base = lo; base < hi; base += step) {
      const int j0 = base + threadIdx.x * E::kVec;
      if (j0 < hi) {
        float x[E::kVec];
        E::unpack(load_stream(row + j0), x);
#pragma unroll
        for (int k = 0; k < E::kVec; ++k) f(j0 + k, x[k]);
      }
    }
  } else {
    for (int j = lo + threadIdx.x; j < hi; j += kThreads) f(j, E::at(row, j));
  }
}

// ------------------------------------------------------------------ K1

template <class E, bool VEC, bool ARGMAX>
__global__ __launch_bounds__(kThreads) void row_stats_kernel(VerifyArgs a, float2* stats) {
  __shared__ float lds_f[kMaxWaves];
  __shared__ int lds_i[kMaxWaves];
  const int nch = num_chunks(a.V);
  const size_t row = blockIdx.x / nch;
  const int c = blockIdx.x % nch;
  const int lo = c * kChunk, hi = min(a.V, lo + kChunk);
  const auto* r = row_ptr<E>(a, row);

  if constexpr (ARGMAX) {
    ArgMax best{-INFINITY, 0x7fffffff};
    for_chunk<E, VEC>(r, lo, hi, [&](int j, float x) { best = argmax_better(best, ArgMax{x, j}); });
    best = block_argmax(best, lds_f, lds_i);
    if (threadIdx.x == 0) stats[blockIdx.x] = make_float2(best.v, __int_as_float(best.i));
  } else {
    float m = -INFINITY;
    for_chunk<E, VEC>(r, lo, hi, [&](int, float x) { m = fmaxf(m, x); });
    m = block_max(m, lds_f);
    float s = 0.f;
    if (m != -INFINITY) {
      const float k = a.k;
      for_chunk<E, VEC>(r, lo, hi, [&](int, float x) { s += fast_exp2((x - m) * k); });
    }
    s = block_sum(s, lds_f);
    if (threadIdx.x == 0) stats[blockIdx.x] = make_float2(m, s);
  }
}

// Global normaliser of one row from its chunk partials, always in chunk order
// so that every kernel that calls it gets bit-identical values.
struct RowNorm {
  float M;      // row maximum
  float invS;   // 1 / sum exp2((l - M) k), rounded to fp32
  double S;     // the sum, fp64
};

__device__ inline double chunk_weight(float2 st, float M, float k) {
  // S_c rescaled from the chunk maximum to the row maximum.
  if (st.x == -INFINITY) return 0.0;
  return (double)st.y * exp2(((double)st.x - (double)M) * (double)k);
}

__device__ inline RowNorm combine_row(const float2* st, int nch, float k) {
  float M = -INFINITY;
  for (int c = 0; c < nch; ++c) M = fmaxf(M, st[c].x);
  double S = 0.0;
  for (int c = 0; c < nch; ++c) S += chunk_weight(st[c], M, k);
  return RowNorm{M, (float)(1.0 / S), S};
}

__device__ inline ArgMax combine_argmax(const float2* st, int nch) {
  ArgMax best{-INFINITY, 0x7fffffff};
  for (int c = 0; c < nch; ++c) best = argmax_better(best, ArgMax{st[c].x, __float_as_int(st[c].y)});
  return best;
}

// p_j and q_j in fp32 from a logit and its row normaliser.  K2 and K3 use this
// one expression so the residual weights they see are bit-identical.
__device__ inline float prob(float x, float M, float invS, float k) {
  return fast_exp2((x - M) * k) * invS;
}

// ------------------------------------------------------------------ K2

template <class E, bool VEC>
__global__ __launch_bounds__(kThreads) void pair_overlap_kernel(VerifyArgs a, const float2* stats,
                                                                float2* pair_stats) {
  __shared__ float lds_f[kMaxWaves];
  __shared__ float norm[4];
  const int nch = num_chunks(a.V);
  const int pair = blockIdx.x / nch;  // b * gamma + i
  const int c = blockIdx.x % nch;
  const int b = pair / a.gamma, i = pair % a.gamma;
  const size_t rp = target_row(b, i, a.gamma), rq = draft_row(b, i, a.gamma, a.B);
  if (threadIdx.x == 0) {
    RowNorm np = combine_row(stats + rp * nch, nch, a.k);
    RowNorm nq = combine_row(stats + rq * nch, nch, a.k);
    norm[0] = np.M; norm[1] = np.invS; norm[2] = nq.M; norm[3] = nq.invS;
  }
  __syncthreads();
  const float Mp = norm[0], invSp = norm[1], Mq = norm[2], invSq = norm[3], k = a.k;
  const int lo = c * kChunk, hi = min(a.V, lo + kChunk);
  const auto* p_row = row_ptr<E>(a, rp);
  const auto* q_row = row_ptr<E>(a, rq);

  float acc_min = 0.f, acc_res = 0.f;
  if constexpr (VEC) {
    constexpr int step = kThreads * E::kVec;
    for (int base = lo; base < hi; base += step) {
      const int j0 = base + threadIdx.x * E::kVec;
      if (j0 < hi) {
        float xp[E::kVec], xq[E::kVec];
        E::unpack(load_stream(p_row + j0), xp);
        E::unpack(load_stream(q_row + j0), xq);
#pragma unroll
        for (int t = 0; t < E::kVec; ++t) {
          const float p = prob(xp[t], Mp, invSp, k), q = prob(xq[t], Mq, invSq, k);
          acc_min += fminf(p, q);
          acc_res += fmaxf(p - q, 0.f);
        }
      }
    }
  } else {
    for (int j = lo + threadIdx.x; j < hi; j += kThreads) {
      const float p = prob(E::at(p_row, j), Mp, invSp, k), q = prob(E::at(q_row, j), Mq, invSq, k);
      acc_min += fminf(p, q);
      acc_res += fmaxf(p - q, 0.f);
    }
  }
  acc_min = block_sum(acc_min, lds_f);
  acc_res = block_sum(acc_res, lds_f);
  if (threadIdx.x == 0) pair_stats[blockIdx.x] = make_float2(acc_min, acc_res);
}

// ------------------------------------------------------------------ K3

// Inverse-CDF search inside one chunk: the first token j in [lo, hi) whose
// running weight (from 0 at lo) exceeds theta.  `weight(j, x)` gives the
// weight of token j with logit x in row `r0` (and `x1` from row `r1` for the
// residual).  If rounding leaves the whole chunk at or below theta, the last
// token with positive weight is returned.  Called by the whole workgroup.
template <class E, bool VEC, class W>
__device__ int chunk_search(const typename E::storage* r0, const typename E::storage* r1, int lo,
                            int hi, float theta, W&& weight, float* lds_f, int* lds_i) {
  constexpr int kPer = VEC ? E::kVec : 1;
  constexpr int step = kThreads * kPer;
  __shared__ int found;
  if (threadIdx.x == 0) found = -1;
  int last_pos = -1;  // per thread: last index with positive weight seen
  float carry = 0.f;
  for (int base = lo; base < hi; base += step) {
    const int j0 = base + threadIdx.x * kPer;
    float w[kPer];
    float s = 0.f;
#pragma unroll
    for (int t = 0; t < kPer; ++t) w[t] = 0.f;
    if (j0 < hi) {
      float x0[kPer], x1[kPer];
      if constexpr (VEC) {
        E::unpack(load_stream(r0 + j0), x0);
        if (r1) E::unpack(load_stream(r1 + j0), x1);
      } else {
        x0[0] = E::at(r0, j0);
        if (r1) x1[0] = E::at(r1, j0);
      }
#pragma unroll
      for (int t = 0; t < kPer; ++t) {
        w[t] = weight(x0[t], r1 ? x1[t] : 0.f);
        if (w[t] > 0.f) last_pos = j0 + t;
        s += w[t];
      }
    }
    float excl, total;
    const float incl = block_scan(s, lds_f, &excl, &total);
    const float start = carry + excl, end = carry + incl;
    if (start <= theta && theta < end) {
      float run = start;
      int pick = -1, lastp = -1;
#pragma unroll
      for (int t = 0; t < kPer; ++t) {
        if (w[t] > 0.f) lastp = j0 + t;
        run += w[t];
        if (pick < 0 && run > theta) pick = j0 + t;
      }
      found = pick >= 0 ? pick : lastp;  // exactly one thread owns theta
    }
    carry += total;
    __syncthreads();
    if (found >= 0) break;
  }
  const int f = found;
  __syncthreads();
  if (f >= 0) return f;
  // rounding guard: the last positive-weight token of the chunk
  // (offsets inside a chunk are < kChunk, so they compare exactly as floats)
  ArgMax lp{last_pos >= 0 ? (float)(last_pos - lo) : -1.f, last_pos};
  lp = block_argmax(lp, lds_f, lds_i);
  return lp.i;
}

template <class E, bool VEC>
__global__ __launch_bounds__(kThreads) void finish_kernel(VerifyArgs a, const float2* stats,
                                                          const float2* pair_stats) {
  __shared__ float lds_f[kMaxWaves];
  __shared__ int lds_i[kMaxWaves];
  __shared__ int accept_s[SPEC_MAX_GAMMA];
  __shared__ int n_s;
  __shared__ int row_s, chunk_s, residual_s;
  __shared__ float theta_s, norm_s[4];
  const int b = blockIdx.x, G = a.gamma, nch = num_chunks(a.V);
  const float k = a.k;
  const int tid = threadIdx.x;
  const float* u = a.uniforms + (size_t)b * (G + 1);

  if (a.temperature == 0.f) {
    // ---- argmax mode
    __shared__ int amax_t[SPEC_MAX_GAMMA + 1], amax_d[SPEC_MAX_GAMMA];
    if (tid <= G) amax_t[tid] = combine_argmax(stats + target_row(b, tid, G) * nch, nch).i;
    if (tid < G) amax_d[tid] = combine_argmax(stats + draft_row(b, tid, G, a.B) * nch, nch).i;
    __syncthreads();
    if (tid < G) {
      const int x = a.tokens[(size_t)b * G + tid];
      const size_t o = (size_t)b * G + tid;
      accept_s[tid] = (x == amax_t[tid]);
      if (a.alpha) a.alpha[o] = (amax_t[tid] == amax_d[tid]) ? 1.f : 0.f;
      if (a.p_draft) a.p_draft[o] = (x == amax_t[tid]) ? 1.f : 0.f;
      if (a.q_draft) a.q_draft[o] = (x == amax_d[tid]) ? 1.f : 0.f;
    }
    __syncthreads();
    if (tid == 0) {
      int n = 0;
      while (n < G && accept_s[n]) ++n;
      a.n_out[b] = n;
      a.t_out[b] = amax_t[n];
    }
    return;
  }

  // ---- ratio tests ([FI] Algorithm 1 step 3; [SD] "The algorithm"), in fp64
  if (tid < G) {
    const size_t rp = target_row(b, tid, G), rq = draft_row(b, tid, G, a.B);
    const RowNorm np = combine_row(stats + rp * nch, nch, k);
    const RowNorm nq = combine_row(stats + rq * nch, nch, k);
    const int x = a.tokens[(size_t)b * G + tid];
    double px = 0.0, qx = 0.0;
    if (x >= 0 && x < a.V) {
      const double lp = (double)E::at(row_ptr<E>(a, rp), x);
      const double lq = (double)E::at(row_ptr<E>(a, rq), x);
      px = exp2((lp - (double)np.M) * (double)k) / np.S;
      qx = exp2((lq - (double)nq.M) * (double)k) / nq.S;
    }
    const double ratio = px / qx;  // IEEE: p/0 = inf (accept), 0/0 = NaN (reject)
    const double uu = (double)u[tid];
    accept_s[tid] = (ratio >= 1.0) || (uu <= ratio);
    const size_t o = (size_t)b * G + tid;
    if (a.p_draft) a.p_draft[o] = (float)px;
    if (a.q_draft) a.q_draft[o] = (float)qx;
    if (a.alpha) {
      double al = 0.0;
      const float2* ps = pair_stats + ((size_t)b * G + tid) * nch;
      for (int c = 0; c < nch; ++c) al += (double)ps[c].x;
      a.alpha[o] = (float)al;
    }
  }
  __syncthreads();

  // ---- accepted prefix and the row to sample from
  if (tid == 0) {
    int n = 0;
    while (n < G && accept_s[n]) ++n;
    n_s = n;
    const double uf = (double)u[G];
    int residual = 0, chunk = nch - 1;
    double theta = 0.0;
    if (n < G) {
      // residual max(0, p_n - q_n) ([FI] eq. (2); [SD] "Exactness")
      const float2* ps = pair_stats + ((size_t)b * G + n) * nch;
      double Sw = 0.0;
      for (int c = 0; c < nch; ++c) Sw += (double)ps[c].y;
      if (Sw > 0.0) {
        residual = 1;
        theta = uf * Sw;
        double P = 0.0;
        for (int c = 0; c < nch; ++c) {
          const double w = (double)ps[c].y;
          if (w > 0.0) chunk = c;
          if (P + w > theta && w > 0.0) { chunk = c; break; }
          P += w;
        }
        theta_s = (float)(theta - P);
        const RowNorm np = combine_row(stats + target_row(b, n, G) * nch, nch, k);
        const RowNorm nq = combine_row(stats + draft_row(b, n, G, a.B) * nch, nch, k);
        norm_s[0] = np.M; norm_s[1] = np.invS; norm_s[2] = nq.M; norm_s[3] = nq.invS;
      }
    }
    if (!residual) {
      // bonus token from p_gamma, or p_n if the residual carried no mass
      const float2* st = stats + target_row(b, n, G) * nch;
      const RowNorm np = combine_row(st, nch, k);
      theta = uf * np.S;
      double P = 0.0;
      for (int c = 0; c < nch; ++c) {
        const double w = chunk_weight(st[c], np.M, k);
        if (w > 0.0) chunk = c;
        if (P + w > theta && w > 0.0) { chunk = c; break; }
        P += w;
      }
      theta_s = (float)(theta - P);
      norm_s[0] = np.M;
    }
    residual_s = residual;
    chunk_s = chunk;
    row_s = n;
  }
  __syncthreads();

  const int n = row_s, c = chunk_s;
  const int lo = c * kChunk, hi = min(a.V, lo + kChunk);
  const float theta = theta_s;
  int t;
  if (residual_s) {
    const float Mp = norm_s[0], invSp = norm_s[1], Mq = norm_s[2], invSq = norm_s[3];
    t = chunk_search<E, VEC>(row_ptr<E>(a, target_row(b, n, G)), row_ptr<E>(a, draft_row(b, n, G, a.B)),
                             lo, hi, theta,
                             [&](float xp, float xq) {
                               return fmaxf(prob(xp, Mp, invSp, k) - prob(xq, Mq, invSq, k), 0.f);
                             },
                             lds_f, lds_i);
  } else {
    const float M = norm_s[0];
    t = chunk_search<E, VEC>(row_ptr<E>(a, target_row(b, n, G)), nullptr, lo, hi, theta,
                             [&](float xp, float) { return fast_exp2((xp - M) * k); }, lds_f, lds_i);
  }
  if (tid == 0) {
    a.n_out[b] = n;
    a.t_out[b] = t;
  }
}

template <class E, bool VEC>
hipError_t launch_typed(const VerifyArgs& a, hipStream_t s) {
  const int nch = num_chunks(a.V);
  const size_t rows = (size_t)a.B * (2 * a.gamma + 1);
  float2* stats = static_cast<float2*>(a.ws);
  float2* pair_stats = stats + rows * nch;
  const bool argmax = a.temperature == 0.f;
  const dim3 blk(kThreads);
  if (argmax)
    row_stats_kernel<E, VEC, true><<<dim3(rows * nch), blk, 0, s>>>(a, stats);
  else
    row_stats_kernel<E, VEC, false><<<dim3(rows * nch), blk, 0, s>>>(a, stats);
  if (!argmax && a.gamma > 0)
    pair_overlap_kernel<E, VEC><<<dim3((size_t)a.B * a.gamma * nch), blk, 0, s>>>(a, stats, pair_stats);
  finish_kernel<E, VEC><<<dim3(a.B), blk, 0, s>>>(a, stats, pair_stats);
  return hipGetLastError();
}

}  // namespace

size_t multipass_workspace_bytes(int B, int gamma, int V) {
  const size_t nch = num_chunks(V);
  return ((size_t)B * (2 * gamma + 1) + (size_t)B * gamma) * nch * sizeof(float2);
}

hipError_t multipass_launch(const VerifyArgs& a, hipStream_t s) {
  const size_t esz = a.dtype == SPEC_BF16 ? 2 : 4;
  const bool aligned = ((uintptr_t)a.target % 16 == 0) && (a.gamma == 0 || (uintptr_t)a.draft % 16 == 0) &&
                       ((size_t)a.V * esz) % 16 == 0;
  if (a.dtype == SPEC_BF16)
    return aligned ? launch_typed<BF16, true>(a, s) : launch_typed<BF16, false>(a, s);
  return aligned ? launch_typed<F32, true>(a, s) : launch_typed<F32, false>(a, s);
}

}  // namespace specv
