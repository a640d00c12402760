// Multi-pass verification path for gfx950.
//
// Three launches on one stream:
//   K1 row_stats     per (row, chunk of kChunk tokens, kChunkArgmax at T = 0): the chunk maximum m_c and
//                    S_c = sum exp2((l - m_c) k), or the chunk argmax at T = 0.
//                    The chunk is read once into registers.
//   K2 pair_overlap  per (draft position, chunk): the two rows' normalisers from
//                    K1's partials (one wave, fixed order), then the chunk's
//                    share of alpha = sum min(p, q) and of the residual mass
//                    sum max(0, p - q).
//   K3 finish        per sequence: fp64 ratio tests, accepted prefix, alpha
//                    totals, then the inverse-CDF sample.  It locates the chunk
//                    holding the sample from the chunk masses and scans only that chunk.
// K2 and K3 combine a row's partials with the same function, so they see
// bit-identical normalisers.
//
// Each logit is read by K1 and again by K2, because the overlap needs both
// rows' normalisers before any element can be compared.  K3 reads one chunk
// per sequence.  The fused path reads every logit once.  This path accepts any
// row alignment and any V.
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
// In argmax mode a chunk costs a few instructions per token, and larger
// chunks (fewer workgroups, more loads in flight each) stream faster: 31 vs
// 29 us at B = 64, gamma = 4, V = 128256 bf16, 357 vs 331 us at B = 256,
// gamma = 8, V = 256000.  At T > 0 the smaller chunk measured faster.
constexpr int kChunkArgmax = 16384;

// Chunks per row.  Argmax chunks tile V + 7 positions: a row that does not
// start on 16 bytes is read from its aligned-down start, up to 7 positions
// early (row_stats_kernel); for aligned rows the count is the same.
__host__ __device__ inline int num_chunks(int V, bool argmax = false) {
  const int ch = argmax ? kChunkArgmax : kChunk;
  return ((argmax ? V + 7 : V) + ch - 1) / ch;
}

// Argmax mode: a row chunk publishes its (value, index) as one 64-bit word,
// and finishing workgroups at the end of the same grid wait for a sequence's
// words, up to kArgFinSlots of them per sequence (beyond that a separate
// finish launch reads them).  The low half is the value's bits with +0.0
// stored as -0.0 (the same value), so a published word is never zero.
constexpr int kArgFinSlots = 1024;
constexpr int kArgFinGroups = 256;  // finishing workgroups at most

__device__ inline void publish_argmax(float2* stats, size_t i, ArgMax best) {
  const uint32_t v = __float_as_uint(best.v);
  st_u64(reinterpret_cast<uint64_t*>(stats) + i, (uint64_t)(v == 0u ? 0x80000000u : v) | ((uint64_t)(uint32_t)best.i << 32));
}

// Row numbering shared by every kernel here: target rows first, then draft rows.
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

// Top-k / top-p: a logit below its row's keep threshold counts as -inf
// (probability 0); without thresholds every logit is kept.
__device__ inline float row_thr(const VerifyArgs& a, size_t row) { return a.thr ? a.thr[row] : -INFINITY; }
__device__ inline float keep(float x, float th) { return x >= th ? x : -INFINITY; }

// A row's normaliser: maximum, 1/S in fp32 and S in fp64.
struct RowNorm {
  float M;
  float invS;
  double S;
};

// This thread's kPer tokens of a chunk in registers, visited in a fixed order:
// vector steps of kThreads * kVec tokens, thread t taking the t-th vector of
// each step.  Needs a 16-byte aligned row base and V a multiple of kVec.
// Tokens at or past `hi` read as -inf.
template <class E, int CH = kChunk>
struct ChunkRegs {
  static constexpr int kPer = CH / kThreads;
  static constexpr int NS = kPer / E::kVec;
  float x[kPer];
  __device__ inline int token(int lo, int t) const {
    return lo + ((t / E::kVec) * kThreads + (int)threadIdx.x) * E::kVec + t % E::kVec;
  }
  u32x4 raw[NS];
  // Issue the chunk's loads without waiting for them.
  __device__ inline void issue(const typename E::storage* row, int lo, int hi) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int j0 = lo + (s * kThreads + (int)threadIdx.x) * E::kVec;
      raw[s] = j0 < hi ? load_stream(row + j0) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ inline void unpack(int lo, int hi) {
    if (lo + CH <= hi) {  // the whole chunk is in range: no per-token select
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        float t[E::kVec];
        E::unpack(raw[s], t);
#pragma unroll
        for (int v = 0; v < E::kVec; ++v) x[s * E::kVec + v] = t[v];
      }
      return;
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int j0 = lo + (s * kThreads + (int)threadIdx.x) * E::kVec;
      float t[E::kVec];
      E::unpack(raw[s], t);
#pragma unroll
      for (int v = 0; v < E::kVec; ++v) x[s * E::kVec + v] = j0 < hi ? t[v] : -INFINITY;
    }
  }
  __device__ inline void load(const typename E::storage* row, int lo, int hi) {
    issue(row, lo, hi);
    unpack(lo, hi);
  }
};

// ChunkRegs for a row that does not start on 16 bytes, in a tensor that does:
// the same tokens per thread, each vector of kVec tokens cut out of the two
// aligned vectors that cover it (the second is the next thread's first, a
// cache hit).  A vector whose pair would run past the row's end is read
// token by token.
template <class E, int CH = kChunk>
struct ShiftedChunk {
  static constexpr int kPer = CH / kThreads;
  static constexpr int NS = kPer / E::kVec;
  float x[kPer];
  __device__ inline int token(int lo, int t) const {
    return lo + ((t / E::kVec) * kThreads + (int)threadIdx.x) * E::kVec + t % E::kVec;
  }
  u32x4 ra_[NS], rb_[NS];
  const typename E::storage* row_;
  int sh_, V_;
  // vector s of this thread is cut from aligned vectors when both lie in the row
  __device__ inline bool whole(int j0) const { return j0 + 2 * E::kVec - sh_ <= V_; }
  __device__ inline void issue(const typename E::storage* row, int lo, int hi, int V) {
    row_ = row;
    V_ = V;
    sh_ = (int)(((uintptr_t)row & 15u) / sizeof(typename E::storage));
    const auto* ra = row - sh_;  // 16-byte aligned; inside the tensor (sh_ > 0 only past its first row)
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int j0 = lo + (s * kThreads + (int)threadIdx.x) * E::kVec;
      const bool w = j0 < hi && whole(j0);
      ra_[s] = w ? load_stream(ra + j0) : u32x4{0u, 0u, 0u, 0u};
      rb_[s] = w ? load_stream(ra + j0 + E::kVec) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ inline void unpack(int lo, int hi) {
    const int o = sh_ * (int)sizeof(typename E::storage);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int j0 = lo + (s * kThreads + (int)threadIdx.x) * E::kVec;
      float t[E::kVec];
      if (j0 < hi && whole(j0)) {
        E::unpack(cut_vector(ra_[s], rb_[s], o), t);
      } else {
#pragma unroll
        for (int v = 0; v < E::kVec; ++v) t[v] = j0 + v < hi ? E::at(row_, j0 + v) : -INFINITY;
      }
#pragma unroll
      for (int v = 0; v < E::kVec; ++v) x[s * E::kVec + v] = t[v];
    }
  }
  __device__ inline void load(const typename E::storage* row, int lo, int hi, int V) {
    issue(row, lo, hi, V);
    unpack(lo, hi);
  }
};

// Whether both logit tensors start on 16 bytes (their rows need not).
__device__ inline bool bases_aligned(const VerifyArgs& a) {
  return ((uintptr_t)a.target & 15u) == 0 && (a.gamma == 0 || ((uintptr_t)a.draft & 15u) == 0);
}

// ------------------------------------------------------------------ K1

// Argmax mode, sequence b: waits for the chunk words of its rows (target rows
// 0..gamma_b, then draft rows 0..gamma_b - 1; the padding rows are never
// written), combines each row's argmax in chunk order and writes the outputs
// ([FI] "Speculative sampling", temperature to zero: keep x_i iff it is the
// target's argmax; alpha_i is 1 iff the two argmaxes agree).  It is the last
// reader of the words and clears them.  A wait that gives up after `polls`
// polls reports -1.
__device__ void argmax_finish(const VerifyArgs& a, float2* stats, int b, int nch, unsigned polls) {
  __shared__ uint64_t w[kArgFinSlots];
  __shared__ int ok_s;
  __shared__ int amax_t[SPEC_MAX_GAMMA + 1], amax_d[SPEC_MAX_GAMMA], acc_s[SPEC_MAX_GAMMA];
  const int tid = threadIdx.x, G = a.gamma, Gb = seq_gamma(a, b);
  uint64_t* words = reinterpret_cast<uint64_t*>(stats);
  uint64_t* wt = words + target_row(b, 0, G) * nch;
  uint64_t* wd = words + draft_row(b, 0, G, a.B) * nch;
  const int nt = (Gb + 1) * nch, nd = Gb * nch, n = nt + nd;
  const int x = tid < Gb ? a.tokens[(size_t)b * G + tid] : 0;  // fetched before the wait
  if (tid >= Gb && tid < G) {
    // padding positions report NaN
    const float nan = __uint_as_float(0x7fc00000u);
    const size_t o = (size_t)b * G + tid;
    if (a.alpha) a.alpha[o] = nan;
    if (a.p_draft) a.p_draft[o] = nan;
    if (a.q_draft) a.q_draft[o] = nan;
  }
  if (tid < kWave) {  // one wave polls every word of the sequence at once
    bool ok = false;
    for (unsigned it = 0; it < polls; ++it) {
      bool all = true;
      for (int j = tid; j < n; j += kWave) {
        const uint64_t v = j < nt ? ld_u64(wt + j) : ld_u64(wd + (j - nt));
        w[j] = v;
        all = all && (uint32_t)v != 0u;
      }
      if (__all(all)) {
        ok = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (tid == 0) ok_s = ok;
  }
  __syncthreads();
  if (!ok_s) {
    if (tid == 0) {
      a.n_out[b] = -1;  // a wait gave up: no result
      a.t_out[b] = -1;
    }
    return;
  }
  auto row_argmax = [&](const uint64_t* r) {
    ArgMax best{-INFINITY, 0x7fffffff};
    for (int c = 0; c < nch; ++c)
      best = argmax_better(best, ArgMax{__uint_as_float((uint32_t)r[c]), (int)(uint32_t)(r[c] >> 32)});
    return best.i;
  };
  if (tid <= Gb) amax_t[tid] = row_argmax(w + tid * nch);
  if (tid < Gb) amax_d[tid] = row_argmax(w + nt + tid * nch);
  __syncthreads();
  for (int j = tid; j < n; j += kThreads) st_u64(j < nt ? wt + j : wd + (j - nt), 0ull);
  if (tid < Gb) {
    const size_t o = (size_t)b * G + tid;
    acc_s[tid] = x == amax_t[tid];
    if (a.alpha) a.alpha[o] = (amax_t[tid] == amax_d[tid]) ? 1.f : 0.f;
    if (a.p_draft) a.p_draft[o] = (x == amax_t[tid]) ? 1.f : 0.f;
    if (a.q_draft) a.q_draft[o] = (x == amax_d[tid]) ? 1.f : 0.f;
  }
  __syncthreads();
  if (tid == 0) {
    int nacc = 0;
    while (nacc < Gb && acc_s[nacc]) ++nacc;
    a.n_out[b] = nacc;
    a.t_out[b] = amax_t[nacc];
  }
  __syncthreads();  // amax_t / amax_d are rewritten by the next sequence
}

template <class E, bool VEC, bool ARGMAX>
__global__ __launch_bounds__(kThreads) void row_stats_kernel(VerifyArgs a, float2* stats, int nfin, unsigned polls) {
  __shared__ float lds_f[kMaxWaves];
  __shared__ int lds_i[kMaxWaves];
  constexpr int CH = ARGMAX ? kChunkArgmax : kChunk;
  const int nch = num_chunks(a.V, ARGMAX);
  if constexpr (ARGMAX) {
    const size_t nrc = (size_t)a.B * (2 * a.gamma + 1) * nch;  // row chunks
    if (blockIdx.x >= nrc) {  // a finishing workgroup
      for (int b = (int)(blockIdx.x - nrc); b < a.B; b += nfin) argmax_finish(a, stats, b, nch, polls);
      return;
    }
  }
  const size_t row = blockIdx.x / nch;
  const int c = blockIdx.x % nch;
  const int lo = c * CH, hi = min(a.V, lo + CH);
  const auto* r = row_ptr<E>(a, row);
  if (a.gamma_seq) {
    // rows past a sequence's draft count are padding: never read
    const size_t nt = (size_t)a.B * (a.gamma + 1);
    const bool target = row < nt;
    const int b = target ? (int)(row / (a.gamma + 1)) : (int)((row - nt) / a.gamma);
    const int i = target ? (int)(row % (a.gamma + 1)) : (int)((row - nt) % a.gamma);
    if (i > seq_gamma(a, b) - (target ? 0 : 1)) return;
  }

  // the chunk's (max, sum of exp2((x - max) k)) from its tokens in registers
  auto chunk_stats = [&](auto& ch) {
    constexpr int kPer = sizeof(ch.x) / sizeof(float);
    if (a.thr) {
      const float th = a.thr[row];
#pragma unroll
      for (int t = 0; t < kPer; ++t) ch.x[t] = keep(ch.x[t], th);
    }
    // four independent chains keep the dependency chains short
    float m0 = -INFINITY, m1 = -INFINITY, m2 = -INFINITY, m3 = -INFINITY;
#pragma unroll
    for (int t = 0; t < kPer; t += 4) {
      m0 = fmaxf(m0, ch.x[t]);
      m1 = fmaxf(m1, ch.x[t + 1]);
      m2 = fmaxf(m2, ch.x[t + 2]);
      m3 = fmaxf(m3, ch.x[t + 3]);
    }
    const float M = block_max(fmaxf(fmaxf(m0, m1), fmaxf(m2, m3)), lds_f);
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int t = 0; t < kPer; t += 4) {
        s0 += fast_exp2((ch.x[t] - M) * a.k);
        s1 += fast_exp2((ch.x[t + 1] - M) * a.k);
        s2 += fast_exp2((ch.x[t + 2] - M) * a.k);
        s3 += fast_exp2((ch.x[t + 3] - M) * a.k);
      }
    }
    const float s = block_sum((s0 + s1) + (s2 + s3), lds_f);
    if (threadIdx.x == 0) stats[blockIdx.x] = make_float2(M, s);
  };

  if constexpr (VEC) {
    ChunkRegs<E, CH> ch;
    ch.load(r, lo, hi);
    if constexpr (ARGMAX) {
      ArgMax best = thread_argmax_first(ch.x, [&](int t) { return ch.token(lo, t); });
      best = block_argmax(best, lds_f, lds_i);
      if (threadIdx.x == 0) publish_argmax(stats, blockIdx.x, best);
    } else {
      chunk_stats(ch);
    }
  } else {
    if constexpr (ARGMAX) {
      if (bases_aligned(a)) {
        // A row that does not start on 16 bytes: 16-byte loads from the
        // aligned-down start ra = r - sh, so position j of the row's stream
        // holds token j - sh.  The chunks tile the positions [0, V + sh); the
        // first sh positions belong to the previous row and are skipped, and
        // the last vector, which may run past the row's end, is read token by
        // token.
        constexpr int kPer = CH / kThreads, NS = kPer / E::kVec;
        const int sh = (int)(((uintptr_t)r & 15u) / sizeof(typename E::storage));
        const auto* ra = r - sh;
        const int end = a.V + sh, plo = c * CH;
        u32x4 raw[NS];
#pragma unroll
        for (int q = 0; q < NS; ++q) {
          const int j0 = plo + (q * kThreads + (int)threadIdx.x) * E::kVec;
          raw[q] = j0 + E::kVec <= end ? load_stream(ra + j0) : u32x4{0u, 0u, 0u, 0u};
        }
        // skipped positions carry index INT_MAX, so a row of -inf still
        // returns its lowest token
        ArgMax best{-INFINITY, 0x7fffffff};
#pragma unroll
        for (int q = 0; q < NS; ++q) {
          const int j0 = plo + (q * kThreads + (int)threadIdx.x) * E::kVec;
          float t[E::kVec];
          E::unpack(raw[q], t);
#pragma unroll
          for (int v = 0; v < E::kVec; ++v) {
            const int j = j0 + v;
            if (j >= sh && j < end)
              best = argmax_better(best, ArgMax{j0 + E::kVec <= end ? t[v] : E::at(ra, j), j - sh});
          }
        }
        best = block_argmax(best, lds_f, lds_i);
        if (threadIdx.x == 0) publish_argmax(stats, blockIdx.x, best);
        return;
      }
    }
    if constexpr (!ARGMAX) {
      if (bases_aligned(a)) {
        ShiftedChunk<E, CH> ch;
        ch.load(r, lo, hi, a.V);
        chunk_stats(ch);
        return;
      }
    }
    // scalar loads (tensors that do not start on 16 bytes); at T > 0 two
    // sweeps over the chunk (the second hits cache)
    if constexpr (ARGMAX) {
      ArgMax best{-INFINITY, 0x7fffffff};
      for (int j = lo + threadIdx.x; j < hi; j += kThreads) best = argmax_better(best, ArgMax{E::at(r, j), j});
      best = block_argmax(best, lds_f, lds_i);
      if (threadIdx.x == 0) publish_argmax(stats, blockIdx.x, best);
    } else {
      const float th = row_thr(a, row);
      float m = -INFINITY;
      for (int j = lo + threadIdx.x; j < hi; j += kThreads) m = fmaxf(m, keep(E::at(r, j), th));
      const float M = block_max(m, lds_f);
      float s = 0.f;
      if (M != -INFINITY)
        for (int j = lo + threadIdx.x; j < hi; j += kThreads) s += fast_exp2((keep(E::at(r, j), th) - M) * a.k);
      s = block_sum(s, lds_f);
      if (threadIdx.x == 0) stats[blockIdx.x] = make_float2(M, s);
    }
  }
}

// Row normaliser from the row's K1 partials, computed by one wave.
__device__ inline RowNorm row_norm(const float2* stats, size_t row, int nch, float k) {
  const WaveNorm w = wave_row_norm(stats + row * nch, nch, k);
  return RowNorm{w.M, (float)(1.0 / w.S), w.S};
}

// p_j and q_j in fp32 from a logit and its row normaliser.  K2 and K3 use this
// one expression so the residual weights they see are bit-identical.
__device__ inline float prob(float x, float M, float invS, float k) { return fast_exp2((x - M) * k) * invS; }

// ------------------------------------------------------------------ K2

template <class E, bool VEC>
__global__ __launch_bounds__(kThreads) void pair_overlap_kernel(VerifyArgs a, const float2* stats,
                                                                float2* pair_stats) {
  __shared__ float lds_f[2 * kMaxWaves];
  __shared__ RowNorm norm_s[2];
  const int nch = num_chunks(a.V);
  const int pair = blockIdx.x / nch;  // b * gamma + i
  const int c = blockIdx.x % nch;
  const int b = pair / a.gamma, i = pair % a.gamma;
  if (i >= seq_gamma(a, b)) return;  // a padding position
  const size_t rp = target_row(b, i, a.gamma), rq = draft_row(b, i, a.gamma, a.B);
  const float l = a.lenience;  // the residual is max(0, p - l q)
  const float k = a.k;
  const float thp = row_thr(a, rp), thq = row_thr(a, rq);
  const int lo = c * kChunk, hi = min(a.V, lo + kChunk);
  const auto* p_row = row_ptr<E>(a, rp);
  const auto* q_row = row_ptr<E>(a, rq);
  const int wid = threadIdx.x / kWave;
  // the row normalisers, combined while the chunk's loads are in flight
  auto norms = [&]() {
    if (wid < 2) {
      const RowNorm n = row_norm(stats, wid == 0 ? rp : rq, nch, k);
      if ((threadIdx.x & (kWave - 1)) == 0) norm_s[wid] = n;
    }
    __syncthreads();
  };
  float acc_min = 0.f, acc_res = 0.f;
  auto overlap = [&](auto& cp, auto& cq) {
    const RowNorm np = norm_s[0], nq = norm_s[1];
    constexpr int kPer = sizeof(cp.x) / sizeof(float);
    float mn[2] = {0.f, 0.f}, rs[2] = {0.f, 0.f};
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
      const float p = prob(keep(cp.x[t], thp), np.M, np.invS, k), q = prob(keep(cq.x[t], thq), nq.M, nq.invS, k);
      mn[t & 1] += fminf(p, q);
      rs[t & 1] += fmaxf(p - l * q, 0.f);
    }
    acc_min = mn[0] + mn[1];
    acc_res = rs[0] + rs[1];
  };
  if constexpr (VEC) {
    ChunkRegs<E> cp, cq;
    cp.issue(p_row, lo, hi);
    cq.issue(q_row, lo, hi);
    norms();
    cp.unpack(lo, hi);
    cq.unpack(lo, hi);
    overlap(cp, cq);
  } else if (bases_aligned(a)) {
    // p and q cut from their own aligned vectors: the same tokens in both
    ShiftedChunk<E> cp, cq;
    cp.issue(p_row, lo, hi, a.V);
    cq.issue(q_row, lo, hi, a.V);
    norms();
    cp.unpack(lo, hi);
    cq.unpack(lo, hi);
    overlap(cp, cq);
  } else {
    norms();
    const RowNorm np = norm_s[0], nq = norm_s[1];
    for (int j = lo + threadIdx.x; j < hi; j += kThreads) {
      const float p = prob(keep(E::at(p_row, j), thp), np.M, np.invS, k);
      const float q = prob(keep(E::at(q_row, j), thq), nq.M, nq.invS, k);
      acc_min += fminf(p, q);
      acc_res += fmaxf(p - l * q, 0.f);
    }
  }
  const float2 r = block_sum2(acc_min, acc_res, lds_f);
  if (threadIdx.x == 0) pair_stats[blockIdx.x] = r;
}

// ------------------------------------------------------------------ K3

// Zero sequence b's row and pair statistics.  The finish block of b is their
// only reader; it calls this after its last read, so every call leaves the
// workspace all-zero, as the fused path's exchange slots require.
__device__ inline void clear_sequence_stats(const VerifyArgs& a, float2* stats, float2* pair_stats, int b, int nch) {
  const int G = a.gamma;
  const float2 z = make_float2(0.f, 0.f);
  for (int r = 0; r < 2 * G + 1; ++r) {
    const size_t row = r <= G ? target_row(b, r, G) : draft_row(b, r - G - 1, G, a.B);
    for (int c = threadIdx.x; c < nch; c += kThreads) stats[row * nch + c] = z;
  }
  if (a.temperature != 0.f)
    for (int j = threadIdx.x; j < G * nch; j += kThreads) pair_stats[(size_t)b * G * nch + j] = z;
}

template <class E, bool VEC>
__global__ __launch_bounds__(kThreads) void finish_kernel(VerifyArgs a, float2* stats, float2* pair_stats) {
  __shared__ float lds_f[kMaxWaves];
  __shared__ int lds_i[kMaxWaves];
  __shared__ double lds_d[kMaxWaves];
  __shared__ int accept_s[SPEC_MAX_GAMMA];
  __shared__ float mass_s[kThreads];
  __shared__ double prefix_s;
  __shared__ int n_s, chunk_s;
  __shared__ float theta_s;
  // G is the padded draft count (the row stride), Gb this sequence's own
  const int b = blockIdx.x, G = a.gamma, nch = num_chunks(a.V, a.temperature == 0.f), Gb = seq_gamma(a, b);
  const float k = a.k;
  const int tid = threadIdx.x;
  const float* u = a.uniforms + (size_t)b * (G + 1);
  if (tid >= Gb && tid < G) {
    // padding positions report NaN
    const float nan = __uint_as_float(0x7fc00000u);
    const size_t o = (size_t)b * G + tid;
    if (a.alpha) a.alpha[o] = nan;
    if (a.p_draft) a.p_draft[o] = nan;
    if (a.q_draft) a.q_draft[o] = nan;
  }

  if (a.temperature == 0.f) {
    // ---- argmax mode: combine each row's chunk argmaxes
    __shared__ int amax_t[SPEC_MAX_GAMMA + 1], amax_d[SPEC_MAX_GAMMA];
    if (tid <= Gb) {
      const float2* st = stats + target_row(b, tid, G) * nch;
      ArgMax best{-INFINITY, 0x7fffffff};
      for (int c = 0; c < nch; ++c) best = argmax_better(best, ArgMax{st[c].x, __float_as_int(st[c].y)});
      amax_t[tid] = best.i;
    }
    if (tid < Gb) {
      const float2* st = stats + draft_row(b, tid, G, a.B) * nch;
      ArgMax best{-INFINITY, 0x7fffffff};
      for (int c = 0; c < nch; ++c) best = argmax_better(best, ArgMax{st[c].x, __float_as_int(st[c].y)});
      amax_d[tid] = best.i;
    }
    __syncthreads();
    if (tid < Gb) {
      const int x = a.tokens[(size_t)b * G + tid];
      const size_t o = (size_t)b * G + tid;
      accept_s[tid] = (x == amax_t[tid]);
      if (a.alpha) a.alpha[o] = (amax_t[tid] == amax_d[tid]) ? 1.f : 0.f;
      if (a.p_draft) a.p_draft[o] = (x == amax_t[tid]) ? 1.f : 0.f;
      if (a.q_draft) a.q_draft[o] = (x == amax_d[tid]) ? 1.f : 0.f;
    }
    __syncthreads();
    clear_sequence_stats(a, stats, pair_stats, b, nch);
    if (tid == 0) {
      int n = 0;
      while (n < Gb && accept_s[n]) ++n;
      a.n_out[b] = n;
      a.t_out[b] = amax_t[n];
    }
    return;
  }

  // ---- ratio tests ([FI] Algorithm 1 step 3; [SD] "The algorithm"), in fp64.
  // Wave w handles draft positions w, w + 4, ...; lane 0 does the test.
  const int wid = tid / kWave, lane = tid & (kWave - 1), nw = kThreads / kWave;
  for (int i = wid; i < Gb; i += nw) {
    const size_t rp = target_row(b, i, G), rq = draft_row(b, i, G, a.B);
    const RowNorm np = row_norm(stats, rp, nch, k), nq = row_norm(stats, rq, nch, k);
    const size_t o = (size_t)b * G + i;
    double al = 0.0;
    for (int c = lane; c < nch; c += kWave) al += (double)pair_stats[o * nch + c].x;
    al = wave_sum(al);
    if (lane == 0) {
      const int x = a.tokens[o];
      double px = 0.0, qx = 0.0;
      if (x >= 0 && x < a.V) {
        px = exp2(((double)keep(E::at(row_ptr<E>(a, rp), x), row_thr(a, rp)) - (double)np.M) * (double)k) / np.S;
        qx = exp2(((double)keep(E::at(row_ptr<E>(a, rq), x), row_thr(a, rq)) - (double)nq.M) * (double)k) / nq.S;
      }
      // q(x) = 0 keeps the draft when p(x) > 0 (ratio +inf) and rejects it
      // when p(x) = 0 (0/0)
      // with lenience l the comparison is against p(x) / (l q(x))
      if (qx > 0.0) {
        const double ratio = px / ((double)a.lenience * qx);
        accept_s[i] = (ratio >= 1.0) || ((double)u[i] <= ratio);
      } else {
        accept_s[i] = px > 0.0;
      }
      if (a.p_draft) a.p_draft[o] = (float)px;
      if (a.q_draft) a.q_draft[o] = (float)qx;
      if (a.alpha) a.alpha[o] = (float)al;
    }
  }
  __syncthreads();
  if (tid == 0) {
    int n = 0;
    while (n < Gb && accept_s[n]) ++n;
    n_s = n;
  }
  __syncthreads();
  const int n = n_s;

  // ---- the sampled row's chunk masses, in chunk order: the residual
  // max(0, p_n - l q_n) ([FI] eq. (2); [SD] "Exactness"; l = 1 there) when a
  // draft was rejected, else p_{gamma_b} (the bonus token).  A residual with no
  // mass falls back to p_n ([LH] "Three candidates explain the acceptance
  // rule": a zero-mass residual is not normalised).
  const float2* res_st = n < Gb ? pair_stats + ((size_t)b * G + n) * nch : nullptr;
  const float2* row_st = stats + target_row(b, n, G) * nch;
  __shared__ RowNorm norm_s[2];
  if (wid < 2 && (wid == 0 || n < Gb)) {
    const RowNorm nr = row_norm(stats, wid == 0 ? target_row(b, n, G) : draft_row(b, n, G, a.B), nch, k);
    if (lane == 0) norm_s[wid] = nr;
  }
  __syncthreads();
  const RowNorm np = norm_s[0];
  double part = 0.0;
  if (res_st)
    for (int c = tid; c < nch; c += kThreads) part += (double)res_st[c].y;
  bool residual = res_st && block_sum(part, lds_d) > 0.0;
  // chunk c's mass: R_c for the residual, S_c rescaled to the row maximum for p_n
  auto mass = [&](int c) -> float {
    if (residual) return res_st[c].y;
    const float2 v = row_st[c];
    return v.x == -INFINITY ? 0.f : v.y * fast_exp2((v.x - np.M) * k);
  };
  const auto* p_row = row_ptr<E>(a, target_row(b, n, G));
  int t;
  for (;;) {
    part = 0.0;
    for (int c = tid; c < nch; c += kThreads) part += (double)mass(c);
    const double theta = (double)u[Gb] * block_sum(part, lds_d);  // the final sample's uniform

    // ---- locate the chunk holding theta: stage up to kThreads masses in LDS
    // with one parallel load, then scan them in order on one thread.
    if (tid == 0) {
      prefix_s = 0.0;
      chunk_s = -1;
    }
    int last = 0;
    for (int base = 0; base < nch; base += kThreads) {
      const int c = base + tid;
      mass_s[tid] = c < nch ? mass(c) : 0.f;
      __syncthreads();
      if (tid == 0 && chunk_s < 0) {
        double P = prefix_s;
        for (int j = 0; j < kThreads && base + j < nch; ++j) {
          const double w = (double)mass_s[j];
          if (w > 0.0) {
            last = base + j;
            if (P + w > theta) {
              chunk_s = base + j;
              break;
            }
          }
          P += w;
        }
        prefix_s = P;
      }
      __syncthreads();
      if (chunk_s >= 0) break;
    }
    if (tid == 0) {
      if (chunk_s < 0) chunk_s = last;  // rounding guard: theta past every chunk
      theta_s = (float)(theta - prefix_s);
    }
    __syncthreads();

    const int c = chunk_s, lo = c * kChunk, hi = min(a.V, lo + kChunk);
    const float thp = row_thr(a, target_row(b, n, G));
    if (residual) {
      const RowNorm nq = norm_s[1];
      const auto* q_row = row_ptr<E>(a, draft_row(b, n, G, a.B));
      const float l = a.lenience;
      const float thq = row_thr(a, draft_row(b, n, G, a.B));
      auto w = [&](float xp, float xq) {
        return fmaxf(prob(keep(xp, thp), np.M, np.invS, k) - l * prob(keep(xq, thq), nq.M, nq.invS, k), 0.f);
      };
      if constexpr (VEC)
        t = tile_search<E, kChunk / kThreads, kThreads>(p_row, q_row, lo, a.V, theta_s, w, lds_f, lds_i);
      else if (bases_aligned(a))
        t = shifted_tile_search<E, kChunk / kThreads>(p_row, q_row, lo, a.V, theta_s, w, lds_f, lds_i);
      else
        t = range_search<E, false, kThreads>(p_row, q_row, lo, hi, theta_s, w, lds_f, lds_i);
      // The chunk masses sum these same per-token weights, so a chunk with
      // positive mass holds a positive weight; should the compiled arithmetic
      // of the two kernels ever differ, draw from the whole row's residual.
      if (t < 0) t = row_search<E, VEC, kThreads>(p_row, q_row, a.V, (double)u[Gb], w, lds_f, lds_i, lds_d);
    } else {
      auto w = [&](float xp, float) { return fast_exp2((keep(xp, thp) - np.M) * k); };
      if constexpr (VEC)
        t = tile_search<E, kChunk / kThreads, kThreads>(p_row, nullptr, lo, a.V, theta_s, w, lds_f, lds_i);
      else if (bases_aligned(a))
        t = shifted_tile_search<E, kChunk / kThreads>(p_row, nullptr, lo, a.V, theta_s, w, lds_f, lds_i);
      else
        t = range_search<E, false, kThreads>(p_row, nullptr, lo, hi, theta_s, w, lds_f, lds_i);
    }
    // No token of the row has a positive residual: p_n and l q_n agree to fp32
    // everywhere, the residual without mass.  Sample p_n itself (t is the same
    // in every thread).
    if (!(residual && t < 0)) break;
    residual = false;
    __syncthreads();
  }
  __syncthreads();
  clear_sequence_stats(a, stats, pair_stats, b, nch);  // no statistic is read after this
  if (a.thr) {
    // every kernel before this one has read the sequence's keep thresholds
    // and this one is done with them: zero them (the workspace is left zero)
    for (int r = tid; r < 2 * G + 1; r += kThreads)
      a.thr[r <= G ? target_row(b, r, G) : draft_row(b, r - G - 1, G, a.B)] = 0.f;
  }

  if (tid == 0) {
    a.n_out[b] = n;
    a.t_out[b] = t;
  }
}

struct Layout {
  size_t stats, pair_stats, total;
};

Layout layout(int B, int gamma, int V) {
  const size_t nch = num_chunks(V), rows = (size_t)B * (2 * gamma + 1);
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  Layout L{};
  L.stats = 0;
  L.pair_stats = up(rows * nch * sizeof(float2));
  L.total = up(L.pair_stats + (size_t)B * gamma * nch * sizeof(float2));
  return L;
}

template <class E, bool VEC>
hipError_t launch_typed(const VerifyArgs& a, hipStream_t s) {
  const size_t rows = (size_t)a.B * (2 * a.gamma + 1);
  const Layout L = layout(a.B, a.gamma, a.V);
  char* ws = static_cast<char*>(a.ws);
  float2* stats = reinterpret_cast<float2*>(ws + L.stats);
  float2* pair_stats = reinterpret_cast<float2*>(ws + L.pair_stats);
  const bool argmax = a.temperature == 0.f;
  const dim3 blk(kThreads);
  if (argmax) {
    // the finishing workgroups run in the same launch when a sequence's chunk
    // words fit their LDS; they are the last in the grid, so they start only
    // once every row chunk has been dispatched
    const int ncha = num_chunks(a.V, true);
    const bool inline_fin = (size_t)(2 * a.gamma + 1) * ncha <= (size_t)kArgFinSlots;
    const int nfin = inline_fin ? std::min(a.B, kArgFinGroups) : 0;
    row_stats_kernel<E, VEC, true><<<dim3(rows * ncha + nfin), blk, 0, s>>>(a, stats, nfin, wait_limit());
    if (inline_fin) return hipGetLastError();
  } else {
    const int nch = num_chunks(a.V);
    row_stats_kernel<E, VEC, false><<<dim3(rows * nch), blk, 0, s>>>(a, stats, 0, 0u);
    if (a.gamma > 0)
      pair_overlap_kernel<E, VEC><<<dim3((size_t)a.B * a.gamma * nch), blk, 0, s>>>(a, stats, pair_stats);
  }
  finish_kernel<E, VEC><<<dim3(a.B), blk, 0, s>>>(a, stats, pair_stats);
  return hipGetLastError();
}

}  // namespace

size_t multipass_workspace_bytes(int B, int gamma, int V) { return layout(B, gamma, V).total; }

hipError_t multipass_launch(const VerifyArgs& a, hipStream_t s) {
  const size_t esz = a.dtype == SPEC_BF16 ? 2 : 4;
  const bool aligned = ((uintptr_t)a.target % 16 == 0) && (a.gamma == 0 || (uintptr_t)a.draft % 16 == 0) &&
                       ((size_t)a.V * esz) % 16 == 0;
  if (a.dtype == SPEC_BF16)
    return aligned ? launch_typed<BF16, true>(a, s) : launch_typed<BF16, false>(a, s);
  return aligned ? launch_typed<F32, true>(a, s) : launch_typed<F32, false>(a, s);
}

}  // namespace specv
