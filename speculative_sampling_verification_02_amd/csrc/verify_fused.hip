// Fused read-once verification path for gfx950.
//
// One persistent kernel whose grid fits the device's residency limit, so all
// of its workgroups run at once.  The vocabulary is cut into tiles of
// PER * 256 tokens.  Most workgroups form compute teams of K = ceil(V / tile).
// A team owns one work item at a time, one tile per workgroup:
//   pair item (b, i), i < gamma:  tiles of target row p_i and draft row q_i
//   bonus item b:                 tiles of target row p_gamma
// Teams step through the items round-robin.  Every logit is read from HBM once.
//
// Pair item, T > 0 (the only place a compute workgroup waits):
//   1. Load the tile's two rows.  Keep e = exp2((l - m_t) k) per token in
//      registers (m_t = the thread's maximum; k = log2(e) / T).
//   2. Publish the tile's (max, sum) of both rows.  Wait until all K tiles of
//      the pair have published.
//   3. Every member combines the K partials in the same order.  It then forms
//      its share of alpha = sum min(p, q) and of the residual mass
//      sum max(0, p - q) from the registers, and publishes both.
// Argmax-mode pairs and bonus items publish a single partial per tile.
//
// The remaining workgroups are finishers.  A finisher waits until all K tiles
// of an item have published.  It then computes alpha and the fp64 ratio test,
// and draws the item's sample: the residual of a rejected pair, or the bonus
// token.  To draw it, it finds the tile holding u * mass and scans that tile
// again with all loads issued up front.  The finisher of a sequence's bonus
// item then waits for the sequence's pair results, forms n and writes the
// outputs.  Compute workgroups never wait for finishers, and finishers of pair
// items wait only for compute workgroups, so every wait ends.
//
// The exchange slots live in the caller's workspace.  Zero means "not yet
// published"; the last reader of each slot sets it back to zero, so a call
// that completes leaves the workspace as it found it (all zero) and no clearing
// launch is needed.  Every wait is bounded; a wait that gives up publishes a
// poison word downstream and the sequence reports n_accepted = -1.
//
// Page abbreviations: [FI] intuitivepapers.ai "Fast Inference from Transformers
// via Speculative Decoding"; [SD] nonconvexcard "Speculative Decoding".

#include <float.h>
#include <math.h>

#include <algorithm>

#include "common.hpp"
#include "specverify.h"
#include "verify_internal.hpp"

namespace specv {
namespace {

// Tokens per thread per row (the tile is 256 times this), the share of
// resident workgroups that finish items (1 / SPECV_FUSED_FIN_DIV), and whether
// a compute workgroup double-buffers its tiles across items.
#ifndef SPECV_FUSED_PER
#define SPECV_FUSED_PER 32
#endif
#ifndef SPECV_FUSED_FIN_DIV
#define SPECV_FUSED_FIN_DIV 8
#endif
#ifndef SPECV_FUSED_PREFETCH
#define SPECV_FUSED_PREFETCH 0
#endif
constexpr int kThreads = 256;
constexpr int kMaxTeam = 128;            // longest supported row: 128 tiles
constexpr unsigned kSpinIters = 1u << 20;

// Published partials are 64-bit words.  A word whose low 32 bits are kEmpty
// has not been written yet.  The low word of every published word is nonzero:
// floats are stored with +0.0 replaced by -0.0 (same value), and the pair
// result carries a marker bit.  kPoison (a NaN pattern no computation here
// produces) marks a slot whose producer gave up waiting.
constexpr uint32_t kEmpty = 0u;
constexpr uint32_t kPoison = 0xffffffffu;
constexpr uint32_t kResMark = 2u;  // pair result: bit 0 = accepted, bit 1 = published

struct FusedParams {
  VerifyArgs a;
  int K;          // tiles per row: the team size
  int tile;       // tokens per tile
  int n_pairs;    // B * gamma
  int n_items;    // B * (gamma + 1): pairs, then one bonus item per sequence
  int nteams;     // compute teams
  int nfin;       // finisher workgroups
  uint64_t* part1;     // [n_items][K][2]  (max, sum) of p and q, or argmax (value, index)
  uint64_t* part2;     // [n_pairs][K]     (overlap share, residual mass share)
  uint64_t* pair_res;  // [n_pairs]        (accept flag | kResMark, sampled token)
};

// ------------------------------------------------------------- cross-WG sync
//
// One workgroup hands data to another only through naturally aligned 64-bit
// relaxed agent-scope atomic stores and loads.  These are single-copy atomic,
// and on gfx950 device-coherent across XCDs (the SC1 scope bit), with no
// cache writeback or invalidate.  A reader polls a slot until it no longer
// holds the kEmpty sentinel, and the poll returns the data itself.  There is
// no read-modify-write atomic anywhere: atomics to one address serialise
// across the device and cost about as much as the work they coordinate.

// Bits of a float for the low word of a published slot: never kEmpty.
__device__ inline uint32_t nz_bits(float a) {
  const uint32_t u = __float_as_uint(a);
  return u == 0u ? 0x80000000u : u;
}
__device__ inline uint64_t pack2(float a, float b) {
  return (uint64_t)nz_bits(a) | ((uint64_t)__float_as_uint(b) << 32);
}
__device__ inline uint64_t pack2i(uint32_t a, uint32_t b) { return (uint64_t)a | ((uint64_t)b << 32); }
__device__ inline float lo_f(uint64_t v) { return __uint_as_float((uint32_t)v); }
__device__ inline float hi_f(uint64_t v) { return __uint_as_float((uint32_t)(v >> 32)); }
__device__ inline bool published(uint64_t v) { return (uint32_t)v != kEmpty; }
__device__ inline bool poisoned(uint64_t v) { return (uint32_t)v == kPoison; }

__device__ inline void st_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint64_t ld_u64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave 0 polls n consecutive 64-bit slots until every one is published and
// copies them to lds[0..n).  Returns true, uniformly over the workgroup, if all
// arrived and none is poisoned.  Gives up after kSpinIters polls, so the kernel
// always terminates.  Called by the whole workgroup.
__device__ inline bool gather(const uint64_t* slots, int n, uint64_t* lds) {
  __shared__ int ok_s;
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    unsigned it = 0;
    bool ok = true;
    for (int base = 0; base < n && ok; base += kWave) {
      const int c = base + lane;
      while (true) {
        const uint64_t v = c < n ? ld_u64(slots + c) : pack2i(1u, 0u);
        if (c < n) lds[c] = v;
        if (__all(published(v))) {
          ok = !__any(poisoned(v));
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        if (++it >= kSpinIters) {
          ok = false;
          break;
        }
      }
    }
    if (lane == 0) ok_s = ok;
  }
  __syncthreads();
  return ok_s != 0;
}

// gather() over two slot ranges at once: [a, a + na) -> la and [b, b + nb) -> lb.
__device__ inline bool gather2(const uint64_t* a, int na, uint64_t* la, const uint64_t* b, int nb, uint64_t* lb) {
  __shared__ int ok_s;
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x, n = na + nb;
    unsigned it = 0;
    bool ok = true;
    for (int base = 0; base < n && ok; base += kWave) {
      const int c = base + lane;
      while (true) {
        uint64_t v = pack2i(1u, 0u);
        if (c < na) {
          v = ld_u64(a + c);
          la[c] = v;
        } else if (c < n) {
          v = ld_u64(b + (c - na));
          lb[c - na] = v;
        }
        if (__all(published(v))) {
          ok = !__any(poisoned(v));
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        if (++it >= kSpinIters) {
          ok = false;
          break;
        }
      }
    }
    if (lane == 0) ok_s = ok;
  }
  __syncthreads();
  return ok_s != 0;
}

// Set n slots back to kEmpty (wave 0).  Only the last reader of a slot clears
// it, after its own gather has returned the slot's data.
__device__ inline void clear_slots(uint64_t* slots, int n) {
  if (threadIdx.x < kWave)
    for (int c = threadIdx.x; c < n; c += kWave) st_u64(slots + c, 0ull);
}

// ------------------------------------------------------------- tile loading

// This thread's PER tokens of a row tile, in token order within each
// 256 * kVec step.  Tokens >= V read as -inf.  load_raw only issues the loads,
// so both rows of a pair can be in flight before either is unpacked.
template <class E, int PER>
struct RawTile {
  static constexpr int NS = PER / E::kVec;
  u32x4 v[NS];
};

// The loads are unconditional: a vector past the end of the row reads the
// row's last vector instead (V >= kVec), and unpack_tile masks it to -inf.
// Straight-line code keeps the raw tiles in registers.
template <class E, int PER>
__device__ inline void load_raw(const typename E::storage* row, int tile_lo, int V, RawTile<E, PER>& r) {
#pragma unroll
  for (int s = 0; s < RawTile<E, PER>::NS; ++s) {
    const int j0 = tile_lo + (s * kThreads + (int)threadIdx.x) * E::kVec;
    r.v[s] = load_stream(row + min(j0, V - E::kVec));
  }
}

template <class E, int PER>
__device__ inline void unpack_tile(const RawTile<E, PER>& r, int tile_lo, int V, float (&x)[PER]) {
  if (tile_lo + kThreads * PER <= V) {  // the whole tile is in range: no per-token select
#pragma unroll
    for (int s = 0; s < RawTile<E, PER>::NS; ++s) {
      float t[E::kVec];
      E::unpack(r.v[s], t);
#pragma unroll
      for (int v = 0; v < E::kVec; ++v) x[s * E::kVec + v] = t[v];
    }
    return;
  }
#pragma unroll
  for (int s = 0; s < RawTile<E, PER>::NS; ++s) {
    const int j0 = tile_lo + (s * kThreads + (int)threadIdx.x) * E::kVec;
    float t[E::kVec];
    E::unpack(r.v[s], t);
#pragma unroll
    for (int v = 0; v < E::kVec; ++v) x[s * E::kVec + v] = j0 < V ? t[v] : -INFINITY;
  }
}

template <class E, int PER>
__device__ inline void load_tile(const typename E::storage* row, int tile_lo, int V, float (&x)[PER]) {
  RawTile<E, PER> r;
  load_raw<E, PER>(row, tile_lo, V, r);
  unpack_tile<E, PER>(r, tile_lo, V, x);
}

__device__ inline int tile_token(int tile_lo, int idx, int kvec) {
  return tile_lo + ((idx / kvec) * kThreads + (int)threadIdx.x) * kvec + idx % kvec;
}

// Thread maximum with four independent max chains (short dependency chains).
template <int PER>
__device__ inline float thread_max(const float (&x)[PER]) {
  static_assert(PER % 4 == 0, "PER must be a multiple of 4");
  // three-input maxima (v_max3_f32): half an instruction per token
  float m0 = fmaxf(x[0], x[1]), m1 = fmaxf(x[2], x[3]);
#pragma unroll
  for (int i = 4; i < PER; i += 4) {
    m0 = fmaxf(m0, fmaxf(x[i], x[i + 1]));
    m1 = fmaxf(m1, fmaxf(x[i + 2], x[i + 3]));
  }
  return fmaxf(m0, m1);
}

// sum_i exp2((x_i - m) k) over four independent accumulators.  With KEEP the
// exponentials replace x in place.  m == -inf (no finite logit) gives 0.
template <int PER, bool KEEP>
__device__ inline float thread_exp_sum(float (&x)[PER], float m, float k) {
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  if (m != -INFINITY) {
#pragma unroll
    for (int i = 0; i < PER; i += 4) {
      const float e0 = fast_exp2((x[i] - m) * k), e1 = fast_exp2((x[i + 1] - m) * k);
      const float e2 = fast_exp2((x[i + 2] - m) * k), e3 = fast_exp2((x[i + 3] - m) * k);
      if (KEEP) {
        x[i] = e0;
        x[i + 1] = e1;
        x[i + 2] = e2;
        x[i + 3] = e3;
      }
      s0 += e0;
      s1 += e1;
      s2 += e2;
      s3 += e3;
    }
  } else if (KEEP) {
#pragma unroll
    for (int i = 0; i < PER; ++i) x[i] = 0.f;
  }
  return (s0 + s1) + (s2 + s3);
}

// The thread's (max, sum) -> the workgroup's (max, sum) relative to that max,
// for two rows at once: returns (M_p, S_p, M_q, S_q).
__device__ inline float4 block_lse2(float mp, float sp, float mq, float sq, float k, float* lds) {
  const float2 M = block_max2(mp, mq, lds);
  const float wp = mp == -INFINITY ? 0.f : sp * fast_exp2((mp - M.x) * k);
  const float wq = mq == -INFINITY ? 0.f : sq * fast_exp2((mq - M.y) * k);
  const float2 S = block_sum2(wp, wq, lds);
  return make_float4(M.x, S.x, M.y, S.y);
}

template <class E, int PER>
__device__ inline ArgMax thread_argmax(const float (&x)[PER], int tile_lo) {
  ArgMax best{-INFINITY, 0x7fffffff};
#pragma unroll
  for (int i = 0; i < PER; ++i) best = argmax_better(best, ArgMax{x[i], tile_token(tile_lo, i, E::kVec)});
  return best;
}

// Row normaliser over the K staged tiles, combined in one fixed order so that
// every workgroup that calls it gets bit-identical values.  `sel` picks the
// (max, sum) half of the float4 partial: 0 -> (x, y), 1 -> (z, w).
struct Norm {
  float M;
  float invS;
  double S;
};

// Normalisers of both rows (sel 0: (x, y) halves, sel 1: (z, w) halves) from
// the K staged partials, computed by wave 0 in one fixed order.
__device__ inline void team_norm2(const float4* st, int K, float k, Norm* np, Norm* nq) {
  __shared__ float sM[2];
  __shared__ double sS[2];
  if (threadIdx.x < kWave) {
    float Mp = -INFINITY, Mq = -INFINITY;
    for (int c = threadIdx.x; c < K; c += kWave) {
      Mp = fmaxf(Mp, st[c].x);
      Mq = fmaxf(Mq, st[c].z);
    }
    Mp = wave_max(Mp);
    Mq = wave_max(Mq);
    double Sp = 0.0, Sq = 0.0;
    for (int c = threadIdx.x; c < K; c += kWave) {
      const float4 v = st[c];
      if (v.x != -INFINITY) Sp += (double)v.y * (double)fast_exp2((v.x - Mp) * k);
      if (v.z != -INFINITY) Sq += (double)v.w * (double)fast_exp2((v.z - Mq) * k);
    }
    Sp = wave_sum(Sp);
    Sq = wave_sum(Sq);
    if (threadIdx.x == 0) {
      sM[0] = Mp;
      sM[1] = Mq;
      sS[0] = Sp;
      sS[1] = Sq;
    }
  }
  __syncthreads();
  *np = Norm{sM[0], (float)(1.0 / sS[0]), sS[0]};
  *nq = Norm{sM[1], (float)(1.0 / sS[1]), sS[1]};
  __syncthreads();
}

// Tile holding theta among K tile masses in tile order: wave 0 scans the
// masses (fp64, fixed order) and takes the first tile whose running mass
// exceeds theta.  *tile and *rest (theta minus the mass before that tile) are
// LDS variables, valid for the whole workgroup on return.  If rounding leaves
// theta past every tile, the last tile with mass is taken.  Called by the
// whole workgroup.
template <class MassFn>
__device__ inline void wave_pick_tile(int K, double theta, MassFn mass, int* tile, float* rest) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    double carry = 0.0;
    int pick = -1, last = 0;
    float left = 0.f;
    for (int base = 0; base < K; base += kWave) {
      const int c = base + lane;
      const double w = c < K ? mass(c) : 0.0;
      const double incl = carry + wave_inclusive_scan(w);
      const unsigned long long hit = __ballot(c < K && w > 0.0 && incl > theta);
      const unsigned long long pos = __ballot(c < K && w > 0.0);
      if (pos) last = base + 63 - __clzll(pos);
      if (hit) {
        const int l = __ffsll((long long)hit) - 1;
        const double before = __shfl(incl - w, l, kWave);
        pick = base + l;
        left = (float)(theta - before);
        break;
      }
      carry = __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) {
      *tile = pick >= 0 ? pick : last;
      *rest = pick >= 0 ? left : (float)(theta - carry);
    }
  }
  __syncthreads();
}

// ------------------------------------------------------ compute workgroups
// A compute workgroup only streams its tile and publishes partials.  It
// never waits for a finisher.  Its loop is software-pipelined: the next
// item's tile loads are issued before the current item is processed (two
// register buffers, used alternately), so the load latency overlaps the
// current item's arithmetic and wait.

template <class E>
__device__ inline const typename E::storage* trow(const VerifyArgs& a, int b, int i) {
  return static_cast<const typename E::storage*>(a.target) + ((size_t)b * (a.gamma + 1) + i) * (size_t)a.V;
}
template <class E>
__device__ inline const typename E::storage* drow(const VerifyArgs& a, int b, int i) {
  return static_cast<const typename E::storage*>(a.draft) + ((size_t)b * a.gamma + i) * (size_t)a.V;
}

// The raw tiles of one item: both rows of a pair, or the bonus row in `p`.
template <class E, int PER>
struct RawPair {
  RawTile<E, PER> p, q;
};

template <class E, int PER>
__device__ __attribute__((always_inline)) void issue_item(const FusedParams& P, int item, int rank, RawPair<E, PER>& r) {
  const VerifyArgs& a = P.a;
  const int lo = rank * P.tile;
  const bool pair = item < P.n_pairs;
  const int b = pair ? item / a.gamma : item - P.n_pairs;
  const int i = pair ? item % a.gamma : a.gamma;
  load_raw<E, PER>(trow<E>(a, b, i), lo, a.V, r.p);
  if (pair) load_raw<E, PER>(drow<E>(a, b, i), lo, a.V, r.q);
}

// LDS view of an item's published first partials.
__device__ inline void unpack_part1(const uint64_t* w, int K, float4* st) {
  for (int c = threadIdx.x; c < K; c += kThreads)
    st[c] = make_float4(lo_f(w[2 * c]), hi_f(w[2 * c]), lo_f(w[2 * c + 1]), hi_f(w[2 * c + 1]));
  __syncthreads();
}

// Pair item, T > 0: the tile stays in registers across the team's one wait.
template <class E, int PER>
__device__ __attribute__((always_inline)) void pair_compute_sample(const FusedParams& P, int item, int rank, const RawPair<E, PER>& raw) {
  __shared__ float lds_f[2 * kMaxWaves];
  __shared__ uint64_t w1[2 * kMaxTeam];
  __shared__ float4 st1[kMaxTeam];
  const VerifyArgs& a = P.a;
  const int G = a.gamma, K = P.K;
  const int b = item / G, i = item % G;
  const float k = a.k;
  const int lo = rank * P.tile;

  float ep[PER], eq[PER];
  unpack_tile<E, PER>(raw.p, lo, a.V, ep);
  unpack_tile<E, PER>(raw.q, lo, a.V, eq);
  const float mp = thread_max<PER>(ep), mq = thread_max<PER>(eq);
  const float sp = thread_exp_sum<PER, true>(ep, mp, k), sq = thread_exp_sum<PER, true>(eq, mq, k);
  const float4 bl = block_lse2(mp, sp, mq, sq, k, lds_f);
  uint64_t* mine = P.part1 + ((size_t)item * K + rank) * 2;
  if (threadIdx.x == 0) {
    st_u64(mine, pack2(bl.x, bl.y));
    st_u64(mine + 1, pack2(bl.z, bl.w));
  }

  // wait for the other tiles of this pair; the poll returns their partials
  if (!gather(P.part1 + (size_t)item * K * 2, 2 * K, w1)) {
    if (threadIdx.x == 0) st_u64(P.part2 + (size_t)item * K + rank, pack2i(kPoison, 0u));
    return;
  }
  unpack_part1(w1, K, st1);
  Norm np, nq;
  team_norm2(st1, K, k, &np, &nq);
  const float fp = mp == -INFINITY ? 0.f : fast_exp2((mp - np.M) * k) * np.invS;
  const float fq = mq == -INFINITY ? 0.f : fast_exp2((mq - nq.M) * k) * nq.invS;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  if (fp > 0.f && fq > 0.f) {
    // sum min(ep fp, eq fq) = fq * sum min(ep (fp / fq), eq); ep <= 1, so the
    // clamp keeps ep * r finite
    const float r = fminf(fp / fq, FLT_MAX);
#pragma unroll
    for (int j = 0; j < PER; j += 4) {
      a0 += fminf(ep[j] * r, eq[j]);
      a1 += fminf(ep[j + 1] * r, eq[j + 1]);
      a2 += fminf(ep[j + 2] * r, eq[j + 2]);
      a3 += fminf(ep[j + 3] * r, eq[j + 3]);
    }
  }
  const float alpha_t = ((a0 + a1) + (a2 + a3)) * fq;
  const float res_t = fmaxf(sp * fp - alpha_t, 0.f);  // sum max(0, p - q) = sum p - sum min(p, q)
  const float2 c2 = block_sum2(alpha_t, res_t, lds_f);
  const float alpha_c = c2.x, res_c = c2.y;
  if (threadIdx.x == 0) st_u64(P.part2 + (size_t)item * K + rank, pack2(alpha_c, res_c));
}

// Pair item at T = 0, or a bonus item: one pass, no waiting.
template <class E, int PER, bool ARGMAX>
__device__ __attribute__((always_inline)) void single_pass_compute(const FusedParams& P, int item, int rank, const RawPair<E, PER>& raw) {
  __shared__ float lds_f[2 * kMaxWaves];
  __shared__ int lds_i[kMaxWaves];
  const VerifyArgs& a = P.a;
  const int G = a.gamma, K = P.K;
  const int lo = rank * P.tile;
  uint64_t w0, w1;
  if (item < P.n_pairs) {  // argmax pair
    float xp[PER], xq[PER];
    unpack_tile<E, PER>(raw.p, lo, a.V, xp);
    unpack_tile<E, PER>(raw.q, lo, a.V, xq);
    const ArgMax ap = block_argmax(thread_argmax<E, PER>(xp, lo), lds_f, lds_i);
    const ArgMax aq = block_argmax(thread_argmax<E, PER>(xq, lo), lds_f, lds_i);
    w0 = pack2i(nz_bits(ap.v), (uint32_t)ap.i);
    w1 = pack2i(nz_bits(aq.v), (uint32_t)aq.i);
  } else {
    float x[PER];
    unpack_tile<E, PER>(raw.p, lo, a.V, x);
    if constexpr (ARGMAX) {
      const ArgMax ab = block_argmax(thread_argmax<E, PER>(x, lo), lds_f, lds_i);
      w0 = pack2i(nz_bits(ab.v), (uint32_t)ab.i);
    } else {
      const float m = thread_max<PER>(x);
      const float sm = thread_exp_sum<PER, false>(x, m, a.k);
      const float4 bl = block_lse2(m, sm, -INFINITY, 0.f, a.k, lds_f);
      w0 = pack2(bl.x, bl.y);
    }
    w1 = pack2i(0x80000000u, 0u);  // unused second word: (-0, 0), published
  }
  if (threadIdx.x == 0) {
    uint64_t* mine = P.part1 + ((size_t)item * K + rank) * 2;
    st_u64(mine, w0);
    st_u64(mine + 1, w1);
  }
}

// ---------------------------------------------------- finisher workgroups

// Combine K argmax partials (value, index) in tile order.
__device__ inline ArgMax combine_argmax(const uint64_t* w, int K, int half) {
  ArgMax g{-INFINITY, 0x7fffffff};
  for (int c = 0; c < K; ++c) {
    const uint64_t v = w[2 * c + half];
    g = argmax_better(g, ArgMax{lo_f(v), (int)(uint32_t)(v >> 32)});
  }
  return g;
}

// Pair item: alpha, the ratio test and, after a rejection, the residual
// sample.  Publishes (accept, token) for the sequence's bonus finisher.
template <class E, int PER, bool ARGMAX>
__device__ void finish_pair(const FusedParams& P, int item) {
  __shared__ float lds_f[kMaxWaves];
  __shared__ int lds_i[kMaxWaves];
  __shared__ uint64_t w1[2 * kMaxTeam], w2[kMaxTeam];
  __shared__ float4 st1[kMaxTeam];
  __shared__ int tile_s, acc_s;
  __shared__ float rest_s;
  const VerifyArgs& a = P.a;
  const int G = a.gamma, K = P.K;
  const int b = item / G, i = item % G;
  const float k = a.k;
  const auto* prow = trow<E>(a, b, i);
  const auto* qrow = drow<E>(a, b, i);
  const size_t o = (size_t)b * G + i;

  if constexpr (ARGMAX) {
    if (!gather(P.part1 + (size_t)item * K * 2, 2 * K, w1)) {
      if (threadIdx.x == 0) st_u64(P.pair_res + item, pack2i(kPoison, 0u));
      return;
    }
    clear_slots(P.part1 + (size_t)item * K * 2, 2 * K);
    if (threadIdx.x == 0) {
      // keep x iff it is the target's argmax; alpha is the indicator that the
      // two argmaxes agree ([FI] "Speculative sampling", temperature to zero)
      const ArgMax gp = combine_argmax(w1, K, 0), gq = combine_argmax(w1, K, 1);
      const int x = a.tokens[o];
      if (a.alpha) a.alpha[o] = gp.i == gq.i ? 1.f : 0.f;
      if (a.p_draft) a.p_draft[o] = x == gp.i ? 1.f : 0.f;
      if (a.q_draft) a.q_draft[o] = x == gq.i ? 1.f : 0.f;
      st_u64(P.pair_res + item, pack2i((x == gp.i ? 1u : 0u) | kResMark, (uint32_t)gp.i));
    }
    return;
  } else {
    // the ratio-test inputs do not depend on the partials: fetch them first
    int x = 0;
    float lp = 0.f, lq = 0.f;
    if (threadIdx.x == 0) {
      x = a.tokens[o];
      if (x >= 0 && x < a.V) {
        lp = E::at(prow, x);
        lq = E::at(qrow, x);
      }
    }
    // part2 is published after part1 by every tile; polling both in one pass
    // returns once both are complete
    if (!gather2(P.part1 + (size_t)item * K * 2, 2 * K, w1, P.part2 + (size_t)item * K, K, w2)) {
      if (threadIdx.x == 0) st_u64(P.pair_res + item, pack2i(kPoison, 0u));
      return;
    }
    // every member has published part2, so every member is done reading part1
    clear_slots(P.part1 + (size_t)item * K * 2, 2 * K);
    clear_slots(P.part2 + (size_t)item * K, K);
    unpack_part1(w1, K, st1);
    Norm np, nq;
    team_norm2(st1, K, k, &np, &nq);
    // alpha and the residual mass (wave 0, fixed order), and the tile holding
    // u * mass, found with a wave-wide prefix scan of the tile masses
    __shared__ double alpha_s, sw_s;
    if (threadIdx.x < kWave) {
      double al = 0.0, sw = 0.0;
      for (int c = threadIdx.x; c < K; c += kWave) {
        al += (double)lo_f(w2[c]);
        sw += (double)hi_f(w2[c]);
      }
      al = wave_sum(al);
      sw = wave_sum(sw);
      if (threadIdx.x == 0) {
        alpha_s = al;
        sw_s = sw;
      }
    }
    if (threadIdx.x == 0) {
      double px = 0.0, qx = 0.0;
      if (x >= 0 && x < a.V) {
        px = exp2(((double)lp - (double)np.M) * (double)k) / np.S;
        qx = exp2(((double)lq - (double)nq.M) * (double)k) / nq.S;
      }
      // accept iff u <= min(1, p(x) / q(x)) ([FI] Algorithm 1 step 3; [SD]
      // "The algorithm").  q(x) = 0 keeps the draft when p(x) > 0 (the ratio
      // is +inf) and rejects it when p(x) = 0 (0/0).
      const double u = (double)a.uniforms[(size_t)b * (G + 1) + i];
      if (qx > 0.0) {
        const double ratio = px / qx;
        acc_s = (ratio >= 1.0) || (u <= ratio);
      } else {
        acc_s = px > 0.0;
      }
      if (a.p_draft) a.p_draft[o] = (float)px;
      if (a.q_draft) a.q_draft[o] = (float)qx;
    }
    __syncthreads();
    if (threadIdx.x == 0 && a.alpha) a.alpha[o] = (float)alpha_s;
    const int acc_i = acc_s;
    int mode = 0;
    if (!acc_i) {
      const double uf = (double)a.uniforms[(size_t)b * (G + 1) + G];
      if (sw_s > 0.0) {
        mode = 1;  // residual max(0, p_i - q_i) ([FI] eq. (2); [SD] "Exactness")
        wave_pick_tile(K, uf * sw_s, [&](int c) { return (double)hi_f(w2[c]); }, &tile_s, &rest_s);
      } else {
        mode = 2;  // no residual mass: sample p_i itself
        wave_pick_tile(K, uf * np.S, [&](int c) {
          return st1[c].x == -INFINITY ? 0.0 : (double)st1[c].y * (double)fast_exp2((st1[c].x - np.M) * k);
        }, &tile_s, &rest_s);
      }
    }
    int t = 0;
    if (mode) {
      const float Mp = np.M, invSp = np.invS, Mq = nq.M, invSq = nq.invS;
      const int tlo = tile_s * P.tile;
      if (mode == 1)
        t = tile_search<E, PER, kThreads>(prow, qrow, tlo, a.V, rest_s, [&](float xp, float xq) {
          return fmaxf(fast_exp2((xp - Mp) * k) * invSp - fast_exp2((xq - Mq) * k) * invSq, 0.f);
        }, lds_f, lds_i);
      else
        t = tile_search<E, PER, kThreads>(prow, nullptr, tlo, a.V, rest_s, [&](float xp, float) {
          return fast_exp2((xp - Mp) * k);
        }, lds_f, lds_i);
    }
    if (threadIdx.x == 0) st_u64(P.pair_res + item, pack2i((uint32_t)acc_s | kResMark, (uint32_t)t));
  }
}

// Bonus item: the token from p_gamma ([FI] Algorithm 1 step 4), then the
// sequence's outputs once every pair result of the sequence is published.
template <class E, int PER, bool ARGMAX>
__device__ void finish_bonus(const FusedParams& P, int item) {
  __shared__ float lds_f[kMaxWaves];
  __shared__ int lds_i[kMaxWaves];
  __shared__ uint64_t w1[2 * kMaxTeam], res[SPEC_MAX_GAMMA];
  __shared__ float4 st1[kMaxTeam];
  __shared__ int tile_s;
  __shared__ float rest_s;
  const VerifyArgs& a = P.a;
  const int G = a.gamma, K = P.K;
  const int b = item - P.n_pairs;
  const float k = a.k;
  const auto* row = trow<E>(a, b, G);
  const bool ok1 = gather(P.part1 + (size_t)item * K * 2, 2 * K, w1);
  if (ok1) clear_slots(P.part1 + (size_t)item * K * 2, 2 * K);
  int t_bonus = -1;
  if (!ok1) {
  } else if constexpr (ARGMAX) {
    t_bonus = combine_argmax(w1, K, 0).i;
  } else {
    unpack_part1(w1, K, st1);
    Norm n, unused;
    team_norm2(st1, K, k, &n, &unused);
    const double uf = (double)a.uniforms[(size_t)b * (G + 1) + G];
    wave_pick_tile(K, uf * n.S, [&](int c) {
      return st1[c].x == -INFINITY ? 0.0 : (double)st1[c].y * (double)fast_exp2((st1[c].x - n.M) * k);
    }, &tile_s, &rest_s);
    const float M = n.M;
    t_bonus = tile_search<E, PER, kThreads>(row, nullptr, tile_s * P.tile, a.V, rest_s,
                                            [&](float xp, float) { return fast_exp2((xp - M) * k); }, lds_f,
                                            lds_i);
  }
  // the sequence's pair results (published by other finishers)
  const bool ok2 = gather(P.pair_res + (size_t)b * G, G, res);
  if (ok2) clear_slots(P.pair_res + (size_t)b * G, G);
  if (threadIdx.x == 0) {
    if (ok1 && ok2) {
      int n = 0;
      while (n < G && ((uint32_t)res[n] & 1u) != 0u) ++n;
      a.n_out[b] = n;
      a.t_out[b] = n < G ? (int)(uint32_t)(res[n] >> 32) : t_bonus;
    } else {
      a.n_out[b] = -1;  // a wait gave up (the device was shared): no result
      a.t_out[b] = -1;
    }
  }
}

// --------------------------------------------------------------- the kernel

template <class E, int PER, bool ARGMAX>
__device__ __attribute__((always_inline)) void compute_item(const FusedParams& P, int item, int rank, const RawPair<E, PER>& raw) {
  if (!ARGMAX && item < P.n_pairs)
    pair_compute_sample<E, PER>(P, item, rank, raw);
  else
    single_pass_compute<E, PER, ARGMAX>(P, item, rank, raw);
}

template <class E, int PER, bool ARGMAX>
__global__ __launch_bounds__(kThreads) void fused_kernel(FusedParams P) {
  const int ncompute = P.nteams * P.K;
  if ((int)blockIdx.x < ncompute) {
    const int team = blockIdx.x / P.K, rank = blockIdx.x % P.K;
#if SPECV_FUSED_PREFETCH
    // two register buffers: the next item's loads are in flight while this
    // item is computed
    RawPair<E, PER> A, B;
    int item = team;
    if (item < P.n_items) issue_item<E, PER>(P, item, rank, A);
    while (item < P.n_items) {
      int next = item + P.nteams;
      if (next < P.n_items) issue_item<E, PER>(P, next, rank, B);
      compute_item<E, PER, ARGMAX>(P, item, rank, A);
      item = next;
      if (item >= P.n_items) break;
      next = item + P.nteams;
      if (next < P.n_items) issue_item<E, PER>(P, next, rank, A);
      compute_item<E, PER, ARGMAX>(P, item, rank, B);
      item = next;
    }
#else
    for (int item = team; item < P.n_items; item += P.nteams) {
      RawPair<E, PER> A;
      issue_item<E, PER>(P, item, rank, A);
      compute_item<E, PER, ARGMAX>(P, item, rank, A);
    }
#endif
  } else {
    // pairs precede bonus items in the item order, so a finisher never waits
    // on an item it has yet to finish itself
    for (int item = blockIdx.x - ncompute; item < P.n_items; item += P.nfin) {
      if (item < P.n_pairs)
        finish_pair<E, PER, ARGMAX>(P, item);
      else
        finish_bonus<E, PER, ARGMAX>(P, item);
    }
  }
}

constexpr int kFinisherDiv = SPECV_FUSED_FIN_DIV;

template <class E>
constexpr int per_thread() {
  return SPECV_FUSED_PER;
}

int tiles_for(int V, int dtype) {
  const int tile = kThreads * (dtype == SPEC_BF16 ? per_thread<BF16>() : per_thread<F32>());
  return (V + tile - 1) / tile;
}

// Slot layout.  The size does not depend on the dtype (both use the larger
// tile count), so one zeroed workspace serves calls of either dtype.
struct Layout {
  size_t off_part1, off_part2, off_res, total;
};

Layout layout(int B, int gamma, int V) {
  const size_t K = std::max(tiles_for(V, SPEC_BF16), tiles_for(V, SPEC_F32));
  const size_t n_items = (size_t)B * (gamma + 1), n_pairs = (size_t)B * gamma;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  Layout L{};
  L.off_part1 = 0;
  L.off_part2 = up(L.off_part1 + 16 * n_items * K);
  L.off_res = up(L.off_part2 + 8 * n_pairs * K);
  L.total = up(L.off_res + 8 * n_pairs);
  return L;
}

// Workgroups of `kern` that fit on the device at once.
template <class Kern>
hipError_t resident_blocks(Kern kern, long* out) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kThreads, 0);
  *out = (long)per_cu * cus;
  return e;
}

template <class E, bool ARGMAX>
hipError_t launch(const VerifyArgs& a, hipStream_t s) {
  constexpr int PER = per_thread<E>();
  const Layout L = layout(a.B, a.gamma, a.V);
  char* ws = static_cast<char*>(a.ws);
  FusedParams P{};
  P.a = a;
  P.tile = kThreads * PER;
  P.K = (a.V + P.tile - 1) / P.tile;
  P.n_pairs = a.B * a.gamma;
  P.n_items = a.B * (a.gamma + 1);
  P.part1 = reinterpret_cast<uint64_t*>(ws + L.off_part1);
  P.part2 = reinterpret_cast<uint64_t*>(ws + L.off_part2);
  P.pair_res = reinterpret_cast<uint64_t*>(ws + L.off_res);

  auto kern = fused_kernel<E, PER, ARGMAX>;
  long resident = 0;
  hipError_t e = resident_blocks(kern, &resident);
  if (e != hipSuccess) return e;
  // The grid never exceeds what is resident at once, so every team's members
  // run concurrently and every wait ends.
  P.nfin = (int)std::min<long>(P.n_items, std::max<long>(1, resident / kFinisherDiv));
  P.nteams = (int)std::min<long>(P.n_items, (resident - P.nfin) / P.K);
  if (P.nteams < 1) return hipErrorNotSupported;

  kern<<<dim3(P.nteams * P.K + P.nfin), dim3(kThreads), 0, s>>>(P);
  return hipGetLastError();
}

}  // namespace

size_t fused_workspace_bytes(int B, int gamma, int V) { return layout(B, gamma, V).total; }

bool fused_supported(int B, int gamma, int V, int dtype) {
  const int vec = dtype == SPEC_BF16 ? BF16::kVec : F32::kVec;
  return B >= 1 && V % vec == 0 && tiles_for(V, dtype) <= kMaxTeam && (size_t)B * (gamma + 1) < (1u << 30);
}

hipError_t fused_launch(const VerifyArgs& a, hipStream_t s) {
  if (!fused_supported(a.B, a.gamma, a.V, a.dtype)) return hipErrorNotSupported;
  if ((uintptr_t)a.target % 16 != 0 || (a.gamma > 0 && (uintptr_t)a.draft % 16 != 0)) return hipErrorNotSupported;
  const bool argmax = a.temperature == 0.f;
  if (a.dtype == SPEC_BF16) return argmax ? launch<BF16, true>(a, s) : launch<BF16, false>(a, s);
  return argmax ? launch<F32, true>(a, s) : launch<F32, false>(a, s);
}

}  // namespace specv
