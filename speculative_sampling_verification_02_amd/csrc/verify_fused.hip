// Fused read-once verification path for gfx950.
//
// One persistent kernel whose grid fits the device's residency limit, so all
// of its workgroups run at once.  Each row is cut into wave tiles of
// kWave * PER contiguous tokens, and each wave owns one wave tile.  A workgroup
// holds four waves, so its tile is four adjacent wave tiles.  Most workgroups
// form compute teams of K = ceil(V / (4 * kWave * PER)).  A team owns one
// work item at a time, one tile per workgroup:
//   pair item (b, i), i < gamma:  tiles of target row p_i and draft row q_i
//   bonus item b:                 tiles of target row p_gamma
// Teams step through the items round-robin.  Every logit is read from HBM once.
//
// Waves work on their own: every reduction is a wave-level DPP reduction and
// every partial is published per wave, so a compute workgroup meets at a
// barrier once per pair item and never otherwise.
//
// Pair item, T > 0 (the only place a compute workgroup waits):
//   1. Load the wave tile of both rows.  Keep e = exp2(l k - c_t) per token
//      in registers (c_t = the thread's maximum times k; k = log2(e) / T).
//   2. Publish the wave's (max, sum) of both rows.
//   3. Wave 0 waits until all 4K waves of the team have published, combines
//      the partials in one fixed order and hands both row normalisers to the
//      other waves through LDS (one barrier that waits on LDS only, so no
//      global load is held up by it).
//   4. Each wave forms its share of alpha = sum min(p, q) and of the residual
//      mass sum max(0, p - q) from its registers and publishes both.
// Argmax-mode pairs and bonus items publish a single partial per wave.
//
// The remaining workgroups are finishers.  A finisher waits until all wave
// tiles of an item have published.  It then computes alpha and the fp64 ratio
// test, and draws the item's sample: the residual of a rejected pair, or the
// bonus token.  To draw it, it finds the wave tile holding u * mass from the
// per-wave masses and scans that one tile (kWave * PER tokens) again.  The
// finisher of a sequence's bonus item then waits for the sequence's pair
// results, forms n and writes the outputs.  Compute workgroups never wait for
// finishers, and finishers of pair items wait only for compute workgroups, so
// every wait ends.
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
#include <limits.h>
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "specverify.h"
#include "verify_internal.hpp"

namespace specv {
namespace {

// Tokens per thread per row (the wave tile is kWave times this) for each
// dtype, and the share of resident workgroups that finish items
// (1 / kFinisherDiv).
constexpr int kPerBF16 = 32;
constexpr int kPerF32 = 32;
constexpr int kFinisherDiv = 8;
// Minimum waves per SIMD the register allocation must allow.
constexpr int kMinWaves = 3;
constexpr int kThreads = 256;
constexpr int kWavesPerGroup = kThreads / kWave;
constexpr int kMaxWaveTiles = 256;  // longest supported row: 256 wave tiles
// Polls a cross-workgroup wait makes before it gives up (spec_set_wait_limit
// can lower it for later launches, to test the give-up path).
constexpr unsigned kDefaultWaitPolls = 1u << 20;
unsigned g_wait_polls = kDefaultWaitPolls;

// Published partials are 64-bit words.  A word whose low 32 bits are kEmpty
// has not been written yet.  The low word of every published word is nonzero:
// floats are stored with +0.0 replaced by -0.0 (same value), and the pair
// result carries a marker bit.  kPoison (a NaN pattern no computation here
// produces) marks a slot whose producer gave up waiting.
constexpr uint32_t kEmpty = 0u;
constexpr uint32_t kPoison = 0xffffffffu;
constexpr uint32_t kResMark = 2u;  // pair result: bit 0 = accepted, bit 1 = published

// The bf16 T > 0 kernel for 16-byte aligned rows without extensions takes
// the bonus items two at a time (two sequences' bonus rows per team round)
// once the teams walk at least this many pairs each: one bonus row alone
// costs about three quarters of a pair's round, so pairing them saves rounds
// on long walks (B=256, gamma=8, V=256000: 524 -> 512 us; B=256, gamma=4,
// V=128256: 136.1 -> 135.7 us), while on short walks the single bonus items,
// given to the teams with fewer pairs, end the launch as soon (B=64,
// gamma=4: 42.9 either way).  The extended kernels keep single bonus items
// (ragged B=64: 33.4 against 34.9), and so do the kernels for rows that do
// not start on 16 bytes.
constexpr int kBonusUnitPairs = 10;

struct FusedParams {
  VerifyArgs a;
  int K;          // workgroups per team
  int W;          // wave tiles per row slot range: 4 K (the last few may lie past V)
  int n_pairs;    // B * gamma
  int n_items;    // B * (gamma + 1): pairs, then one bonus item per sequence
  int nteams;     // compute teams
  int nfin;       // finisher workgroups
  uint64_t* part1;     // [n_items][W][2]  (max, sum) of p and q, or argmax (value, index)
  uint64_t* part2;     // [n_pairs][W]     (overlap share, residual mass share)
  uint64_t* pair_res;  // [n_pairs]        (accept flag | kResMark, sampled token)
  unsigned polls;      // bound of every wait
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

// Workgroup barrier for LDS data only: the fences order LDS accesses, so the
// barrier waits for this wave's LDS operations but not for its outstanding
// global loads (a full __syncthreads() would drain those too).
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One wave polls n consecutive 64-bit slots until every one is published and
// copies them to lds[0..n).  Returns true, uniformly over the wave, if all
// arrived and none is poisoned.  Gives up after `limit` polls, so the kernel
// always terminates.  Called by all lanes of one wave.
__device__ inline bool wave_poll(const uint64_t* a, int na, uint64_t* la, const uint64_t* b, int nb,
                                 uint64_t* lb, unsigned limit) {
  const int lane = threadIdx.x & (kWave - 1), n = na + nb;
  unsigned it = 0;
  for (int base = 0; base < n; base += kWave) {
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
        if (__any(poisoned(v))) return false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      if (++it >= limit) return false;
    }
  }
  return true;
}

// The same for at most 2 kWave slots of one array: each poll reads every slot
// at once, so it costs one memory round trip (wave_poll polls 64 slots at a
// time, one round trip each).
__device__ inline bool wave_poll_once(const uint64_t* a, int n, uint64_t* lds, unsigned limit) {
  // the lane index is made opaque here, so the per-lane offsets are formed
  // at each wait instead of being hoisted out of the compute loop (where they
  // would hold registers through the whole item)
  int lane;
  asm volatile("" : "=v"(lane) : "0"((int)(threadIdx.x & (kWave - 1))));
  const int c0 = lane, c1 = lane + kWave;
  const uint32_t o0 = (uint32_t)c0 * 8u, o1 = (uint32_t)c1 * 8u;
  const char* base = reinterpret_cast<const char*>(a);
  unsigned it = 0;
  while (true) {
    uint64_t v0 = pack2i(1u, 0u), v1 = pack2i(1u, 0u);
    if (c0 < n) v0 = ld_u64(reinterpret_cast<const uint64_t*>(base + o0));
    if (c1 < n) v1 = ld_u64(reinterpret_cast<const uint64_t*>(base + o1));
    if (__all(published(v0) && published(v1))) {
      if (c0 < n) lds[c0] = v0;
      if (c1 < n) lds[c1] = v1;
      return !__any(poisoned(v0) || poisoned(v1));
    }
    __builtin_amdgcn_s_sleep(1);
    if (++it >= limit) return false;
  }
}

// wave_poll for at most NL kWave slots: every poll reads all of them at once
// (one memory round trip).
template <int NL>
__device__ inline bool wave_poll_all(const uint64_t* a, int na, uint64_t* la, const uint64_t* b, int nb,
                                     uint64_t* lb, unsigned limit) {
  const int lane = threadIdx.x & (kWave - 1), n = na + nb;
  unsigned it = 0;
  while (true) {
    uint64_t v[NL];
    bool all = true, bad = false;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int c = lane + j * kWave;
      v[j] = pack2i(1u, 0u);
      if (c < na)
        v[j] = ld_u64(a + c);
      else if (c < n)
        v[j] = ld_u64(b + (c - na));
    }
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      all = all && published(v[j]);
      bad = bad || poisoned(v[j]);
    }
    if (__all(all)) {
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int c = lane + j * kWave;
        if (c < na)
          la[c] = v[j];
        else if (c < n)
          lb[c - na] = v[j];
      }
      return !__any(bad);
    }
    __builtin_amdgcn_s_sleep(1);
    if (++it >= limit) return false;
  }
}

// Whole-workgroup wait: wave 0 polls, then a barrier.  Finishers only.
__device__ inline bool gather2(const uint64_t* a, int na, uint64_t* la, const uint64_t* b, int nb, uint64_t* lb,
                               unsigned limit) {
  __shared__ int ok_s;
  if (threadIdx.x < kWave) {
    const bool ok = na + nb <= 4 * kWave ? wave_poll_all<4>(a, na, la, b, nb, lb, limit)
                                         : wave_poll(a, na, la, b, nb, lb, limit);
    if (threadIdx.x == 0) ok_s = ok;
  }
  __syncthreads();
  return ok_s != 0;
}
__device__ inline bool gather(const uint64_t* slots, int n, uint64_t* lds, unsigned limit) {
  return gather2(slots, n, lds, nullptr, 0, nullptr, limit);
}

// Set n slots back to kEmpty (wave 0).  Only the last reader of a slot clears
// it, after its own poll has returned the slot's data.
__device__ inline void clear_slots(uint64_t* slots, int n) {
  if (threadIdx.x < kWave)
    for (int c = threadIdx.x; c < n; c += kWave) st_u64(slots + c, 0ull);
}

// ------------------------------------------------------------- tile loading
//
// Wave tile c of a row is tokens [c * kWave * PER, (c + 1) * kWave * PER).
// Lane l holds vectors s = 0 .. PER / kVec - 1 at token
// tile_lo + (s * kWave + l) * kVec, so each load instruction of a wave reads
// 1 KiB of contiguous memory.

template <class E, int PER>
struct RawTile {
  static constexpr int NS = PER / E::kVec;
  u32x4 v[NS];
};

__device__ inline int wave_lane() { return threadIdx.x & (kWave - 1); }

// The loads are unconditional: a vector past the end of the row reads the
// row's last vector instead (V >= kVec), and unpack_tile masks it to -inf.
// Straight-line code keeps the raw tiles in registers.
template <class E, int PER>
__device__ inline void load_raw(const typename E::storage* row, int tile_lo, int V, RawTile<E, PER>& r) {
#pragma unroll
  for (int s = 0; s < RawTile<E, PER>::NS; ++s) {
    const int j0 = tile_lo + (s * kWave + wave_lane()) * E::kVec;
    r.v[s] = load_stream(row + min(j0, V - E::kVec));
  }
}

// PER_TOKEN: V need not be a multiple of kVec, so the vector that straddles
// V is masked token by token.
template <class E, int PER, bool PER_TOKEN = false>
__device__ inline void unpack_tile(const RawTile<E, PER>& r, int tile_lo, int V, float (&x)[PER]) {
  if (tile_lo + kWave * PER <= V) {  // the whole tile is in range: no per-token select
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
    const int j0 = tile_lo + (s * kWave + wave_lane()) * E::kVec;
    float t[E::kVec];
    E::unpack(r.v[s], t);
#pragma unroll
    for (int v = 0; v < E::kVec; ++v) x[s * E::kVec + v] = (PER_TOKEN ? j0 + v : j0) < V ? t[v] : -INFINITY;
  }
}

// A row that does not start on 16 bytes, copied from its aligned-down start
// (sh tokens earlier): each vector is cut from the two aligned vectors that
// cover it.  The copies run to the end of the tensor, so the vector that
// straddles the row's end holds the next row's first tokens (unpack_tile
// masks them to -inf).  Only where the second aligned vector would run past
// the tensor's end (the tensor's last row; `avail` = tokens from the row's
// start to the end of the tensor) are the tokens read one by one.
template <class E, int PER, class Avail>
__device__ inline void fix_shifted_tail(float (&x)[PER], int tile_lo, int V, const typename E::storage* row, int sh,
                                        Avail&& avail_fn) {
  if (tile_lo + kWave * PER <= V) return;  // not the row's last tile
  const int avail = avail_fn();
  if (tile_lo + kWave * PER + E::kVec - sh <= avail) return;
#pragma unroll
  for (int s = 0; s < PER / E::kVec; ++s) {
    const int j0 = tile_lo + (s * kWave + (int)(threadIdx.x & (kWave - 1))) * E::kVec;
    if (j0 + 2 * E::kVec - sh > avail) {
#pragma unroll
      for (int v = 0; v < E::kVec; ++v) x[s * E::kVec + v] = j0 + v < V ? E::at(row, j0 + v) : -INFINITY;
    }
  }
}

// Tokens from the start of target row i of sequence b, or of its draft row,
// to the end of that logit tensor, at most 2^30.
template <bool DRAFT>
__device__ inline int tokens_to_end(const VerifyArgs& a, int b, int i) {
  const long rows = DRAFT ? (long)a.B * a.gamma : (long)a.B * (a.gamma + 1);
  const long r = DRAFT ? (long)b * a.gamma + i : (long)b * (a.gamma + 1) + i;
  return (int)min((rows - r) * (long)a.V, 1L << 30);
}

template <int KVEC>
__device__ inline int tile_token(int tile_lo, int idx) {
  return tile_lo + ((idx / KVEC) * kWave + wave_lane()) * KVEC + idx % KVEC;
}

// Three-input maximum as one instruction.  The compiler rebalances chains of
// fmaxf into trees of two-input maxima, which costs about 1.4 instructions per
// two tokens instead of one.
__device__ inline float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Thread maximum with two independent chains of three-input maxima: half an
// instruction per token.
template <int PER>
__device__ inline float thread_max(const float (&x)[PER]) {
  static_assert(PER % 4 == 0, "PER must be a multiple of 4");
  float m0 = fmaxf(x[0], x[1]), m1 = fmaxf(x[2], x[3]);
#pragma unroll
  for (int i = 4; i < PER; i += 4) {
    m0 = max3f(m0, x[i], x[i + 1]);
    m1 = max3f(m1, x[i + 2], x[i + 3]);
  }
  return fmaxf(m0, m1);
}

// Exponents are kept in the scaled domain y = l * k (k = log2(e) / T): a
// maximum m becomes c = m * k, rounded once, and a token's weight relative to
// it is exp2(fma(l, k, -c)) -- one instruction for the argument.  Every later
// combination subtracts the same rounded c values, so that rounding cancels
// exactly.  This needs l * k finite for every logit (|l| log2(e) / T below
// FLT_MAX), which holds whenever l / T is representable at all.

// sum_i exp2(l_i k - c) over four independent accumulators.  With KEEP the
// weights replace x in place.  c == -inf (no finite logit) gives 0 and leaves
// x as it is: a caller skips such a thread, whose scale factor is then 0.
// (Filling x with zeros there costs a register copy per token; a branch-free
// form that selected the shift instead gave a wrong overlap for f32 tiles at
// T = 1e-3 on gfx950, so the branch stays.)
template <int PER, bool KEEP>
__device__ inline float thread_exp_sum(float (&x)[PER], float c, float k) {
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  if (c != -INFINITY) {
#pragma unroll
    for (int i = 0; i < PER; i += 4) {
      const float e0 = fast_exp2(fmaf(x[i], k, -c)), e1 = fast_exp2(fmaf(x[i + 1], k, -c));
      const float e2 = fast_exp2(fmaf(x[i + 2], k, -c)), e3 = fast_exp2(fmaf(x[i + 3], k, -c));
      if (KEEP) {
        x[i] = e0;
        x[i + 1] = e1;
        x[i + 2] = e2;
        x[i + 3] = e3;
      }
      if (i == 0) {  // 0 + e is not foldable to e (signed zeros): start from e
        s0 = e0;
        s1 = e1;
        s2 = e2;
        s3 = e3;
      } else {
        s0 += e0;
        s1 += e1;
        s2 += e2;
        s3 += e3;
      }
    }
  }
  return (s0 + s1) + (s2 + s3);
}

// The threads' (scaled max c, sum s relative to c) -> the wave's (scaled max,
// sum relative to it), identical in every lane.
__device__ inline float2 wave_lse(float c, float s) {
  const float C = wave_max(c);
  const float w = c == -INFINITY ? 0.f : s * fast_exp2(c - C);
  return make_float2(C, wave_sum(w));
}

template <class E, int PER>
__device__ inline ArgMax thread_argmax(const float (&x)[PER], int tile_lo) {
  return thread_argmax_first(x, [&](int i) { return tile_token<E::kVec>(tile_lo, i); });
}

// Row normalisers of both rows of an item from its W published word pairs
// (lds[2c] = (scaled max, sum) of p in wave tile c, lds[2c + 1] the same for
// q): M = max_c m_c and S = sum_c s_c exp2(m_c - M) in fp64, in one fixed
// order; M is in the scaled domain (a logit times k).  Called by all lanes of one wave; every lane gets the result.
struct Norm2 {
  float Mp, Mq;
  double Sp, Sq;
};

__device__ inline Norm2 wave_norm2(const uint64_t* w, int W) {
  const int lane = wave_lane();
  float Mp = -INFINITY, Mq = -INFINITY;
  for (int c = lane; c < W; c += kWave) {
    Mp = fmaxf(Mp, lo_f(w[2 * c]));
    Mq = fmaxf(Mq, lo_f(w[2 * c + 1]));
  }
  Mp = wave_max(Mp);
  Mq = wave_max(Mq);
  double Sp = 0.0, Sq = 0.0;
  for (int c = lane; c < W; c += kWave) {
    const float mp = lo_f(w[2 * c]), mq = lo_f(w[2 * c + 1]);
    if (mp != -INFINITY) Sp += (double)hi_f(w[2 * c]) * (double)fast_exp2(mp - Mp);
    if (mq != -INFINITY) Sq += (double)hi_f(w[2 * c + 1]) * (double)fast_exp2(mq - Mq);
  }
  return Norm2{Mp, Mq, wave_sum(Sp), wave_sum(Sq)};
}

// Mass of wave tile c of the p row, relative to the row's scaled maximum M.
__device__ inline double p_tile_mass(const uint64_t* w, int c, float M) {
  const float m = lo_f(w[2 * c]);
  return m == -INFINITY ? 0.0 : (double)hi_f(w[2 * c]) * (double)fast_exp2(m - M);
}

// Tile holding theta among W tile masses in tile order: wave 0 scans the
// masses (fp64, fixed order) and takes the first tile whose running mass
// exceeds theta.  *tile and *rest (theta minus the mass before that tile) are
// LDS variables, valid for the whole workgroup on return.  If rounding leaves
// theta past every tile, the last tile with mass is taken.  Called by the
// whole workgroup.
template <class MassFn>
__device__ inline void wave_pick_tile(int W, double theta, MassFn mass, int* tile, float* rest) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    double carry = 0.0;
    int pick = -1, last = 0;
    float left = 0.f;
    for (int base = 0; base < W; base += kWave) {
      const int c = base + lane;
      const double w = c < W ? mass(c) : 0.0;
      const double incl = carry + wave_inclusive_scan(w);
      const unsigned long long hit = __ballot(c < W && w > 0.0 && incl > theta);
      const unsigned long long pos = __ballot(c < W && w > 0.0);
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
// A compute workgroup only streams its tiles and publishes partials.  It
// never waits for a finisher.

template <class E>
__device__ inline const typename E::storage* trow(const VerifyArgs& a, int b, int i) {
  return static_cast<const typename E::storage*>(a.target) + ((size_t)b * (a.gamma + 1) + i) * (size_t)a.V;
}
template <class E>
__device__ inline const typename E::storage* drow(const VerifyArgs& a, int b, int i) {
  return static_cast<const typename E::storage*>(a.draft) + ((size_t)b * a.gamma + i) * (size_t)a.V;
}

// The raw wave tiles of one item: both rows of a pair, or the bonus row in `p`.
template <class E, int PER>
struct RawPair {
  RawTile<E, PER> p, q;
};

// Per-sequence draft counts in LDS.  Every workgroup of an extended launch
// with draft counts (B <= kGammaLds; larger batches take the multipass path)
// stages the prefix sums of the clamped gamma_b once, at its start:
// gamma_pre[b] is the number of live pairs of the sequences before b.  Every
// later lookup (an item's row, the dense walk over the live items) is then an
// LDS read instead of a memory round trip on the path to the next item's
// copies.
constexpr int kGammaLds = 2048;
__shared__ int gamma_pre[kGammaLds + 1];

// Wave 0 of the workgroup fills gamma_pre; the caller then synchronises the
// workgroup before any lookup.
__device__ inline void stage_gamma(const VerifyArgs& a) {
  if (!a.gamma_seq || threadIdx.x >= (unsigned)kWave) return;
  const int lane = wave_lane();
  if (lane == 0) gamma_pre[0] = 0;
  int acc = 0;
  for (int b0 = 0; b0 < a.B; b0 += kWave) {
    const int b = b0 + lane;
    const int g = b < a.B ? seq_gamma(a, b) : 0;
    const int incl = (int)wave_inclusive_scan((float)g);  // exact: at most 2048
    if (b < a.B) gamma_pre[b + 1] = acc + incl;
    acc += __builtin_amdgcn_readlane(incl, kWave - 1);
  }
}

template <bool EXT>
__device__ inline int seq_gamma_of(const VerifyArgs& a, int b) {
  if constexpr (!EXT) return a.gamma;
  return a.gamma_seq ? gamma_pre[b + 1] - gamma_pre[b] : a.gamma;
}

// With per-sequence draft counts the teams and finishers walk the live items
// only, densely: the pairs (b, i) with i < gamma_b, by b then i, then the B
// bonus items (pairs first, so a finisher never waits on an item it has yet
// to finish itself).  Every item keeps its own slots.  live_item maps a dense
// index (the same in every lane) to its item by two ballots over the staged
// prefix sums; it is called by whole waves.  Without draft counts both are
// the identity.
template <bool EXT>
__device__ inline int live_count(const FusedParams& P) {
  if constexpr (!EXT) return P.n_items;
  return P.a.gamma_seq ? gamma_pre[P.a.B] + P.a.B : P.n_items;
}
template <bool EXT>
__device__ inline int live_item(const FusedParams& P, int d) {
  if constexpr (!EXT) return d;
  const VerifyArgs& a = P.a;
  if (!a.gamma_seq) return d;
  const int n_lpairs = gamma_pre[a.B];
  if (d >= n_lpairs) return P.n_pairs + (d - n_lpairs);  // a bonus item
  // the 64-sequence chunks wholly before d (each lane reads the prefix at the
  // end of one chunk; at most 32 chunks), then the sequences of d's chunk
  // wholly before d: both a prefix of the lanes
  const int lane = wave_lane();
  const int ce = lane * kWave < a.B ? gamma_pre[min((lane + 1) * kWave, a.B)] : INT_MAX;
  const int b0 = __popcll(__ballot(ce <= d)) * kWave;
  const int pe = b0 + lane < a.B ? gamma_pre[b0 + lane + 1] : INT_MAX;
  const int b = b0 + __popcll(__ballot(pe <= d));
  return b * a.gamma + (d - gamma_pre[b]);
}


// The k-th live item (dense index) of team t, or n_live after its last.  The
// pairs go round-robin, so the first n_pairs mod nteams teams hold one more;
// the bonus items, half a pair's work each, then fill the lighter teams two
// deep before any team gets a third, which keeps every team within half a
// pair of the mean.
__device__ inline int team_dense(int t, int k, int nt, int n_live, int n_lpairs) {
  const int np_t = t < n_lpairs ? (n_lpairs - 1 - t) / nt + 1 : 0;
  if (k < np_t) return t + k * nt;
  const int j = k - np_t;                   // this team's j-th bonus item
  const int r = n_lpairs % nt, light = nt - r;
  int bonus;
  if (t >= r && j < 2) bonus = j * light + (t - r);
  else bonus = 2 * light + (j - (t >= r ? 2 : 0)) * nt + t;
  const int d = n_lpairs + bonus;
  return d < n_live ? d : n_live;
}

template <class E, int PER, bool EXT>
__device__ __attribute__((always_inline)) void issue_item(const FusedParams& P, int item, int lo, RawPair<E, PER>& r) {
  const VerifyArgs& a = P.a;
  const bool pair = item < P.n_pairs;
  const int b = pair ? item / a.gamma : item - P.n_pairs;
  const int i = pair ? item % a.gamma : seq_gamma_of<EXT>(a, b);  // a bonus item reads row gamma_b
  load_raw<E, PER>(trow<E>(a, b, i), lo, a.V, r.p);
  if (pair) load_raw<E, PER>(drow<E>(a, b, i), lo, a.V, r.q);
}


// Row normalisers handed from wave 0 to the other waves, double-buffered by
// item parity: a buffer is rewritten two items later, after every wave has
// passed the barrier of the item in between.
struct __align__(16) NormMsg {
  float Mp, Mq, invSp, invSq;
  int ok, pad0, pad1, pad2;
};

// The keep thresholds of an item's rows: the target row's and, for a pair, the
// draft row's (-inf: nothing filtered).  Loaded ahead of the item's compute.
struct ItemThr {
  float p, q;
};
template <bool EXT, bool THR, bool TWO_BONUS = false>
__device__ inline ItemThr item_thr(const FusedParams& P, int item) {
  ItemThr t{-INFINITY, -INFINITY};
  if constexpr (THR) {
    const VerifyArgs& a = P.a;
    if (a.thr && item < P.n_items) {
      if (item < P.n_pairs) {
        const int b = item / a.gamma, i = item % a.gamma;
        t.p = thr_target(a, b, i);
        t.q = thr_draft(a, b, i);
      } else {
        const int b = item - P.n_pairs;  // the bonus row is target row gamma_b
        t.p = thr_target(a, b, seq_gamma_of<EXT>(a, b));
        // a unit of two bonus items: the second sequence's bonus row in q
        if (TWO_BONUS && b + 1 < a.B) t.q = thr_target(a, b + 1, seq_gamma_of<EXT>(a, b + 1));
      }
    }
  }
  return t;
}

// Top-k / top-p filtering (extended kernels): a logit below its row's keep
// threshold becomes -inf, i.e. probability 0.
template <int PER>
__device__ inline void mask_below(float (&x)[PER], float t) {
#pragma unroll
  for (int j = 0; j < PER; ++j) x[j] = x[j] >= t ? x[j] : -INFINITY;
}

// Pair item, T > 0, in three steps.  Phase 1 turns the wave tile into kept
// weights and publishes the wave's (scaled max, sum) of both rows.
template <class E, int PER, bool THR, bool SHIFT = false>
__device__ __attribute__((always_inline)) void pair_phase1(const FusedParams& P, int item, int c, int lo,
                                                           const RawPair<E, PER>& raw, const ItemThr& th,
                                                           float (&ep)[PER], float (&eq)[PER], float& mp, float& mq,
                                                           float& sp, float& sq) {
  const VerifyArgs& a = P.a;
  const float k = a.k;
  unpack_tile<E, PER, SHIFT>(raw.p, lo, a.V, ep);
  unpack_tile<E, PER, SHIFT>(raw.q, lo, a.V, eq);
  if constexpr (SHIFT) {  // rows that do not start on 16 bytes
    const int b = item / a.gamma, i = item % a.gamma;
    const auto* pr = trow<E>(a, b, i);
    const auto* qr = drow<E>(a, b, i);
    fix_shifted_tail<E, PER>(ep, lo, a.V, pr, (int)(((uintptr_t)pr & 15u) / sizeof(typename E::storage)),
                             [&] { return tokens_to_end<false>(a, b, i); });
    fix_shifted_tail<E, PER>(eq, lo, a.V, qr, (int)(((uintptr_t)qr & 15u) / sizeof(typename E::storage)),
                             [&] { return tokens_to_end<true>(a, b, i); });
  }
  if constexpr (THR) {
    mask_below<PER>(ep, th.p);
    mask_below<PER>(eq, th.q);
  }
  mp = thread_max<PER>(ep) * k;  // scaled maxima
  mq = thread_max<PER>(eq) * k;
  sp = thread_exp_sum<PER, true>(ep, mp, k);
  sq = thread_exp_sum<PER, true>(eq, mq, k);
  const float2 lp = wave_lse(mp, sp), lq = wave_lse(mq, sq);
  uint64_t* part1 = P.part1 + (size_t)item * P.W * 2;
  if (wave_lane() == 0) {
    st_u64(part1 + 2 * c, pack2(lp.x, lp.y));
    st_u64(part1 + 2 * c + 1, pack2(lq.x, lq.y));
  }
}

// Barrier, then every wave reads *m from LDS.  Written in assembly so that
// the compiler adds no wait for this wave's outstanding buffer loads into
// LDS: the compiler cannot tell that they target the stage, not *m, and a
// wait for them here would hold every wave until the next item's tiles have
// arrived.  The barrier follows the completion of this wave's own LDS writes
// (lgkmcnt(0)), so the writer's message is visible after it; the loads into
// the stage are ordered by the explicit vmcnt wait before the stage is read.
__device__ __attribute__((always_inline)) inline NormMsg lds_exchange_msg(const NormMsg* m) {
  const uint32_t addr =
      (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) NormMsg*)m);
  float4 v;
  int ok;
  asm volatile(
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_barrier\n\t"
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b32 %1, %2 offset:16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v), "=&v"(ok)
      : "v"(addr)
      : "memory");
  return NormMsg{v.x, v.y, v.z, v.w, ok, 0, 0, 0};
}

// The team wait: wave 0 polls until every wave of the team has published its
// phase-1 partials, combines them in one fixed order and hands both row
// normalisers to the other waves through msg[parity] (one LDS-only barrier).
// Called by the whole workgroup.  WIDE kernels (rows of more than 64 wave
// tiles, up to 128) read all 4 kWave slots in each poll; the others poll at
// most 2 kWave (a separate instantiation: the wider poll's code slowed the
// narrow kernel by 8% though it never ran there).
template <bool WIDE>
__device__ __attribute__((always_inline)) inline NormMsg pair_wait(const FusedParams& P, int item, int parity,
                                                                   uint64_t* w1, NormMsg* msg) {
  if (threadIdx.x < kWave) {
    const uint64_t* part1 = P.part1 + (size_t)item * P.W * 2;
    bool ok;
    if constexpr (WIDE)
      ok = 2 * P.W <= 4 * kWave ? wave_poll_all<4>(part1, 2 * P.W, w1, nullptr, 0, nullptr, P.polls)
                                : wave_poll(part1, 2 * P.W, w1, nullptr, 0, nullptr, P.polls);
    else
      ok = 2 * P.W <= 2 * kWave ? wave_poll_once(part1, 2 * P.W, w1, P.polls)
                                : wave_poll(part1, 2 * P.W, w1, nullptr, 0, nullptr, P.polls);
    NormMsg m{0.f, 0.f, 0.f, 0.f, 0, 0, 0, 0};
    if (ok) {
      const Norm2 n = wave_norm2(w1, P.W);
      m = NormMsg{n.Mp, n.Mq, (float)(1.0 / n.Sp), (float)(1.0 / n.Sq), 1, 0, 0, 0};
    }
    if (threadIdx.x == 0) msg[parity] = m;
  }
  return lds_exchange_msg(msg + parity);
}

// Phase 2: the wave's share of alpha = sum min(p, q) and of the residual mass
// sum max(0, p - q) from the kept weights, published as one word.
//
// With p = ep fp and q = eq fq (fp, fq the thread's scale factors) and
// r = fp / fq, sum min(p, q) = fq sum min(ep r, eq), and min(a, b) =
// (a + b - |a - b|) / 2 turns that into fq (r sp + sq - sum |ep r - eq|) / 2:
// one fused multiply-add and one add with an absolute-value operand per token.
// The subtraction loses a few ulps of the thread's p and q mass (absolute),
// far below the overlap's tolerance.  r is an exact quotient (fq can be
// subnormal at low temperature, where the hardware reciprocal flushes to
// zero).  Above 2^64 the thread's q mass is under 2^-53 of its p mass and its
// share of the overlap is taken as 0, which also keeps every term finite.
template <int PER, bool EXT>
__device__ __attribute__((always_inline)) void pair_phase2(const FusedParams& P, int item, int c, const NormMsg& m,
                                                           const float (&ep)[PER], const float (&eq)[PER],
                                                           float mp, float mq, float sp, float sq) {
  uint64_t* mine2 = P.part2 + (size_t)item * P.W + c;
  if (!m.ok) {
    if (wave_lane() == 0) st_u64(mine2, pack2i(kPoison, 0u));
    return;
  }
  const float fp = mp == -INFINITY ? 0.f : fast_exp2(mp - m.Mp) * m.invSp;
  const float fq = mq == -INFINITY ? 0.f : fast_exp2(mq - m.Mq) * m.invSq;
  // sum_x min(ep r, eq) over the thread's tokens, by the |a - b| form
  auto overlap = [&](float r) {
    float d0 = fabsf(fmaf(ep[0], r, -eq[0])), d1 = fabsf(fmaf(ep[1], r, -eq[1]));
    float d2 = fabsf(fmaf(ep[2], r, -eq[2])), d3 = fabsf(fmaf(ep[3], r, -eq[3]));
#pragma unroll
    for (int j = 4; j < PER; j += 4) {
      d0 += fabsf(fmaf(ep[j], r, -eq[j]));
      d1 += fabsf(fmaf(ep[j + 1], r, -eq[j + 1]));
      d2 += fabsf(fmaf(ep[j + 2], r, -eq[j + 2]));
      d3 += fabsf(fmaf(ep[j + 3], r, -eq[j + 3]));
    }
    return fmaxf(0.5f * (fmaf(r, sp, sq) - ((d0 + d1) + (d2 + d3))), 0.f);
  };
  float alpha_t = 0.f, lmin_t = 0.f;
  const float r = fp / fq;
  if (fp > 0.f && fq > 0.f && r <= 0x1p64f) alpha_t = overlap(r) * fq;
  // The residual sum max(0, p - l q) = sum p - sum min(p, l q); with l = 1
  // the second sum is alpha.  For l < 1 (only in the extended kernels, so the
  // exact path carries no code for it) it is the same overlap with q scaled
  // by l (ratio r / l).
  lmin_t = alpha_t;
  if constexpr (EXT) {
    const float l = P.a.lenience;
    if (l != 1.f) {
      const float rl = r / l;
      lmin_t = fp > 0.f && fq > 0.f && rl <= 0x1p64f ? overlap(rl) * (l * fq) : 0.f;
    }
  }
  const float res_t = fmaxf(sp * fp - lmin_t, 0.f);
  const float alpha_w = wave_sum(alpha_t), res_w = wave_sum(res_t);
  if (wave_lane() == 0) st_u64(mine2, pack2(alpha_w, res_w));
}

// The three steps back to back: the tile stays in registers across the wait.
template <class E, int PER, bool EXT, bool WIDE, bool THR>
__device__ __attribute__((always_inline)) void pair_compute_sample(const FusedParams& P, int item, int c, int lo,
                                                                   int parity, const RawPair<E, PER>& raw,
                                                                   uint64_t* w1, NormMsg* msg) {
  float ep[PER], eq[PER], mp, mq, sp, sq;
  pair_phase1<E, PER, THR>(P, item, c, lo, raw, item_thr<EXT, THR>(P, item), ep, eq, mp, mq, sp, sq);
  const NormMsg m = pair_wait<WIDE>(P, item, parity, w1, msg);
  pair_phase2<PER, EXT>(P, item, c, m, ep, eq, mp, mq, sp, sq);
}

// Pair item at T = 0, or a bonus item: one pass, no waiting.
template <class E, int PER, bool ARGMAX, bool THR, bool SHIFT = false>
__device__ __attribute__((always_inline)) void single_pass_compute(const FusedParams& P, int item, int c, int lo,
                                                                   const RawPair<E, PER>& raw, const ItemThr& th) {
  const VerifyArgs& a = P.a;
  uint64_t w0, w1;
  if (item < P.n_pairs) {  // argmax pair
    float xp[PER], xq[PER];
    unpack_tile<E, PER>(raw.p, lo, a.V, xp);
    unpack_tile<E, PER>(raw.q, lo, a.V, xq);
    const ArgMax ap = wave_argmax(thread_argmax<E, PER>(xp, lo));
    const ArgMax aq = wave_argmax(thread_argmax<E, PER>(xq, lo));
    w0 = pack2i(nz_bits(ap.v), (uint32_t)ap.i);
    w1 = pack2i(nz_bits(aq.v), (uint32_t)aq.i);
  } else {
    float x[PER];
    unpack_tile<E, PER, SHIFT>(raw.p, lo, a.V, x);
    if constexpr (SHIFT) {  // the bonus row, not starting on 16 bytes
      const int b = item - P.n_pairs, g = seq_gamma_of<true>(a, b);
      const auto* r = trow<E>(a, b, g);
      fix_shifted_tail<E, PER>(x, lo, a.V, r, (int)(((uintptr_t)r & 15u) / sizeof(typename E::storage)),
                               [&] { return tokens_to_end<false>(a, b, g); });
    }
    if constexpr (ARGMAX) {
      const ArgMax ab = wave_argmax(thread_argmax<E, PER>(x, lo));
      w0 = pack2i(nz_bits(ab.v), (uint32_t)ab.i);
    } else {
      if constexpr (THR) mask_below<PER>(x, th.p);
      const float m = thread_max<PER>(x) * a.k;
      const float sm = thread_exp_sum<PER, false>(x, m, a.k);
      const float2 l = wave_lse(m, sm);
      w0 = pack2(l.x, l.y);
    }
    w1 = pack2i(0x80000000u, 0u);  // unused second word: (-0, 0), published
  }
  if (wave_lane() == 0) {
    uint64_t* mine = P.part1 + ((size_t)item * P.W + c) * 2;
    st_u64(mine, w0);
    st_u64(mine + 1, w1);
  }
}

// Wait until this wave's vector memory operations are complete (vmcnt(0);
// the other counters are left alone).
__device__ inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// bf16 compute loop with the next item staged in LDS.  Waves 1..3 copy the
// next item's tiles (all four waves' tiles) from HBM straight into LDS while
// the current item is computed from registers; wave 0 issues no global loads,
// so its polls of the exchange slots never wait behind them (vector memory
// operations of a wave complete in order).  Per item:
//   every wave copies its raw vectors from the stage; barrier (stage free);
//   waves 1..3 start the next item's copy; compute; waves 1..3 wait for their
//   copies; barrier (stage full).
// Each of the 2 * 4 * NS wave loads of an item moves 1 KiB of one row into
// 1 KiB of LDS, lane l writing bytes [16 l, 16 l + 16).
template <int PER, bool SHIFT>
constexpr int stage_vectors() { return 2 * (kWavesPerGroup * (PER / BF16::kVec) + (SHIFT ? 1 : 0)) * kWave; }

template <int PER, bool ARGMAX, bool EXT, bool WIDE, bool THR, bool SHIFT, bool UNITS>
__device__ __attribute__((always_inline)) void compute_loop_staged(const FusedParams& P, int team, int rank,
                                                                   u32x4* stage, uint64_t* w1, NormMsg* msg) {
  using E = BF16;
  static_assert(!ARGMAX, "the argmax kernel loads without the stage");
  constexpr int NS = PER / E::kVec;
  constexpr int kLoads = 2 * kWavesPerGroup * NS;
  const VerifyArgs& a = P.a;
  // the wave index is uniform across the wave: keep it (and everything derived
  // from it) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave), lane = wave_lane();
  const int c = rank * kWavesPerGroup + wave;
  const int lo = c * kWave * PER;
  const unsigned row_bytes = (unsigned)a.V * (unsigned)sizeof(E::storage);

  // Each copy is one buffer load into LDS: the resource starts at the copy's
  // first vector and ends at the end of the row, so vectors past V read as
  // zero (unpack_tile masks them to -inf) and all address arithmetic is
  // scalar; lane l moves bytes [16 l, 16 l + 16).
  //
  // Rows that do not start on 16 bytes (V not a multiple of kVec; the tensors
  // themselves start on 16 bytes) are copied from their 16-byte aligned-down
  // start: a row starting sh tokens past that boundary has token t at
  // position t + sh of the copy.  Such rows take one KiB more per row, so the
  // slot also holds the vector after the tile, and every lane cuts its
  // vectors out of the two aligned vectors that cover them.
  constexpr int kCopyBytes = kWave * 16;                  // one copy: 16 bytes per lane
  constexpr int kRowLoads = kWavesPerGroup * NS;          // copies per row tile of the workgroup
  constexpr int kSlotVec = (kRowLoads + (SHIFT ? 1 : 0)) * kWave;  // vectors per row slot of the stage
  static_assert(NS * E::kVec == PER && (kRowLoads & (kRowLoads - 1)) == 0, "stage copy shape");
  constexpr bool shifted = SHIFT;  // V % kVec != 0
  constexpr bool units = UNITS;  // bonus items two at a time
  const unsigned tile_bytes = (unsigned)(rank * kWavesPerGroup * kWave * PER * (int)sizeof(E::storage));
  auto shift_of = [](const E::storage* row) {  // tokens of the row's start past 16 bytes
    return (int)(((uintptr_t)row & 15u) / sizeof(E::storage));
  };
  auto issue = [&](int item) {  // waves 1..3
    const bool pair = item < P.n_pairs;
    const int b = pair ? item / a.gamma : item - P.n_pairs;
    // a bonus item reads row gamma_b (padding items are never issued); a
    // bonus unit also reads the next sequence's bonus row into the q slot
    const int i = pair ? item % a.gamma : seq_gamma_of<EXT>(a, b);
    const bool two = pair || (units && b + 1 < a.B);
    const int i2 = pair ? i : (two ? seq_gamma_of<EXT>(a, b + 1) : 0);
    if constexpr (!shifted) {
      const E::storage* prow = trow<E>(a, b, i);
      const E::storage* qrow = pair ? drow<E>(a, b, i) : (two ? trow<E>(a, b + 1, i2) : prow);
      const int n = two ? 2 * kRowLoads : kRowLoads;
      // Copy l moves the (l mod kRowLoads)-th KiB of this workgroup's tile of
      // row l / kRowLoads (the four wave tiles are adjacent, vector s of wave w
      // being KiB w * NS + s) into KiB l of the stage.
      for (int l = wave - 1; l < n; l += kWavesPerGroup - 1) {
        const unsigned off = tile_bytes + (unsigned)(l & (kRowLoads - 1)) * kCopyBytes;
        const uint64_t addr = reinterpret_cast<uint64_t>(l < kRowLoads ? prow : qrow) + off;
        const uint64_t uaddr = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(addr >> 32)) << 32) |
                               (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)addr);
        // bytes from the copy's first vector to the row's end (rows are
        // shorter than 2^31 bytes); a signed max stays a scalar instruction
        const int nrec = max((int)row_bytes - (int)off, 0);
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(uaddr), (short)0, nrec, 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)&stage[l * kWave], 16,
                                                 (unsigned)lane * 16u, 0, 0, 0);
      }
    } else {
      // each row from its aligned-down start, kRowLoads + 1 copies into its
      // own slot; copies bounded by the end of the tensor
      const E::storage* rows[2] = {trow<E>(a, b, i),
                                   pair ? drow<E>(a, b, i) : (two ? trow<E>(a, b + 1, i2) : nullptr)};
      int first = wave - 1;  // this wave's first copy of the row: copies l with l mod 3 == wave - 1
      for (int r = 0; r < (two ? 2 : 1); ++r) {
        const int sh = shift_of(rows[r]);
        const E::storage* base = rows[r] - sh;  // 16-byte aligned
        const int left = r == 0 ? tokens_to_end<false>(a, b, i)
                                : (pair ? tokens_to_end<true>(a, b, i) : tokens_to_end<false>(a, b + 1, i2));
        const int ext = (sh + left) * (int)sizeof(E::storage);
        for (int l = first; l < kRowLoads + 1; l += kWavesPerGroup - 1) {
          const unsigned off = tile_bytes + (unsigned)l * kCopyBytes;
          const uint64_t addr = reinterpret_cast<uint64_t>(base) + off;
          const uint64_t uaddr = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(addr >> 32)) << 32) |
                                 (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)addr);
          const int nrec = max(ext - (int)off, 0);
          const __amdgpu_buffer_rsrc_t rs =
              __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(uaddr), (short)0, nrec, 0x00020000);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rs, (__attribute__((address_space(3))) void*)&stage[r * kSlotVec + l * kWave], 16, (unsigned)lane * 16u,
              0, 0, 0);
        }
        first = (first + (kWavesPerGroup - 1) - (kRowLoads + 1) % (kWavesPerGroup - 1)) % (kWavesPerGroup - 1);
      }
    }
  };

  // The teams walk units round-robin: first the live pairs, then the bonus
  // items two at a time (two sequences' bonus rows, a pair's worth of copies
  // and arithmetic, where one bonus row alone took three quarters of a pair's
  // round).  A unit is named by its first item; the last unit of an odd batch
  // holds one bonus row.
  const int n_live = live_count<EXT>(P);
  const int n_lpairs = n_live - a.B;
  auto lookup = [&](int k) {
    if (!units) {
      const int dk = team_dense(team, k, P.nteams, n_live, n_lpairs);
      return dk < n_live ? live_item<EXT>(P, dk) : P.n_items;
    }
    const int u = k * P.nteams + team;
    if (u < n_lpairs) return live_item<EXT>(P, u);
    const int j = 2 * (u - n_lpairs);
    return j < a.B ? P.n_pairs + j : P.n_items;
  };
  int kth = 0;
  int item = lookup(0);
  if (wave != 0 && item < P.n_items) issue(item);
  // With draft counts the unit after the next one is looked up a round
  // ahead, so the LDS lookups of the walk stay off the path to the copies.
  int ahead = EXT ? lookup(1) : 0;
  if (wave != 0) wait_vmem();
  lds_barrier();
  // keep thresholds, loaded when the unit's tiles are issued (one unit ahead)
  ItemThr th = item_thr<EXT, THR, UNITS>(P, item);
  int parity = 0;
  int pend = -1;  // pipelined: the pair item whose kept weights wait in (ep, eq)
  float ep[PER], eq[PER], mp = 0.f, mq = 0.f, sp = 0.f, sq = 0.f;
  // dispatch class of this workgroup: which third of the grid (the grid fills
  // every compute unit once before it places a second workgroup on any)
  const int slot_class = (int)((blockIdx.x * 3u) / gridDim.x);
  int round = 0;
  while (item < P.n_items) {
    {
      switch ((round + slot_class) % 3) {  // s_setprio takes an immediate
        case 0: __builtin_amdgcn_s_setprio(0); break;
        case 1: __builtin_amdgcn_s_setprio(1); break;
        default: __builtin_amdgcn_s_setprio(2); break;
      }
    }
    ++round;
    RawPair<E, PER> A;
    int sh_p = 0, sh_q = 0;
    if constexpr (shifted) {
      const bool pair = item < P.n_pairs;
      const int b = pair ? item / a.gamma : item - P.n_pairs;
      const int i = pair ? item % a.gamma : seq_gamma_of<EXT>(a, b);
      sh_p = shift_of(trow<E>(a, b, i));
      sh_q = pair ? shift_of(drow<E>(a, b, i))
                  : (units && b + 1 < a.B ? shift_of(trow<E>(a, b + 1, seq_gamma_of<EXT>(a, b + 1))) : 0);
#pragma unroll
      for (int v = 0; v < NS; ++v) {
        const int j = (wave * NS + v) * kWave + lane;
        A.p.v[v] = cut_vector(stage[j], stage[j + 1], sh_p * (int)sizeof(E::storage));
        A.q.v[v] = cut_vector(stage[kSlotVec + j], stage[kSlotVec + j + 1], sh_q * (int)sizeof(E::storage));
      }
    } else {
#pragma unroll
      for (int v = 0; v < NS; ++v) {
        A.p.v[v] = stage[(wave * NS + v) * kWave + lane];
        A.q.v[v] = stage[kSlotVec + (wave * NS + v) * kWave + lane];
      }
    }
    lds_barrier();
    ++kth;
    const int next = EXT ? ahead : lookup(kth);
    if (wave != 0 && next < P.n_items) issue(next);
    if constexpr (EXT) ahead = lookup(kth + 1);
    const ItemThr th_next = item_thr<EXT, THR, UNITS>(P, next);
    {
      // Two pair items in flight: phase 1 of this item runs while the team
      // exchange of the previous one completes, and only then is the previous
      // one finished.  (Copying the new weights into the pending set costs a
      // register move per token but needs fewer registers than two sets that
      // swap roles.)
      if (item < P.n_pairs) {
        float xp[PER], xq[PER], cp, cq, s_p, s_q;
        pair_phase1<E, PER, THR, SHIFT>(P, item, c, lo, A, th, xp, xq, cp, cq, s_p, s_q);
        if (pend >= 0) {
          const NormMsg m = pair_wait<WIDE>(P, pend, parity, w1, msg);
          pair_phase2<PER, EXT>(P, pend, c, m, ep, eq, mp, mq, sp, sq);
          parity ^= 1;
        }
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          ep[j] = xp[j];
          eq[j] = xq[j];
        }
        mp = cp;
        mq = cq;
        sp = s_p;
        sq = s_q;
        pend = item;
      } else {
        single_pass_compute<E, PER, ARGMAX, THR, SHIFT>(P, item, c, lo, A, th);
        if (units && item - P.n_pairs + 1 < a.B) {  // the unit's second bonus row, staged in q
          const RawPair<E, PER> A2{A.q, A.q};
          single_pass_compute<E, PER, ARGMAX, THR, SHIFT>(P, item + 1, c, lo, A2, ItemThr{th.q, -INFINITY});
        }
        if (pend >= 0) {
          const NormMsg m = pair_wait<WIDE>(P, pend, parity, w1, msg);
          pair_phase2<PER, EXT>(P, pend, c, m, ep, eq, mp, mq, sp, sq);
          parity ^= 1;
          pend = -1;
        }
      }
    }
    if (wave != 0) wait_vmem();
    lds_barrier();
    item = next;
    th = th_next;
  }
  if (pend >= 0) {
    const NormMsg m = pair_wait<WIDE>(P, pend, parity, w1, msg);
    pair_phase2<PER, EXT>(P, pend, c, m, ep, eq, mp, mq, sp, sq);
  }
}

// ---------------------------------------------------- finisher workgroups

// The finisher's inverse-CDF search covers a group of consecutive wave tiles,
// enough that each of its threads scans at least one whole vector.
template <class E, int PER>
struct SearchShape {
  // the smallest group whose tokens split into whole vectors per thread
  static constexpr int group_for() {
    int g = 1;
    while ((g * kWave * PER) % (kThreads * E::kVec) != 0) ++g;
    return g;
  }
  static constexpr int kGroup = group_for();
  static constexpr int kTokens = kGroup * kWave * PER;  // tokens per search group
  static constexpr int kPer = kTokens / kThreads;       // tokens per thread
};

// Combine W argmax partials (value, index) in tile order.
__device__ inline ArgMax combine_argmax(const uint64_t* w, int W, int half) {
  ArgMax g{-INFINITY, 0x7fffffff};
  for (int c = 0; c < W; ++c) {
    const uint64_t v = w[2 * c + half];
    g = argmax_better(g, ArgMax{lo_f(v), (int)(uint32_t)(v >> 32)});
  }
  return g;
}

// Pair item: alpha, the ratio test and, after a rejection, the residual
// sample.  Publishes (accept, token) for the sequence's bonus finisher.
template <class E, int PER, bool ARGMAX, bool EXT, bool SHIFT>
__device__ void finish_pair(const FusedParams& P, int item, uint64_t* w1, uint64_t* w2) {
  using S = SearchShape<E, PER>;
  __shared__ float lds_f[kMaxWaves];
  __shared__ int lds_i[kMaxWaves];
  __shared__ double lds_d[kMaxWaves];
  __shared__ int tile_s, acc_s;
  __shared__ float rest_s;
  __shared__ float Mp_s, Mq_s;
  __shared__ double Sp_s, Sq_s, alpha_s, sw_s;
  const VerifyArgs& a = P.a;
  const int G = a.gamma, W = P.W;
  const int b = item / G, i = item % G;
  const float k = a.k;
  const auto* prow = trow<E>(a, b, i);
  const auto* qrow = drow<E>(a, b, i);
  const size_t o = (size_t)b * G + i;
  uint64_t* part1 = P.part1 + (size_t)item * W * 2;
  uint64_t* part2 = P.part2 + (size_t)item * W;
  // only live pairs (i < gamma_b) reach a finisher: the bonus finisher
  // writes the padding positions' outputs
  const int gb = seq_gamma_of<EXT>(a, b);

  if constexpr (ARGMAX) {
    if (!gather(part1, 2 * W, w1, P.polls)) {
      if (threadIdx.x == 0) st_u64(P.pair_res + item, pack2i(kPoison, 0u));
      return;
    }
    clear_slots(part1, 2 * W);
    if (threadIdx.x == 0) {
      // keep x iff it is the target's argmax; alpha is the indicator that the
      // two argmaxes agree ([FI] "Speculative sampling", temperature to zero)
      const ArgMax gp = combine_argmax(w1, W, 0), gq = combine_argmax(w1, W, 1);
      const int x = a.tokens[o];
      if (a.alpha) a.alpha[o] = gp.i == gq.i ? 1.f : 0.f;
      if (a.p_draft) a.p_draft[o] = x == gp.i ? 1.f : 0.f;
      if (a.q_draft) a.q_draft[o] = x == gq.i ? 1.f : 0.f;
      st_u64(P.pair_res + item, pack2i((x == gp.i ? 1u : 0u) | kResMark, (uint32_t)gp.i));
    }
    return;
  } else {
    // the ratio-test inputs and both uniforms do not depend on the partials:
    // fetch them first, so that their round trips overlap the wait
    int x = 0;
    float lp = 0.f, lq = 0.f, u_i = 0.f;
    const float u_fin = a.uniforms[(size_t)b * (G + 1) + gb];  // the final sample's uniform
    if (threadIdx.x == 0) {
      u_i = a.uniforms[(size_t)b * (G + 1) + i];
      x = a.tokens[o];
      if (x >= 0 && x < a.V) {
        lp = E::at(prow, x);
        lq = E::at(qrow, x);
        if (EXT && a.thr) {  // a filtered-out token has probability 0
          if (lp < thr_target(a, b, i)) lp = -INFINITY;
          if (lq < thr_draft(a, b, i)) lq = -INFINITY;
        }
      }
    }
    // part2 is published after part1 by every wave; polling both in one pass
    // returns once both are complete
    if (!gather2(part1, 2 * W, w1, part2, W, w2, P.polls)) {
      if (threadIdx.x == 0) st_u64(P.pair_res + item, pack2i(kPoison, 0u));
      return;
    }
    // Every wave has published part2, so every wave is done reading part1.
    // The slots are cleared after the result is out: stores issued here would
    // hold up the barriers below.
    // Normalisers, alpha and the residual mass (wave 0, fixed order):
    if (threadIdx.x < kWave) {
      const Norm2 n = wave_norm2(w1, W);
      double al = 0.0, sw = 0.0;
      for (int c = threadIdx.x; c < W; c += kWave) {
        al += (double)lo_f(w2[c]);
        sw += (double)hi_f(w2[c]);
      }
      al = wave_sum(al);
      sw = wave_sum(sw);
      if (threadIdx.x == 0) {
        Mp_s = n.Mp;
        Mq_s = n.Mq;
        Sp_s = n.Sp;
        Sq_s = n.Sq;
        alpha_s = al;
        sw_s = sw;
      }
    }
    __syncthreads();
    const float Mp = Mp_s, Mq = Mq_s;
    const double Sp = Sp_s, Sq = Sq_s;
    double px = 0.0, qx = 0.0;  // thread 0's; stored with the result, after the search
    if (threadIdx.x == 0) {
      if (x >= 0 && x < a.V) {
        px = exp2((double)lp * (double)k - (double)Mp) / Sp;
        qx = exp2((double)lq * (double)k - (double)Mq) / Sq;
      }
      // accept iff u <= min(1, p(x) / q(x)) ([FI] Algorithm 1 step 3; [SD]
      // "The algorithm").  q(x) = 0 keeps the draft when p(x) > 0 (the ratio
      // is +inf) and rejects it when p(x) = 0 (0/0).
      // With lenience l the comparison is against p(x) / (l q(x)) ([FI]
      // "The acceptance rate is the overlap of p and q", lenience factor).
      const double u = (double)u_i;
      if (qx > 0.0) {
        const double ratio = px / ((double)a.lenience * qx);
        acc_s = (ratio >= 1.0) || (u <= ratio);
      } else {
        acc_s = px > 0.0;
      }
    }
    __syncthreads();
    const int acc_i = acc_s;
    int mode = 0;
    const double uf = (double)u_fin;
    // search groups of S::kGroup consecutive wave tiles, in token order
    const int ng = (W + S::kGroup - 1) / S::kGroup;
    auto pick_p_tile = [&]() {
      wave_pick_tile(ng, uf * Sp, [&](int g) {
        double m = 0.0;
        for (int c = g * S::kGroup; c < min(W, (g + 1) * S::kGroup); ++c) m += p_tile_mass(w1, c, Mp);
        return m;
      }, &tile_s, &rest_s);
    };
    if (!acc_i) {
      if (sw_s > 0.0) {
        mode = 1;  // residual max(0, p_i - l q_i) ([FI] eq. (2); [SD] "Exactness"; l = 1 there)
        wave_pick_tile(ng, uf * sw_s, [&](int g) {
          double m = 0.0;
          for (int c = g * S::kGroup; c < min(W, (g + 1) * S::kGroup); ++c) m += (double)hi_f(w2[c]);
          return m;
        }, &tile_s, &rest_s);
      } else {
        // the residual has no mass: sample p_i itself ([LH] "Three candidates
        // explain the acceptance rule": a zero-mass residual is not normalised)
        mode = 2;
        pick_p_tile();
      }
    }
    int t = 0;
    // rows that do not start on 16 bytes take the searches that cut each
    // vector from the two aligned vectors covering it
    constexpr bool shifted = SHIFT;
    if (mode) {
      const float invSp = (float)(1.0 / Sp), invSq = (float)((double)a.lenience / Sq);  // l / S_q
      // keep thresholds of the two rows (-inf: nothing filtered)
      const float tp = EXT && a.thr ? thr_target(a, b, i) : -INFINITY;
      const float tq = EXT && a.thr ? thr_draft(a, b, i) : -INFINITY;
      if (mode == 1) {
        auto residual = [&](float xp, float xq) {
          const float wp = xp >= tp ? fast_exp2(fmaf(xp, k, -Mp)) : 0.f;
          const float wq = xq >= tq ? fast_exp2(fmaf(xq, k, -Mq)) : 0.f;
          // both products rounded (no fused multiply-add), so equal p and q
          // give exactly 0
          return fmaxf(__fmul_rn(wp, invSp) - __fmul_rn(wq, invSq), 0.f);
        };
        if constexpr (shifted)
          t = shifted_tile_search<E, S::kPer>(prow, qrow, tile_s * S::kTokens, a.V, rest_s, residual, lds_f, lds_i);
        else
          t = tile_search<E, S::kPer, kThreads>(prow, qrow, tile_s * S::kTokens, a.V, rest_s, residual, lds_f, lds_i);
        // No token of the picked tile has a positive residual in this
        // arithmetic: the tile's mass, formed from the overlap identity over
        // whole tiles, was rounding noise.  Draw from the residual of the whole
        // row instead, token by token in the arithmetic of the search.
        if (t < 0) t = row_search<E, !shifted, kThreads>(prow, qrow, a.V, uf, residual, lds_f, lds_i, lds_d);
        // No token of the row has a positive residual either: p_i and l q_i
        // agree to fp32 everywhere, the residual without mass.  Sample p_i.
        if (t < 0) {
          mode = 2;
          pick_p_tile();
        }
      }
      if (mode == 2) {
        auto pw = [&](float xp, float) { return xp >= tp ? fast_exp2(fmaf(xp, k, -Mp)) : 0.f; };
        if constexpr (shifted)
          t = shifted_tile_search<E, S::kPer>(prow, nullptr, tile_s * S::kTokens, a.V, rest_s, pw, lds_f, lds_i);
        else
          t = tile_search<E, S::kPer, kThreads>(prow, nullptr, tile_s * S::kTokens, a.V, rest_s, pw, lds_f, lds_i);
      }
    }
    if (threadIdx.x == 0) {
      st_u64(P.pair_res + item, pack2i((uint32_t)acc_s | kResMark, (uint32_t)t));
      if (a.p_draft) a.p_draft[o] = (float)px;
      if (a.q_draft) a.q_draft[o] = (float)qx;
      if (a.alpha) a.alpha[o] = (float)alpha_s;
    }
    clear_slots(part1, 2 * W);
    clear_slots(part2, W);
    if (threadIdx.x == 0) {
      if constexpr (EXT) {
        // this finisher is the last reader of the pair's two keep thresholds
        // (the compute workgroups read them before publishing): zero them, so
        // the workspace is left zero
        if (a.thr) {
          a.thr[(size_t)b * (G + 1) + i] = 0.f;
          a.thr[(size_t)a.B * (G + 1) + o] = 0.f;
        }
      }
    }
  }
}

// Bonus item: the token from p_gamma ([FI] Algorithm 1 step 4), then the
// sequence's outputs once every pair result of the sequence is published.
template <class E, int PER, bool ARGMAX, bool EXT, bool SHIFT>
__device__ void finish_bonus(const FusedParams& P, int item, uint64_t* w1, uint64_t* res) {
  using S = SearchShape<E, PER>;
  __shared__ float lds_f[kMaxWaves];
  __shared__ int lds_i[kMaxWaves];
  __shared__ int tile_s;
  __shared__ float rest_s, M_s;
  __shared__ double S_s;
  const VerifyArgs& a = P.a;
  const int G = a.gamma, W = P.W;
  const int b = item - P.n_pairs;
  const float k = a.k;
  const int gb = seq_gamma_of<EXT>(a, b);
  const auto* row = trow<E>(a, b, gb);  // the bonus row follows the sequence's last draft
  uint64_t* part1 = P.part1 + (size_t)item * W * 2;
  // The row's partials and the sequence's pair results (published by other
  // finishers, usually long before) in one wait.  The bonus token is drawn
  // only when every draft was kept.
  uint64_t* pres = P.pair_res + (size_t)b * G;
  const float u_fin = a.uniforms[(size_t)b * (G + 1) + gb];  // fetched before the wait
  const bool ok1 = gather2(part1, 2 * W, w1, pres, gb, res, P.polls);
  int n_acc = 0;
  while (n_acc < gb && ((uint32_t)res[n_acc] & 1u) != 0u) ++n_acc;
  int t_bonus = -1;
  if (!ok1 || n_acc < gb) {
  } else if constexpr (ARGMAX) {
    t_bonus = combine_argmax(w1, W, 0).i;
  } else {
    if (threadIdx.x < kWave) {
      const Norm2 n = wave_norm2(w1, W);
      if (threadIdx.x == 0) {
        M_s = n.Mp;
        S_s = n.Sp;
      }
    }
    __syncthreads();
    const float M = M_s;
    const float tb = EXT && a.thr ? thr_target(a, b, gb) : -INFINITY;  // the bonus row's keep threshold
    const double uf = (double)u_fin;
    wave_pick_tile((W + S::kGroup - 1) / S::kGroup, uf * S_s, [&](int g) {
      double m = 0.0;
      for (int c = g * S::kGroup; c < min(W, (g + 1) * S::kGroup); ++c) m += p_tile_mass(w1, c, M);
      return m;
    }, &tile_s, &rest_s);
    auto bw = [&](float xp, float) { return xp >= tb ? fast_exp2(fmaf(xp, k, -M)) : 0.f; };
    // rows that do not start on 16 bytes take the search that cuts each vector
    // from the two aligned vectors covering it
    if constexpr (SHIFT)
      t_bonus = shifted_tile_search<E, S::kPer>(row, nullptr, tile_s * S::kTokens, a.V, rest_s, bw, lds_f, lds_i);
    else
      t_bonus = tile_search<E, S::kPer, kThreads>(row, nullptr, tile_s * S::kTokens, a.V, rest_s, bw, lds_f, lds_i);
  }
  if constexpr (EXT) {
    // the padding positions (never scheduled as items): NaN outputs
    const float nan = __uint_as_float(0x7fc00000u);
    for (int i = gb + (int)threadIdx.x; i < G; i += (int)blockDim.x) {
      const size_t o = (size_t)b * G + i;
      if (a.alpha) a.alpha[o] = nan;
      if (a.p_draft) a.p_draft[o] = nan;
      if (a.q_draft) a.q_draft[o] = nan;
    }
  }
  if constexpr (EXT) {
    // the last reader of the bonus row's keep threshold; the padding rows'
    // thresholds are never read: zero them all
    if (a.thr && ok1) {
      for (int i = gb + (int)threadIdx.x; i <= G; i += (int)blockDim.x) a.thr[(size_t)b * (G + 1) + i] = 0.f;
      for (int i = gb + (int)threadIdx.x; i < G; i += (int)blockDim.x)
        a.thr[(size_t)a.B * (G + 1) + (size_t)b * G + i] = 0.f;
    }
  }
  if (ok1) {  // the last reader of both; cleared after the draw, whose barriers would wait for the stores
    clear_slots(part1, 2 * W);
    clear_slots(pres, gb);
  }
  if (threadIdx.x == 0) {
    if (ok1) {
      a.n_out[b] = n_acc;
      a.t_out[b] = n_acc < gb ? (int)(uint32_t)(res[n_acc] >> 32) : t_bonus;
    } else {
      a.n_out[b] = -1;  // a wait gave up (the device was shared): no result
      a.t_out[b] = -1;
    }
  }
}

// --------------------------------------------------------------- the kernel

// LDS of one workgroup.  Region A is the bf16 stage on a compute workgroup and
// the finisher's copies of an item's slots on a finisher (a workgroup is one
// or the other); the compute workgroup's poll buffer and normaliser messages
// follow it.
template <class E, int PER, bool ARGMAX, bool SHIFT>
struct Pool {
  // Only the bf16 T > 0 kernel stages.  In argmax mode each wave loads its own
  // tiles when their item comes up: with no team exchange to hide and little
  // arithmetic per token, the three workgroups of a compute unit cover each
  // other's load latency, and that measured faster than the stage (36.9 vs
  // 41.8 us on the B=64 workload); at T > 0 the stage wins (42.5 vs 51.0 us).
  static constexpr bool kStaged = std::is_same<E, BF16>::value && !ARGMAX;
  static constexpr int kFinBytes = (3 * kMaxWaveTiles + SPEC_MAX_GAMMA) * 8;
  static constexpr int kStageBytes = kStaged ? stage_vectors<PER, SHIFT>() * 16 : 0;
  static constexpr int kABytes = kStageBytes > kFinBytes ? kStageBytes : kFinBytes;
  static constexpr int kBytes = kABytes + 2 * kMaxWaveTiles * 8 + 2 * (int)sizeof(NormMsg);
};

// THR: the launch filters by keep thresholds (extended kernels at T > 0 only).
// SHIFT: bf16 rows that do not start on 16 bytes (V % kVec != 0), T > 0,
// with none of the extensions.
// UNITS: the staged loop takes the bonus items two at a time (bf16, T > 0,
// none of the extensions, long team walks).
template <class E, int PER, bool ARGMAX, bool EXT, bool WIDE, bool THR, bool SHIFT, bool UNITS = false>
__global__ __launch_bounds__(kThreads, kMinWaves) void fused_kernel(FusedParams P) {
  using L = Pool<E, PER, ARGMAX, SHIFT>;
  __shared__ __align__(16) unsigned char pool[L::kBytes];
  uint64_t* poll_buf = reinterpret_cast<uint64_t*>(pool + L::kABytes);
  NormMsg* msg = reinterpret_cast<NormMsg*>(pool + L::kABytes + 2 * kMaxWaveTiles * 8);
  uint64_t* fin_w1 = reinterpret_cast<uint64_t*>(pool);
  uint64_t* fin_w2 = fin_w1 + 2 * kMaxWaveTiles;
  uint64_t* fin_res = fin_w2 + kMaxWaveTiles;
  if constexpr (EXT) {
    stage_gamma(P.a);
    __syncthreads();
  }
  const int ncompute = P.nteams * P.K;
  // role of this workgroup: compute (team, rank) or finisher f
  int team = -1, rank = 0, f = 0;
  if ((int)blockIdx.x < ncompute) {
    team = blockIdx.x / P.K;
    rank = blockIdx.x % P.K;
  } else {
    f = blockIdx.x - ncompute;
  }
  if (team >= 0) {
    if constexpr (L::kStaged) {
      compute_loop_staged<PER, ARGMAX, EXT, WIDE, THR, SHIFT, UNITS>(P, team, rank, reinterpret_cast<u32x4*>(pool), poll_buf,
                                                              msg);
    } else {
      const int c = rank * kWavesPerGroup + (int)threadIdx.x / kWave;  // this wave's tile
      const int lo = c * kWave * PER;
      int parity = 0;
      const int n_live = live_count<EXT>(P);
      const int n_lpairs = n_live - P.a.B;
      for (int kth = 0;; ++kth) {
        const int d = team_dense(team, kth, P.nteams, n_live, n_lpairs);
        if (d >= n_live) break;
        const int item = live_item<EXT>(P, d);
        RawPair<E, PER> A;
        issue_item<E, PER, EXT>(P, item, lo, A);
        if (!ARGMAX && item < P.n_pairs) {
          pair_compute_sample<E, PER, EXT, WIDE, THR>(P, item, c, lo, parity, A, poll_buf, msg);
          parity ^= 1;
        } else {
          single_pass_compute<E, PER, ARGMAX, THR>(P, item, c, lo, A, item_thr<EXT, THR>(P, item));
        }
      }
    }
  } else {
    // pairs precede bonus items in the item order, so a finisher never waits
    // on an item it has yet to finish itself
    const int n_live = live_count<EXT>(P);
    for (int d = f; d < n_live; d += P.nfin) {
      const int item = live_item<EXT>(P, d);
      if (item < P.n_pairs)
        finish_pair<E, PER, ARGMAX, EXT, SHIFT>(P, item, fin_w1, fin_w2);
      else
        finish_bonus<E, PER, ARGMAX, EXT, SHIFT>(P, item, fin_w1, fin_res);
    }
  }
}

template <class E>
constexpr int per_of() { return std::is_same<E, BF16>::value ? kPerBF16 : kPerF32; }
static_assert(per_of<BF16>() % 8 == 0 && per_of<F32>() % 8 == 0, "tile shape");

int per_for(int dtype) { return dtype == SPEC_BF16 ? per_of<BF16>() : per_of<F32>(); }

// Workgroups per team for a row of V tokens.
int groups_for(int V, int per) {
  const int group_tokens = kThreads * per;
  return (V + group_tokens - 1) / group_tokens;
}

// Slot layout; the same for both dtypes, so one zeroed workspace serves calls
// of either.
struct Layout {
  size_t off_part1, off_part2, off_res, total;
};

Layout layout(int B, int gamma, int V) {
  // the larger slot count of the two dtypes
  const size_t W = (size_t)std::max(groups_for(V, per_of<BF16>()), groups_for(V, per_of<F32>())) * kWavesPerGroup;
  const size_t n_items = (size_t)B * (gamma + 1), n_pairs = (size_t)B * gamma;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  Layout L{};
  L.off_part1 = 0;
  L.off_part2 = up(L.off_part1 + 16 * n_items * W);
  L.off_res = up(L.off_part2 + 8 * n_pairs * W);
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

template <class E, bool ARGMAX, bool EXT = false, bool SHIFT = false>
hipError_t launch(const VerifyArgs& a, hipStream_t s) {
  const Layout L = layout(a.B, a.gamma, a.V);
  char* ws = static_cast<char*>(a.ws);
  FusedParams P{};
  P.a = a;
  P.K = groups_for(a.V, per_of<E>());
  P.W = P.K * kWavesPerGroup;
  P.n_pairs = a.B * a.gamma;
  P.n_items = a.B * (a.gamma + 1);
  P.part1 = reinterpret_cast<uint64_t*>(ws + L.off_part1);
  P.part2 = reinterpret_cast<uint64_t*>(ws + L.off_part2);
  P.pair_res = reinterpret_cast<uint64_t*>(ws + L.off_res);
  P.polls = g_wait_polls;

  // rows of more than 64 wave tiles take the wide team wait (T > 0 only)
  // keep thresholds take their own instantiations, so the other extended
  // launches carry no code for them
  constexpr bool kThrOk = EXT && !ARGMAX;
  const bool thr = kThrOk && a.thr != nullptr;
  using Kern = void (*)(FusedParams);
  Kern kern;
  if constexpr (SHIFT) {
    static_assert(std::is_same<E, BF16>::value && !ARGMAX, "shifted rows: the bf16 T > 0 kernels");
    kern = P.W > kWave ? (thr ? fused_kernel<E, per_of<E>(), false, EXT, true, kThrOk, true>
                              : fused_kernel<E, per_of<E>(), false, EXT, true, false, true>)
                       : (thr ? fused_kernel<E, per_of<E>(), false, EXT, false, kThrOk, true>
                              : fused_kernel<E, per_of<E>(), false, EXT, false, false, true>);
  } else {
    kern = !ARGMAX && P.W > kWave
               ? (thr ? fused_kernel<E, per_of<E>(), ARGMAX, EXT, !ARGMAX, kThrOk, false>
                      : fused_kernel<E, per_of<E>(), ARGMAX, EXT, !ARGMAX, false, false>)
               : (thr ? fused_kernel<E, per_of<E>(), ARGMAX, EXT, false, kThrOk, false>
                      : fused_kernel<E, per_of<E>(), ARGMAX, EXT, false, false, false>);
  }
  long resident = 0;
  hipError_t e = resident_blocks(kern, &resident);
  if (e != hipSuccess) return e;
  // The grid never exceeds what is resident at once, so every team's members
  // run concurrently and every wait ends.
  P.nfin = (int)std::min<long>(P.n_items, std::max<long>(1, resident / kFinisherDiv));
  P.nteams = (int)std::min<long>(P.n_items, (resident - P.nfin) / P.K);
  if (P.nteams < 1) return hipErrorNotSupported;
  if constexpr (std::is_same<E, BF16>::value && !ARGMAX && !EXT && !SHIFT) {
    if ((long)a.B * a.gamma >= (long)kBonusUnitPairs * P.nteams) {
      // the same kernel with the bonus items two at a time (same resources;
      // the grid is sized again from its own residency all the same)
      kern = P.W > kWave ? fused_kernel<E, per_of<E>(), false, false, true, false, false, true>
                         : fused_kernel<E, per_of<E>(), false, false, false, false, false, true>;
      e = resident_blocks(kern, &resident);
      if (e != hipSuccess) return e;
      P.nfin = (int)std::min<long>(P.n_items, std::max<long>(1, resident / kFinisherDiv));
      P.nteams = (int)std::min<long>(P.n_items, (resident - P.nfin) / P.K);
      if (P.nteams < 1) return hipErrorNotSupported;
    }
  }
  kern<<<dim3(P.nteams * P.K + P.nfin), dim3(kThreads), 0, s>>>(P);
  return hipGetLastError();
}

}  // namespace

void set_wait_limit(unsigned polls) { g_wait_polls = polls ? polls : kDefaultWaitPolls; }
unsigned wait_limit() { return g_wait_polls; }

size_t fused_workspace_bytes(int B, int gamma, int V) { return layout(B, gamma, V).total; }

// Shapes of the T > 0 path.  bf16 rows need not start on 16 bytes (the
// staged kernel copies them from their aligned-down start); fp32 rows and the
// argmax kernels load each lane's vectors directly and need V % kVec == 0.
bool fused_supported(int B, int gamma, int V, int dtype) {
  const int vec = dtype == SPEC_BF16 ? 1 : F32::kVec;
  return B >= 1 && V % vec == 0 && groups_for(V, per_for(dtype)) * kWavesPerGroup <= kMaxWaveTiles &&
         (size_t)B * (gamma + 1) < (1u << 30);
}

hipError_t fused_launch(const VerifyArgs& a, hipStream_t s) {
  if (!fused_supported(a.B, a.gamma, a.V, a.dtype)) return hipErrorNotSupported;
  if (a.gamma_seq && a.B > kGammaLds) return hipErrorNotSupported;
  if ((uintptr_t)a.target % 16 != 0 || (a.gamma > 0 && (uintptr_t)a.draft % 16 != 0)) return hipErrorNotSupported;
  const bool argmax = a.temperature == 0.f;
  const int vec = a.dtype == SPEC_BF16 ? BF16::kVec : F32::kVec;
  const bool shifted = a.V % vec != 0;
  // The extended kernels take lenience below 1, per-sequence draft counts and
  // top-k / top-p thresholds; lenience and the filters do not change argmax
  // mode.
  const bool ext = a.gamma_seq != nullptr || (!argmax && (a.lenience != 1.f || a.thr != nullptr));
  // rows that do not start on 16 bytes: only the plain bf16 T > 0 kernel
  // takes them (the others fall back to the multipass path)
  if (shifted && (argmax || a.dtype != SPEC_BF16)) return hipErrorNotSupported;
  if (a.dtype == SPEC_BF16) {
    if (argmax) return ext ? launch<BF16, true, true>(a, s) : launch<BF16, true>(a, s);
    if (shifted) return ext ? launch<BF16, false, true, true>(a, s) : launch<BF16, false, false, true>(a, s);
    return ext ? launch<BF16, false, true>(a, s) : launch<BF16, false>(a, s);
  }
  if (argmax) return ext ? launch<F32, true, true>(a, s) : launch<F32, true>(a, s);
  return ext ? launch<F32, false, true>(a, s) : launch<F32, false>(a, s);
}

}  // namespace specv
