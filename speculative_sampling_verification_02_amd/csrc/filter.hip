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
// With a workspace and top-k <= 64, three kernels: a streaming kernel lists
// each 8192-token chunk's values at or above a pivot the chunk has k values
// above (their union holds every value >= tau_k), a list-fed kernel (256
// threads per row) runs the exact pick below on the union, and the row kernel
// takes only the rows whose lists overflowed.  Otherwise the row kernel alone:
//
// One workgroup of 1024 threads per row, with the row held in registers (one
// read from memory).  Every pass over the row is a few instructions per token:
//   1. the row maximum (each thread keeps its own maximum too);
//   2. top-k with k <= 1024: a lower bound of tau_k from the thread maxima
//      (each wave's ceil(k/16)-th largest, the smallest of the 16), and the
//      values at or above it copied to an LDS list;
//   3. otherwise, and for top-p, a 16-bin histogram in octaves of softmax
//      weight below the maximum: counts for top-k, fp64 masses for top-p.
//      Each lane owns its own column of bins in LDS, so the additions never
//      contend.  The bin where the running count (mass) from the top reaches
//      k (top_p of the total) is copied to the list;
//   4. the exact threshold is picked inside the list by 8-bit radix passes
//      over the listed keys' range (counts, or masses in 2^-40 fixed point,
//      so sums do not depend on the order of the atomic additions).
// The list is kept in per-thread columns: each thread appends its own
// candidates, with no scan or atomic.  A crossing bin too large for the list
// is refined once (16 finer bins inside it).  With top-k active and its
// survivors listed, top-p runs on the list alone and the row needs no
// exponential pass.  Rows that still do not fit, rows longer than the
// registers hold and rows with no finite logit take a radix select over the
// whole row from memory instead (8 bits per pass).
//
// Masses are exp2((l - m) log2(e) / T) in fp32 (m the row maximum).  The
// histogram adds them in fp64 (each lane in its own fixed order), the lists in
// 2^-40 fixed point; against the exact sum of the same fp32 weights the two
// differ by under 2^-41 per token, far below the fp32 exponential's own ulp.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "specverify.h"
#include "verify_internal.hpp"

namespace specv {
namespace {

constexpr int kFT = 1024;        // threads per row
constexpr int kFNV = 16;         // 16-byte vectors per thread held in registers
constexpr int kNB = 16;          // bins per histogram level (one wave reduces one bin)
constexpr int kCap = 32768;      // slots of the LDS candidate list
constexpr int kCol = kCap / 1024 - 1;  // candidates a thread may list (its column has one spare slot)
constexpr double kMassScale = 1099511627776.0;  // 2^40
static_assert(kFT / kWave == kNB, "one wave per bin in the reductions");

struct FilterArgs {
  const void* target;  // [B][gamma+1][V]
  const void* draft;   // [B][gamma][V]
  int nt;              // target rows B (gamma + 1); rows past nt are draft rows
  int V;
  float k;             // log2(e) / T
  int top_k;           // active when 0 < top_k < V
  float top_p;         // active when top_p < 1
  float* thr;          // [rows] out: keep threshold (-inf: keep all)
  // chunk candidate lists (nullptr: the row kernel works from the row alone)
  int nch;             // chunks of kLChunk tokens per row
  uint32_t* lcount;    // [rows][nch] listed values, kListCap + 1 on overflow
  float* lvals;        // [rows][nch][kListCap]
  int marked_only;     // row kernel: only rows whose threshold holds kMarkedBits
};

// Chunk candidate lists for top-k with k <= kListK.  A streaming kernel lists,
// for every chunk of kLChunk tokens of a row, the values at or above a pivot
// the chunk has at least k values at or above; the union over the row's chunks
// then holds every value >= the row's k-th largest (a chunk whose pivot were
// above it would hold k larger values), so the exact selection runs on the
// union instead of the row.
constexpr int kListK = 64;
// threshold word of a row the list-fed kernel leaves to the row kernel (a NaN
// pattern; a threshold is a logit or -inf)
constexpr uint32_t kMarkedBits = 0x7fc0beefu;
constexpr int kListCap = 256;
constexpr int kLT = 256;           // threads of the list kernel
constexpr int kLChunk = kLT * 32;  // tokens per chunk

struct FilterLds {
  union {
    uint32_t cnt[kNB][kFT];  // per-lane count bins
    double mass[kNB][kFT];   // per-lane mass bins
    float cand[kCap];        // candidate logits: slot s of thread t at s * kFT + t
  } big;
  uint32_t cnt256[256];
  unsigned long long m256[256];
  uint32_t pcnt[2][256];              // the candidate picks' bins, double-buffered
  unsigned long long pmass[2][256];
  double bin_val[kNB];
  float redf[2 * kMaxWaves];
  uint32_t ncand;
  int pick_b;
  double pick_before;
  uint32_t prefix_s, need_s;
  uint32_t kmin_s, kmax_s;
  unsigned long long above_s;
  double target_s;
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

// Elements j0 .. j0 + kVec - 1 of a row that may not be 16-byte aligned, in
// the layout of one 16-byte vector of E (elements at or past V read as 0; the
// callers skip them).
template <class E>
__device__ inline u32x4 load_vec_scalar(const typename E::storage* row, int j0, int V) {
  uint32_t w[4];
  if constexpr (std::is_same<E, BF16>::value) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = j0 + 2 * k < V ? (uint32_t)row[j0 + 2 * k] : 0u;
      const uint32_t hi = j0 + 2 * k + 1 < V ? (uint32_t)row[j0 + 2 * k + 1] : 0u;
      w[k] = lo | (hi << 16);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = j0 + k < V ? __float_as_uint(row[j0 + k]) : 0u;
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

__device__ inline unsigned long long fixed_mass(float w) {
  return (unsigned long long)((double)w * kMassScale + 0.5);
}

// One wave scans 256 bin values from bin 255 down to 0 and finds the first
// bin b at which (sum of the bins above b) + bin b >= need.  Returns b (-1
// when the total falls short) and *before = the sum above b, the same in
// every lane.  Values are exact integers (counts, or fixed-point masses below
// 2^53) or fp64 sums; the scan adds them in one fixed order.
template <class F>
__device__ inline int wave_pick_desc(F binval, double need, double* before_out) {
  const int lane = threadIdx.x;
  double c[4], s = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c[i] = binval(255 - 4 * lane - i);
    s += c[i];
  }
  const double incl = wave_inclusive_scan(s);
  double acc = __shfl_up(incl, 1);
  if (lane == 0) acc = 0.0;
  int found = -1;
  double before = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (found < 0 && acc + c[i] >= need) {
      found = 255 - 4 * lane - i;
      before = acc;
    }
    acc += c[i];
  }
  const unsigned long long hit = __ballot(found >= 0);
  if (!hit) {
    *before_out = 0.0;
    return -1;
  }
  const int leader = __ffsll((long long)hit) - 1;
  *before_out = lane_d(before, leader);
  return __builtin_amdgcn_readlane(found, leader);
}

// ---------------------------------------------------------------- fallback
// Radix select over the whole row read from memory, 8 bits per pass: top-k by
// counts, then top-p by 2^-40 fixed-point mass.  Exact for any row; slower,
// since every pass re-reads the row and bins contend.
// One chunk of one row per workgroup: thread t holds vectors v = 0 .. NV-1 of
// the chunk at tokens lo + (v kLT + t) kVec.  The pivot is the smallest over
// the 4 waves of each wave's m-th largest thread maximum, m = ceil(k / 4): a
// wave then has m maxima at or above it, each a value of the chunk, so the
// chunk has at least 4 m >= k values >= pivot (a chunk with fewer than k
// values gets pivot -inf and lists them all).  The values >= pivot are listed
// in thread order, or the count is marked as overflowed (kListCap + 1).
template <class E, bool ALIGNED>
__global__ __launch_bounds__(kLT) void chunk_list_kernel(FilterArgs f) {
  constexpr int KV = E::kVec;
  constexpr int NV = kLChunk / kLT / KV;
  constexpr int NW = kLT / kWave;
  __shared__ float wm[NW];
  __shared__ uint32_t wsum[NW];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int V = f.V;
  auto row_of = [&](int r) {
    return r < f.nt ? static_cast<const typename E::storage*>(f.target) + (size_t)r * V
                    : static_cast<const typename E::storage*>(f.draft) + (size_t)(r - f.nt) * V;
  };
  // chunk w = r nch + ch of the rows (one per workgroup)
  const int w = blockIdx.x, lo = (w % f.nch) * kLChunk;
  const auto* row = row_of(w / f.nch);
  // ordinary cached loads: the verification that follows reads the same rows
  // (measured 4 us per step faster than streaming loads on the B=64 batch)
  u32x4 cur[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int j0 = lo + (v * kLT + tid) * KV;
    cur[v] = j0 >= V ? u32x4{0u, 0u, 0u, 0u} : ALIGNED ? load_cached(row + j0) : load_vec_scalar<E>(row, j0, V);
  }
  float x[NV * KV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int j0 = lo + (v * kLT + tid) * KV;
    float t[KV];
    E::unpack(cur[v], t);
#pragma unroll
    for (int e = 0; e < KV; ++e) x[v * KV + e] = j0 + e < V ? t[e] : -INFINITY;
  }
  // element i of this thread lies in the row (the last chunk may end early)
  auto in_row = [&](int i) { return lo + ((i / KV) * kLT + tid) * KV + i % KV < V; };
  float tm = -INFINITY;
#pragma unroll
  for (int i = 0; i < NV * KV; ++i) tm = fmaxf(tm, x[i]);
  // the m-th largest of the wave's thread maxima: the largest key K with at
  // least m keys >= K, bit by bit from the top (one ballot per bit)
  const int m = (f.top_k + NW - 1) / NW;  // <= kListK / 4 <= kWave
  const uint32_t key = key_of<32>(tm);
  uint32_t pre = 0;
#pragma unroll
  for (int b = 31; b >= 0; --b) {
    const uint32_t t = pre | (1u << b);
    if (__popcll(__ballot(key >= t)) >= m) pre = t;
  }
  const float mth = value_of<32>(pre);
  if (lane == 0) wm[wid] = mth;
  __syncthreads();
  float pivot = wm[0];
#pragma unroll
  for (int q = 1; q < NW; ++q) pivot = fminf(pivot, wm[q]);
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < NV * KV; ++i) c += in_row(i) && x[i] >= pivot ? 1u : 0u;
  // offsets: inclusive scan within the wave, then the waves' totals
  uint32_t incl = c;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t o = (uint32_t)__shfl_up((int)incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) wsum[wid] = incl;
  __syncthreads();
  uint32_t base = 0, total = 0;
#pragma unroll
  for (int q = 0; q < NW; ++q) {
    base += q < wid ? wsum[q] : 0u;
    total += wsum[q];
  }
  if (tid == 0) f.lcount[w] = total <= (uint32_t)kListCap ? total : (uint32_t)kListCap + 1u;
  if (total <= (uint32_t)kListCap) {
    uint32_t o = base + incl - c;
    float* out = f.lvals + (size_t)w * kListCap;
#pragma unroll
    for (int i = 0; i < NV * KV; ++i) {
      if (in_row(i) && x[i] >= pivot) out[o++] = x[i];
    }
  }
}

template <class E, bool ALIGNED>
__device__ __attribute__((always_inline)) inline float radix_threshold(const typename E::storage* row,
                                                                       const FilterArgs f, FilterLds& L) {
  constexpr int KB = std::is_same<E, BF16>::value ? 16 : 32;
  constexpr int kPasses = KB / 8;
  const int tid = threadIdx.x;
  auto for_each = [&](auto fn) {
    for (int j0 = tid * E::kVec; j0 < f.V; j0 += kFT * E::kVec) {
      float t[E::kVec];
      E::unpack(ALIGNED ? load_cached(row + j0) : load_vec_scalar<E>(row, j0, f.V), t);
#pragma unroll
      for (int e = 0; e < E::kVec; ++e)
        if (ALIGNED || j0 + e < f.V) fn(t[e]);
    }
  };
  const bool use_k = f.top_k > 0 && f.top_k < f.V;
  const bool use_p = f.top_p < 1.f;

  uint32_t tau_k = 0;  // the smallest key: keep all
  if (use_k) {
    __syncthreads();
    if (tid == 0) {
      L.prefix_s = 0;
      L.need_s = (uint32_t)f.top_k;  // rank from the top among the keys that share the prefix
    }
    for (int pass = 0; pass < kPasses; ++pass) {
      const int shift = KB - 8 * (pass + 1);
      const uint32_t mask = pass == 0 ? 0u : (~0u << (shift + 8)) & (KB == 32 ? ~0u : 0xffffu);
      for (int b = tid; b < 256; b += kFT) L.cnt256[b] = 0;
      __syncthreads();
      const uint32_t prefix = L.prefix_s;
      for_each([&](float x) {
        const uint32_t key = key_of<KB>(x);
        if ((key & mask) == prefix) atomicAdd(&L.cnt256[(key >> shift) & 0xffu], 1u);
      });
      __syncthreads();
      if (tid == 0) {
        const uint32_t need = L.need_s;
        uint32_t acc = 0;
        for (int b = 255; b >= 0; --b) {
          if (acc + L.cnt256[b] >= need) {
            L.need_s = need - acc;
            L.prefix_s = prefix | ((uint32_t)b << shift);
            break;
          }
          acc += L.cnt256[b];
        }
      }
      __syncthreads();
    }
    tau_k = L.prefix_s;
  }

  uint32_t tau_p = 0;
  if (use_p) {
    // the row maximum, for weights exp2((l - m) k) in (0, 1]
    float m = -INFINITY;
    for_each([&](float x) { m = fmaxf(m, x); });
    m = block_max(m, L.redf);
    __syncthreads();
    if (tid == 0) {
      L.prefix_s = 0;
      L.above_s = 0;
    }
    for (int pass = 0; pass < kPasses; ++pass) {
      const int shift = KB - 8 * (pass + 1);
      const uint32_t mask = pass == 0 ? 0u : (~0u << (shift + 8)) & (KB == 32 ? ~0u : 0xffffu);
      for (int b = tid; b < 256; b += kFT) L.m256[b] = 0;
      __syncthreads();
      const uint32_t prefix = L.prefix_s;
      for_each([&](float x) {
        const uint32_t key = key_of<KB>(x);
        if (key >= tau_k && (key & mask) == prefix && x != -INFINITY)
          atomicAdd(&L.m256[(key >> shift) & 0xffu], fixed_mass(__builtin_amdgcn_exp2f((x - m) * f.k)));
      });
      __syncthreads();
      if (tid == 0) {
        if (pass == 0) {
          unsigned long long total = 0;
          for (int b = 0; b < 256; ++b) total += L.m256[b];
          L.target_s = (double)f.top_p * (double)total;
        }
        unsigned long long acc = L.above_s;
        for (int b = 255; b >= 0; --b) {
          if ((double)(acc + L.m256[b]) >= L.target_s) {
            L.above_s = acc;
            L.prefix_s = prefix | ((uint32_t)b << shift);
            break;
          }
          acc += L.m256[b];
        }
      }
      __syncthreads();
    }
    tau_p = L.prefix_s;
  }
  return (use_k || use_p) ? value_of<KB>(max(tau_k, tau_p)) : -INFINITY;
}

// ------------------------------------------------------------- fast path

// ALIGNED: 16-byte aligned rows of whole vectors (V a multiple of the vector
// width); otherwise elements are loaded one by one and checked against V.
// The radix pick of the threshold kernels (see the row kernel): over the
// listed values >= lo, slot q of thread t at cand[q NT + t], my_n of them in
// this thread's column.  `weight(x)` is the softmax weight of value x on the
// scale of base and need (MASS only).  Called by all NT threads of the
// workgroup.
template <class E, int NT, bool MASS, class LdsT, class WFn>
__device__ __attribute__((always_inline)) inline float list_pick(LdsT& L, const float* cand, uint32_t my_n, float lo,
                                                               double base, double need, WFn weight, float top_p) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  constexpr int KB = std::is_same<E, BF16>::value ? 16 : 32;
  // key range of the listed values >= lo
  if (tid == 0) {
    L.kmin_s = 0xffffffffu;
    L.kmax_s = 0u;
  }
  __syncthreads();
  uint32_t kmn = 0xffffffffu, kmx = 0u;
  for (uint32_t q = 0; q < my_n; ++q) {  // this thread's column of the list
    const float x = cand[q * NT + tid];
    if (x >= lo) {
      const uint32_t key = key_of<KB>(x);
      kmn = min(kmn, key);
      kmx = max(kmx, key);
    }
  }
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) {
    kmn = min(kmn, (uint32_t)__shfl_xor((int)kmn, off));
    kmx = max(kmx, (uint32_t)__shfl_xor((int)kmx, off));
  }
  if (lane == 0) {
    atomicMin(&L.kmin_s, kmn);
    atomicMax(&L.kmax_s, kmx);
  }
  __syncthreads();
  const uint32_t kmin = L.kmin_s, span = L.kmax_s - L.kmin_s;
  const int nbits = span ? 32 - __clz((int)span) : 0;
  uint32_t prefix = 0;  // chosen high bits of (key - kmin)
  // each pass picks bits [shift, hi) of (key - kmin), hi falling from nbits
  // to 0; a span of one key still takes one pass (the mass total).  The
  // bins are double-buffered: a pass clears the next pass's set, so it
  // needs only the barrier after its additions and the one after the pick.
  if (tid < 256) {
    if constexpr (MASS) L.pmass[0][tid] = 0ull;
    else L.pcnt[0][tid] = 0u;
  }
  __syncthreads();
  int hi = nbits, buf = 0;
  do {
    const int shift = hi > 8 ? hi - 8 : 0;
    const uint32_t hi_mask = hi >= 32 ? 0u : ~0u << hi;
    const uint32_t dmask = (1u << (hi - shift)) - 1u;
    if (tid < 256) {
      if constexpr (MASS) L.pmass[buf ^ 1][tid] = 0ull;
      else L.pcnt[buf ^ 1][tid] = 0u;
    }
    for (uint32_t q = 0; q < my_n; ++q) {
      const float x = cand[q * NT + tid];
      const uint32_t d = key_of<KB>(x) - kmin;
      if (x >= lo && (d & hi_mask) == prefix) {
        if constexpr (MASS)
          atomicAdd(&L.pmass[buf][(d >> shift) & dmask], fixed_mass(weight(x)));
        else
          atomicAdd(&L.pcnt[buf][(d >> shift) & dmask], 1u);
      }
    }
    __syncthreads();
    auto binv = [&](int b) -> double {
      if constexpr (MASS) return (double)L.pmass[buf][b] / kMassScale;
      else return (double)L.pcnt[buf][b];
    };
    if (wid == 0) {
      if constexpr (MASS) {
        if (need < 0.0) {  // top_p of the listed total (wave 0 only needs it)
          double s = 0.0;
#pragma unroll
          for (int i = 0; i < 4; ++i) s += (double)L.pmass[buf][lane * 4 + i];
          need = (double)top_p * (wave_sum(s) / kMassScale);
          base = 0.0;
        }
      }
      double before;
      int b = wave_pick_desc(binv, need - base, &before);
      if (b < 0) {
        // the list's total fell short of need by rounding (the fixed-point
        // list against the histogram's fp64 sum): keep all of this prefix
        b = 0;
        before = 0.0;
        for (int q = 255; q >= 0; --q) {
          if (binv(q) > 0.0) {
            b = q;
            break;
          }
        }
        for (int q = 255; q > b; --q) before += binv(q);
      }
      if (lane == 0) {
        L.pick_b = b;
        L.pick_before = before;
      }
    }
    __syncthreads();  // every read of this pass's bins is done
    base += L.pick_before;
    prefix |= (uint32_t)L.pick_b << shift;
    hi = shift;
    buf ^= 1;
  } while (hi > 0);
  return value_of<KB>(kmin + prefix);
}

// The thresholds of the rows whose chunk lists all fit, from the lists alone
// (one 256-thread workgroup per row, about 40 KB of LDS, so every row of a
// batch is resident at once).  The union of a row's lists, value i in slot
// i / kLTT of thread i % kLTT, holds every value >= the row's k-th largest,
// and with it the row maximum: the exact k-th largest and, with top-p, the
// nucleus of the survivors are the row kernel's own picks on the union, so
// the thresholds are those of the row path.  Every list entry and count is set
// back to zero.  A row with an overflowed chunk, more listed values than the
// LDS holds, or no finite value gets kMarkedBits for the row kernel.
constexpr int kLTT = 256;
constexpr int kListSlots = 8192;
struct ListLds {
  float cand[kListSlots];
  uint32_t pcnt[2][256];
  unsigned long long pmass[2][256];
  float redf[2 * kMaxWaves];
  uint32_t kmin_s, kmax_s;
  int pick_b;
  double pick_before;
  uint32_t lpre[257];  // exclusive prefix of the row's chunk list counts
  uint32_t lovf;
};

template <class E>
__global__ __launch_bounds__(kLTT) void list_threshold_kernel(FilterArgs f) {
  __shared__ ListLds L;
  const int tid = threadIdx.x, r = blockIdx.x;
  const size_t s0 = (size_t)r * f.nch;
  if (tid == 0) {
    uint32_t acc = 0, ovf = 0;
    for (int c = 0; c < f.nch; ++c) {
      L.lpre[c] = acc;
      const uint32_t n = f.lcount[s0 + c];
      ovf |= n > (uint32_t)kListCap ? 1u : 0u;
      acc += min(n, (uint32_t)kListCap);
    }
    L.lpre[f.nch] = acc;
    L.lovf = ovf;
  }
  __syncthreads();
  const uint32_t total = L.lpre[f.nch];
  const bool listed = L.lovf == 0u && total <= (uint32_t)kListSlots;
  if (tid < f.nch) f.lcount[s0 + tid] = 0u;
  uint32_t my_n = 0;
  float lmax = -INFINITY;
  int c = 0;
  for (uint32_t i = tid, q = 0; i < total; i += kLTT, ++q) {
    while (L.lpre[c + 1] <= i) ++c;  // the chunk of entry i (i grows, so c only advances)
    float* src = f.lvals + (s0 + c) * kListCap + (i - L.lpre[c]);
    const float x = *src;
    *src = 0.f;
    if (listed) {
      L.cand[q * kLTT + tid] = x;
      lmax = fmaxf(lmax, x);
      ++my_n;
    }
  }
  if (!listed) {
    if (tid == 0) f.thr[r] = __uint_as_float(kMarkedBits);
    return;
  }
  const float mx = block_max(lmax, L.redf);  // the row maximum
  if (mx == -INFINITY) {
    if (tid == 0) f.thr[r] = __uint_as_float(kMarkedBits);
    return;
  }
  const float k = f.k;
  auto weight = [&](float x) { return __builtin_amdgcn_exp2f((x - mx) * k); };
  const float tau_k = list_pick<E, kLTT, false>(L, L.cand, my_n, -INFINITY, 0.0, (double)f.top_k, weight, f.top_p);
  float tau_p = -INFINITY;
  if (f.top_p < 1.f) tau_p = list_pick<E, kLTT, true>(L, L.cand, my_n, tau_k, 0.0, -1.0, weight, f.top_p);
  if (tid == 0) f.thr[r] = fmaxf(tau_k, tau_p);
}

template <class E, bool ALIGNED>
__global__ __launch_bounds__(kFT) void row_threshold_kernel(FilterArgs f) {
  constexpr int KV = E::kVec;
  __shared__ FilterLds L;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int r = blockIdx.x;
  const auto* row = r < f.nt ? static_cast<const typename E::storage*>(f.target) + (size_t)r * f.V
                             : static_cast<const typename E::storage*>(f.draft) + (size_t)(r - f.nt) * f.V;
  const int V = f.V;
  const bool use_k = f.top_k > 0 && f.top_k < V;
  const bool use_p = f.top_p < 1.f;
  if (!use_k && !use_p) {
    if (tid == 0) f.thr[r] = -INFINITY;
    return;
  }
  // after the list-fed kernel: only the rows it marked
  if (f.marked_only && __float_as_uint(f.thr[r]) != kMarkedBits) return;
  // rows longer than the registers hold take the radix select from memory
  bool fallback = V > kFT * kFNV * KV;

  // the row, in registers: vector v of thread t holds tokens (v kFT + t) KV ..
  u32x4 raw[kFNV];
#pragma unroll
  for (int v = 0; v < kFNV; ++v) {
    const int j0 = (v * kFT + tid) * KV;
    raw[v] = fallback || j0 >= V ? u32x4{0u, 0u, 0u, 0u}
             : ALIGNED          ? load_cached(row + j0)
                                : load_vec_scalar<E>(row, j0, V);
  }
  auto each = [&](auto fn) {
#pragma unroll
    for (int v = 0; v < kFNV; ++v) {
      const int j0 = (v * kFT + tid) * KV;
      if (j0 < V) {
        // a copy of the words that is opaque to the compiler, so every pass
        // unpacks afresh instead of keeping up to 128 unpacked values live
        u32x4 w = raw[v];
        asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
        float t[KV];
        E::unpack(w, t);
#pragma unroll
        for (int e = 0; e < KV; ++e)
          if (ALIGNED || j0 + e < V) fn(t[e]);
      }
    }
  };

  // ---- 1. row maximum; each thread's own maximum is kept for the top-k pivot
  float tmax = -INFINITY;
  if (!fallback) each([&](float x) { tmax = fmaxf(tmax, x); });
  float mx = -INFINITY;
  if (!fallback) {
    mx = block_max(tmax, L.redf);
    fallback = mx == -INFINITY;  // no finite logit
  }
  const float k = f.k;
  // Histogram bins are two octaves of softmax weight wide: t(x) ~ (m - x) k / 2,
  // bin = clamp(t, 0, 15) truncated (bin 15 also takes the tail and -inf).
  // A second level splits one bin j into 16: bin = clamp(16 (t - j), 0, 15).
  const float c = 0.5f * k, mc = mx * c;
  auto binof = [](float t) { return (int)__builtin_amdgcn_fmed3f(t, 0.f, 15.f); };
  int lv_j = 0;     // the bin a second level refines
  uint32_t my_n = 0;  // values this thread has in the candidate list

  // One pass over the row.  Values in range are those >= lo and, at level 1,
  // those of level-0 bin lv_j; `b` is the bin at the pass's level.
  //   kind 0: per-lane count histogram, reduced to L.bin_val[16]
  //   kind 1: per-lane fp64 mass histogram, reduced to L.bin_val[16]
  //   kind 2: copy the values in range whose bin is jsel to the candidate
  //           list; returns how many there were
  //   kind 3: copy every value >= lo (no bins); returns how many there were
  // The per-lane additions are branchless (out of range adds 0).
  auto run_pass = [&](auto level_c, auto kind_c, float lo, int jsel) -> uint32_t {
    constexpr int LEVEL = decltype(level_c)::value;
    constexpr int kind = decltype(kind_c)::value;
    auto locate = [&](float x, int* b) -> bool {
      const float t = fmaf(x, -c, mc);
      const int b0 = binof(t);
      if constexpr (LEVEL == 0) {
        *b = b0;
        return x >= lo;
      } else {
        *b = binof(fmaf(t, 16.f, -16.f * (float)lv_j));
        return b0 == lv_j && x >= lo;
      }
    };
    __syncthreads();  // the LDS region may still hold a candidate list or bins
    if constexpr (kind == 0) {
#pragma unroll
      for (int b = 0; b < kNB; ++b) L.big.cnt[b][tid] = 0u;
      each([&](float x) {
        int b;
        const bool in = locate(x, &b);
        __hip_atomic_fetch_add(&L.big.cnt[b][tid], (uint32_t)in, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      });
    } else if constexpr (kind == 1) {
#pragma unroll
      for (int b = 0; b < kNB; ++b) L.big.mass[b][tid] = 0.0;
      each([&](float x) {
        int b;
        const bool in = locate(x, &b);
        const float w = in ? __builtin_amdgcn_exp2f((x - mx) * k) : 0.f;
        __hip_atomic_fetch_add(&L.big.mass[b][tid], (double)w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      });
    } else {
      static_assert(kind == 2 || kind == 3, "pass kinds 0-3");
      // Each thread lists its own candidates in its column of the list (slot
      // s of thread t at s * kFT + t: no bank conflicts, no scan, no atomic).
      // The write is branchless: every value goes to the next free slot, and
      // only a candidate advances it (the column's spare slot takes the
      // writes past the last usable one).  A thread with more than kCol
      // candidates makes the list overflow.
      uint32_t cnt = 0;
      each([&](float x) {
        bool in;
        if constexpr (kind == 3) {
          in = x >= lo;
        } else {
          int b;
          in = locate(x, &b) && b == jsel;
        }
        L.big.cand[min(cnt, (uint32_t)kCol) * kFT + tid] = x;
        cnt += (uint32_t)in;
      });
      my_n = min(cnt, (uint32_t)kCol);
      const float2 r = block_sum2((float)cnt, cnt > (uint32_t)kCol ? 1.f : 0.f, L.redf);  // exact: <= 2^17
      if (tid == 0) L.ncand = r.y > 0.f ? (uint32_t)kCap + 1u : (uint32_t)r.x;
    }
    __syncthreads();
    if constexpr (kind >= 2) return L.ncand;
    // wave w sums bin w over all lanes in one fixed order
    double s = 0.0;
    if constexpr (kind == 0) {
#pragma unroll
      for (int i = 0; i < kFT / kWave; ++i) s += (double)L.big.cnt[wid][lane + i * kWave];
    } else {
#pragma unroll
      for (int i = 0; i < kFT / kWave; ++i) s += L.big.mass[wid][lane + i * kWave];
    }
    s = wave_sum(s);
    if (lane == 0) L.bin_val[wid] = s;
    __syncthreads();
    return 0u;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  // first bin from the top whose running sum (from `base`) reaches need:
  // returns the bin (-1 if none) and the running sum above it
  auto crossing = [&](double base, double need, double* above) {
    double acc = base;
    for (int b = 0; b < kNB; ++b) {
      if (acc + L.bin_val[b] >= need) {
        *above = acc;
        return b;
      }
      acc += L.bin_val[b];
    }
    *above = acc;
    return -1;
  };
  // Radix pick over the listed values >= lo: the largest key K (returned as
  // its value) with base + W(listed keys >= K) >= need, W a count (MASS
  // false) or the 2^-40 fixed-point softmax mass (MASS true).  need < 0 (mass
  // only) means top_p of the listed values' own total, with base 0.  The
  // 8-bit digits are taken over the keys' actual range [kmin, kmax], so the
  // first pass already spreads a narrow list over many bins (few colliding
  // LDS atomics) and a list of close values needs few passes.  Keys are the
  // 16 significant bits for bf16 rows (the list holds widened bf16 values).
  auto pick = [&](auto mass_c, float lo, double base, double need) -> float {
    return list_pick<E, kFT, decltype(mass_c)::value>(L, L.big.cand, my_n, lo, base, need,
                                                      [&](float x) { return __builtin_amdgcn_exp2f((x - mx) * k); },
                                                      f.top_p);
  };
  using BF = std::integral_constant<bool, false>;
  using BT = std::integral_constant<bool, true>;
  // the rank-th largest listed value >= lo (ties counted)
  auto select_kth = [&](uint32_t rank, float lo) { return pick(BF{}, lo, 0.0, (double)rank); };
  // the nucleus threshold of the listed values >= lo: base + mass(>= tau) >=
  // target (target < 0: top_p of their own total)
  auto nucleus = [&](double base, double target, float lo) { return pick(BT{}, lo, base, target); };

  // ---- 2-4. the filters, as a sequence of passes; each (level, kind) of
  // run_pass has one call site, so its unrolled body is instantiated once
  enum { K_PIVOT, K_HIST0, K_COPY0, K_HIST1, K_COPY1, P_START, P_SURV, P_HIST0, P_COPY0, P_HIST1, P_COPY1, DONE };
  float tau_k = -INFINITY, tau_p = -INFINITY, pivot = -INFINITY;
  bool survivors_listed = false;  // the list holds every value >= tau_k
  double above = 0.0, target = 0.0;
  uint32_t n = 0;
  int j = 0;
  int state = fallback ? DONE : !use_k ? P_START : f.top_k <= kFT ? K_PIVOT : K_HIST0;
  while (state != DONE) {
    if (state == P_START) {
      if (!use_p) {
        state = DONE;
      } else if (survivors_listed) {  // the nucleus of the listed survivors: no pass
        tau_p = nucleus(0.0, -1.0, tau_k);
        state = DONE;
      } else {
        state = use_k && above + (double)n <= (double)kCap ? P_SURV : P_HIST0;
      }
      continue;
    }
    if (state == K_PIVOT) {
      // A lower bound of tau_k with few values above it: each wave finds the
      // m-th largest of its 64 thread maxima (m = ceil(k / 16), by m rounds
      // of a wave maximum that knocks out one holder), and the pivot is the
      // smallest of the 16.  Every wave then holds m maxima >= pivot, and
      // each maximum is a value of the row: at least 16 m >= k values are
      // >= pivot, so tau_k >= pivot and the exact k-th largest is among them.
      const int m = (f.top_k + kNB - 1) / kNB;
      float v = tmax, mth = -INFINITY;
      for (int r = 0; r < m; ++r) {
        mth = wave_max(v);
        const unsigned long long hit = __ballot(v == mth);
        if (lane == __ffsll((long long)hit) - 1) v = -INFINITY;
      }
      pivot = -block_max(-mth, L.redf);
    }
    const bool lv1 = state == K_HIST1 || state == K_COPY1 || state == P_HIST1 || state == P_COPY1;
    const int kind = (state == K_HIST0 || state == K_HIST1) ? 0
                     : (state == P_HIST0 || state == P_HIST1) ? 1
                     : (state == K_PIVOT || state == P_SURV) ? 3 : 2;
    const float lo = state == K_PIVOT ? pivot : state > P_START ? tau_k : -INFINITY;
    uint32_t got;
    if (kind == 3)
      got = run_pass(I0{}, I3{}, lo, 0);
    else if (!lv1)
      got = kind == 0 ? run_pass(I0{}, I0{}, lo, j)
            : kind == 1 ? run_pass(I0{}, I1{}, lo, j) : run_pass(I0{}, I2{}, lo, j);
    else
      got = kind == 0 ? run_pass(I1{}, I0{}, lo, j)
            : kind == 1 ? run_pass(I1{}, I1{}, lo, j) : run_pass(I1{}, I2{}, lo, j);
    double ab = 0.0;
    switch (state) {
      case K_PIVOT:
        n = got;
        if (n <= (uint32_t)kCap) {
          tau_k = select_kth((uint32_t)f.top_k, -INFINITY);
          survivors_listed = true;
          state = P_START;
        } else {
          state = K_HIST0;
        }
        break;
      case K_HIST0:  // found: all V values are counted (-inf in bin 15) and k < V
        j = crossing(0.0, (double)f.top_k, &above);
        state = K_COPY0;
        break;
      case P_HIST0: {
        double total = 0.0;
        for (int b = 0; b < kNB; ++b) total += L.bin_val[b];
        target = (double)f.top_p * total;
        j = crossing(0.0, target, &above);  // found: the running sum ends at total > target
        state = P_COPY0;
        break;
      }
      case K_HIST1:
      case P_HIST1:
        j = crossing(above, state == K_HIST1 ? (double)f.top_k : target, &ab);
        above = ab;
        state = j < 0 ? DONE : state == K_HIST1 ? K_COPY1 : P_COPY1;
        fallback = j < 0;
        break;
      default:  // a list was copied
        n = got;
        if (n > (uint32_t)kCap) {
          if (state == K_COPY0 || state == P_COPY0) {  // refine the crossing bin once
            lv_j = j;
            state = state == K_COPY0 ? K_HIST1 : P_HIST1;
          } else {
            fallback = true;
            state = DONE;
          }
        } else if (state == K_COPY0 || state == K_COPY1) {
          tau_k = select_kth((uint32_t)((double)f.top_k - above), -INFINITY);
          state = P_START;
        } else if (state == P_SURV) {
          tau_p = nucleus(0.0, -1.0, tau_k);
          state = DONE;
        } else {
          tau_p = nucleus(above, target, -INFINITY);
          state = DONE;
        }
        break;
    }
  }
  const float t = fallback ? radix_threshold<E, ALIGNED>(row, f, L) : fmaxf(tau_k, tau_p);
  if (tid == 0) f.thr[r] = t;
}

// ------------------------------------------------- streaming nucleus path
//
// top-p without top-k, on aligned rows, with a workspace: four launches that
// spread every row over the whole device (the row kernel holds one row per
// compute unit at a time).
//   1. nucleus_stats_kernel, one 128-thread workgroup per chunk of kNChunk
//      tokens of a row (eight share a compute unit, so one's loads overlap
//      another's arithmetic): the chunk's maximum scaled logit c = fl(m k)
//      and its softmax weights exp2(fma(l, k, -c)) summed per octave.  Token
//      l falls in octave floor(fl(l k)), a function of l alone, so a tie
//      group never straddles two octaves, within a chunk or across chunks.
//      The bins are the 31 octaves from floor(c) down and a tail bin for
//      every lower one.  A weight in bin b lies in [2^-b-1, 2^-b+1) and is
//      added as the integer trunc(w 2^(24 + b)) < 2^25 (at most 2^-23 of it
//      lost) to the thread's own LDS column with an integer atomic (LDS float
//      atomics are an order of magnitude slower on gfx950); integer sums are
//      exact, so the order of the additions does not matter.
//   2. nucleus_cross_kernel, one wave per row: the row's octave masses (each
//      chunk's scaled by exp2(c_chunk - C), C the row's maximum, in fp64 and
//      one fixed order), the total Z, the crossing octave o* (the first from
//      the top at which the running mass reaches top_p Z) with the mass above
//      it, and the logit interval [lo, hi) of octave o*.
//   3. nucleus_list_kernel, per chunk: lists the chunk's values in [lo, hi)
//      (at most kNThreadCap per thread and kChunkCap per chunk).
//   4. nucleus_pick_kernel, per row: the exact threshold within the row's
//      lists (the row kernel's radix pick over 2^-40 fixed-point weights
//      exp2(fma(l, k, -C)), starting from the mass above o*).
// A row the path cannot finish (no finite logit, a crossing inside a chunk's
// tail bin or more than 64 octaves down, an overflowing list) gets
// kMarkedBits, and the row kernel takes it.  The path leaves its workspace
// zero: the cross kernel clears the chunk records it read, and the pick
// kernel the row's record, list counts and lists.
constexpr int kNT = 128;              // threads of the chunk kernels
constexpr int kNPer = 64;             // tokens per thread
constexpr int kNChunk = kNT * kNPer;  // tokens per chunk
constexpr int kOB = 32;               // octave bins of a chunk, the last one the tail
constexpr int kNThreadCap = 16;       // values a thread may list per chunk
constexpr int kChunkCap = 512;        // values a chunk may list
constexpr int kNCap = kListSlots;     // values a row may list in all
constexpr uint32_t kChunkOverflow = kChunkCap + 1;
// Waves per SIMD the chunk kernels' registers allow (an fp32 chunk's raw words
// take twice a bf16 chunk's).
template <class E>
constexpr int chunk_waves() { return std::is_same<E, BF16>::value ? 4 : 3; }

struct ChunkStat {
  float c;  // fl(m k), m the chunk's maximum logit (-inf: no finite logit)
  float pad;
  double mass[kOB];  // weights relative to exp2(c), per octave below floor(c)
};
struct RowCross {
  float C;       // the row's maximum scaled logit
  float octave;  // o*, an integer as a float; NaN: the row is left to the row kernel
  float lo, hi;  // the logits of octave o*: lo <= l < hi
  double base;   // mass of the octaves above o*, relative to exp2(C)
  double target;  // top_p times the row's total mass
};

template <class E>
__device__ inline const typename E::storage* filter_row(const FilterArgs& f, int r) {
  return r < f.nt ? static_cast<const typename E::storage*>(f.target) + (size_t)r * f.V
                  : static_cast<const typename E::storage*>(f.draft) + (size_t)(r - f.nt) * f.V;
}

// The raw vectors of one chunk: vector s of thread t at lo + (s kNT + t) kVec.
template <class E>
struct ChunkRaw {
  u32x4 v[kNPer / E::kVec];
};

// Loads chunk q (row q / nch); vectors past V read as zero (V is a multiple
// of kVec) and are masked to -inf by unpack_chunk.
template <class E>
__device__ inline void issue_chunk(const FilterArgs& f, int nch, int q, ChunkRaw<E>& raw) {
  const int lo = (q % nch) * kNChunk;
  const auto* row = filter_row<E>(f, q / nch);
#pragma unroll
  for (int s = 0; s < kNPer / E::kVec; ++s) {
    const int j0 = lo + (s * kNT + (int)threadIdx.x) * E::kVec;
    raw.v[s] = j0 < f.V ? load_cached(row + j0) : u32x4{0u, 0u, 0u, 0u};
  }
}

template <class E>
__device__ inline void unpack_chunk(const ChunkRaw<E>& raw, int lo, int V, float (&x)[kNPer]) {
  constexpr int NS = kNPer / E::kVec;
  if (lo + kNChunk <= V) {  // no per-token select
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      float t[E::kVec];
      E::unpack(raw.v[s], t);
#pragma unroll
      for (int e = 0; e < E::kVec; ++e) x[s * E::kVec + e] = t[e];
    }
    return;
  }
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int j0 = lo + (s * kNT + (int)threadIdx.x) * E::kVec;
    float t[E::kVec];
    E::unpack(raw.v[s], t);
#pragma unroll
    for (int e = 0; e < E::kVec; ++e) x[s * E::kVec + e] = j0 < V ? t[e] : -INFINITY;
  }
}

// floor(x) as an integer in one instruction; out of range saturates (-inf
// gives INT_MIN), which a C++ conversion would leave undefined.
__device__ inline int floor_i32(float x) {
  int r;
  asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}
// Octave of a token: floor(fl(l k)).
__device__ inline int octave_of(float x, float k) { return floor_i32(x * k); }

// The smallest float v (-inf included) with octave_of(v, k) >= o, over the
// order-preserving keys of the floats (octave_of is non-decreasing in v for
// k > 0).  +inf if there is none below +inf.  The search starts from the key
// of o / k, which lies within a few keys of the answer, and steps one key at a
// time (at most kOctSteps each way); a start that far off takes a binary
// search instead.  Either way the answer is the same float.
constexpr int kOctSteps = 8;
__device__ inline float first_in_octave(int o, float k) {
  auto value = [](uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key ^ 0x80000000u) : ~key);
  };
  auto key_of_f = [](float v) {
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  };
  const uint32_t kmin = 0x007fffffu, kmax = 0xff800000u;  // the keys of -inf and +inf
  if (octave_of(value(kmin), k) >= o) return -INFINITY;
  // invariant of the search: octave_of(value(lo)) < o <= octave_of(value(hi))
  uint32_t lo = kmin, hi = kmax;
  const float guess = (float)((double)o / (double)k);
  uint32_t g = guess != guess ? kmax : key_of_f(guess);
  g = g < kmin ? kmin : (g > kmax ? kmax : g);
  if (octave_of(value(g), k) >= o) {
    hi = g;
    for (int i = 0; i < kOctSteps && hi - 1u > kmin; ++i) {  // step down while the key below still qualifies
      if (octave_of(value(hi - 1u), k) < o) {
        lo = hi - 1u;
        break;
      }
      --hi;
    }
  } else {
    lo = g;
    for (int i = 0; i < kOctSteps && lo + 1u < kmax; ++i) {  // step up until a key qualifies
      if (octave_of(value(lo + 1u), k) >= o) {
        hi = lo + 1u;
        break;
      }
      ++lo;
    }
  }
  while (hi - lo > 1u) {
    const uint32_t mid = lo + (hi - lo) / 2u;
    if (octave_of(value(mid), k) >= o)
      hi = mid;
    else
      lo = mid;
  }
  return value(hi);
}

// One chunk per workgroup: work(raw, q) on chunk q = the workgroup's index
// (called by the whole workgroup).
template <class E, class Work>
__device__ __attribute__((always_inline)) inline void chunk_loop(const FilterArgs& f, int nch, int nq, Work work) {
  const int q = blockIdx.x;
  if (q >= nq) return;
  ChunkRaw<E> A;
  issue_chunk<E>(f, nch, q, A);
  work(A, q);
}

template <class E>
__global__ __launch_bounds__(kNT, chunk_waves<E>()) void nucleus_stats_kernel(FilterArgs f, int nch, int nq,
                                                                              ChunkStat* stats) {
  // hist[b][t] (bin b of thread t's column: the lanes of an addition hit
  // distinct banks) and, after the transpose, hist as [t][kOB + 1] (a
  // thread's bins in a padded row: summing one bin over rows hits distinct
  // banks)
  __shared__ uint32_t hist[kNT * (kOB + 1)];
  __shared__ uint64_t part[kNT / kOB][kOB];
  __shared__ float redf[2 * kMaxWaves];
  const int tid = threadIdx.x;
  const float k = f.k;
  // LDS byte address of hist[b][tid] is col + (24 + b) * 4 kNT: one shift-add
  // from the exponent e = 24 + b below
  const uint32_t col = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint32_t*)&hist[tid] -
                       24u * 4u * (uint32_t)kNT;
  chunk_loop<E>(f, nch, nq, [&](const ChunkRaw<E>& raw, int q) {
    float x[kNPer];
    unpack_chunk<E>(raw, (q % nch) * kNChunk, f.V, x);
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < kNPer; ++i) tmax = fmaxf(tmax, x[i]);
    const float m = block_max(tmax, redf);  // its first barrier also ends the last chunk's reads of hist
#pragma unroll
    for (int b = 0; b < kOB; ++b) hist[b * kNT + tid] = 0u;
    const float c = m * k;
    if (c != -INFINITY) {  // uniform over the workgroup
      const uint32_t top = (uint32_t)floor_i32(c);
#pragma unroll
      for (int i = 0; i < kNPer; ++i) {
        const float w = fast_exp2(fmaf(x[i], k, -c));
        // e = 24 + the octaves below the top one, at most 24 + the tail bin
        // (-inf, octave INT_MIN, wraps to a large value and lands in the tail
        // with weight 0)
        const uint32_t e = min(top + 24u - (uint32_t)octave_of(x[i], k), (uint32_t)(24 + kOB - 1));
        const uint32_t qw = (uint32_t)__builtin_amdgcn_ldexpf(w, (int)e);
        __hip_atomic_fetch_add((__attribute__((address_space(3))) uint32_t*)(uintptr_t)(col + e * 4u * (uint32_t)kNT),
                               qw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
    __syncthreads();
    uint32_t colv[kOB];
#pragma unroll
    for (int b = 0; b < kOB; ++b) colv[b] = hist[b * kNT + tid];
    __syncthreads();
#pragma unroll
    for (int b = 0; b < kOB; ++b) hist[tid * (kOB + 1) + b] = colv[b];
    __syncthreads();
    {  // thread t sums bin t % kOB over one group of kNT / kG columns (exact)
      constexpr int kG = kNT / kOB;
      const int b = tid % kOB, g = tid / kOB;
      uint64_t sum = 0;
#pragma unroll 8
      for (int j = 0; j < kNT / kG; ++j) sum += hist[(g * (kNT / kG) + j) * (kOB + 1) + b];
      part[g][b] = sum;
    }
    __syncthreads();
    ChunkStat* st = stats + (size_t)q;
    if (tid < kOB) {
      uint64_t sum = 0;  // below 2^39: exact in fp64
#pragma unroll
      for (int g = 0; g < kNT / kOB; ++g) sum += part[g][tid];
      st->mass[tid] = __builtin_amdgcn_ldexp((double)sum, -(24 + tid));
    }
    if (tid == 0) st->c = c;
  });
}

__global__ __launch_bounds__(kWave) void nucleus_cross_kernel(FilterArgs f, int nch, ChunkStat* stats,
                                                               RowCross* rc) {
  const int lane = threadIdx.x, r = blockIdx.x;
  ChunkStat* st = stats + (size_t)r * nch;
  float cm = -INFINITY;
  for (int c = lane; c < nch; c += kWave) cm = fmaxf(cm, st[c].c);
  const float C = wave_max(cm);
  const float nan = __uint_as_float(0x7fc00000u);
  RowCross out{C, nan, 0.f, 0.f, 0.0, 0.0};
  if (C != -INFINITY) {
    const int R = floor_i32(C);
    // lane j: the row's octave R - j, from every chunk's bin j - d (d the
    // chunk's top octave below R), the chunks in order; bins past a chunk's
    // tail start are not resolved, so the crossing must lie above `limit`.
    // The chunks' offsets and scale factors are formed by the lanes in
    // parallel, kWave chunks at a time.
    double bin = 0.0, zpart = 0.0;
    int limit = kWave;
    for (int c0 = 0; c0 < nch; c0 += kWave) {
      const int cl = c0 + lane;
      const float cc = cl < nch ? st[cl].c : -INFINITY;
      const int dl = cc == -INFINITY ? kWave + kOB : R - floor_i32(cc);
      const double sl = cc == -INFINITY ? 0.0 : exp2((double)cc - (double)C);
      const int n = min(kWave, nch - c0);
      // kU chunks at a time: every record load is issued before any is used
      constexpr int kU = 16;
      for (int i0 = 0; i0 < n; i0 += kU) {
        double mb[kU], mz[kU];
        int d[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int i = i0 + u < n ? i0 + u : n - 1;  // past the end: a repeat, not added
          d[u] = __builtin_amdgcn_readlane(dl, i);
          const ChunkStat& cs = st[c0 + i];
          const int b = lane - d[u];
          mb[u] = b >= 0 && b < kOB - 1 ? cs.mass[b] : 0.0;
          mz[u] = lane < kOB ? cs.mass[lane] : 0.0;
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          if (i0 + u < n) {
            const double sc = lane_d(sl, i0 + u);
            bin += mb[u] * sc;
            zpart += mz[u] * sc;
            limit = min(limit, d[u] + kOB - 1);
          }
        }
      }
    }
    const double Z = wave_sum(zpart);
    const double target = (double)f.top_p * Z;
    const double incl = wave_inclusive_scan(bin);
    const unsigned long long reach = __ballot(incl >= target);
    if (reach) {
      const int j = __ffsll((long long)reach) - 1;
      const double above = j > 0 ? lane_d(incl, j - 1) : 0.0;
      if (j < limit) {
        out.octave = (float)(R - j);
        out.base = above;
        out.target = target;
        out.lo = first_in_octave(R - j, f.k);
        out.hi = first_in_octave(R - j + 1, f.k);
      }
    }
  }
  // every record of the row has been read: clear them
  for (int c = 0; c < nch; ++c) {
    double* w = reinterpret_cast<double*>(st + c);
    for (int i = lane; i < (int)(sizeof(ChunkStat) / sizeof(double)); i += kWave) w[i] = 0.0;
  }
  if (lane == 0) rc[r] = out;
}

template <class E>
__global__ __launch_bounds__(kNT, chunk_waves<E>()) void nucleus_list_kernel(FilterArgs f, int nch, int nq,
                                                                             const RowCross* rc, uint32_t* lcnt,
                                                                             float* lvals) {
  __shared__ float cand[kNThreadCap + 1][kNT];  // slot s of thread t at cand[s][t]; slot kNThreadCap spare
  __shared__ float redf[2 * kMaxWaves];
  const int tid = threadIdx.x;
  chunk_loop<E>(f, nch, nq, [&](const ChunkRaw<E>& raw, int q) {
    // a row left to the row kernel has the empty interval [0, 0) and lists
    // nothing
    const float lo = rc[q / nch].lo, hi = rc[q / nch].hi;
    float x[kNPer];
    unpack_chunk<E>(raw, (q % nch) * kNChunk, f.V, x);
    // branchless: every value is written to the thread's next free slot (the
    // spare slot once the column is full), and only a value in [lo, hi)
    // advances it
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < kNPer; ++i) {
      cand[min(cnt, (uint32_t)kNThreadCap)][tid] = x[i];
      cnt += (x[i] >= lo && x[i] < hi) ? 1u : 0u;
    }
    const uint32_t mine = min(cnt, (uint32_t)kNThreadCap);
    float excl, total;
    block_scan((float)mine, redf, &excl, &total);  // exact: at most kNT kNThreadCap
    const int over = __syncthreads_or(cnt > (uint32_t)kNThreadCap) || total > (float)kChunkCap;
    if (!over) {
      float* dst = lvals + (size_t)q * kChunkCap + (uint32_t)excl;
      for (uint32_t j = 0; j < mine; ++j) dst[j] = cand[j][tid];
    }
    if (tid == 0) lcnt[q] = over ? kChunkOverflow : (uint32_t)total;
  });
}

// The pick kernel's gather: the row's listed values, entry i in slot i / kLTT
// of thread i % kLTT, at most kNCap of them.
constexpr int kGatherSteps = kNCap / kLTT;

template <class E>
__global__ __launch_bounds__(kLTT) void nucleus_pick_kernel(FilterArgs f, int nch, RowCross* rc, uint32_t* lcnt,
                                                           float* lvals) {
  __shared__ ListLds L;
  const int tid = threadIdx.x, r = blockIdx.x;
  const RowCross x = rc[r];
  uint32_t* cnt = lcnt + (size_t)r * nch;
  if (tid == 0) {  // exclusive prefix of the chunk counts
    uint32_t acc = 0, ovf = 0;
    for (int c = 0; c < nch; ++c) {
      const uint32_t n = cnt[c];
      L.lpre[c] = acc;
      ovf |= n > (uint32_t)kChunkCap ? 1u : 0u;
      acc += min(n, (uint32_t)kChunkCap);
    }
    L.lpre[nch] = acc;
    L.lovf = ovf;
  }
  __syncthreads();
  const uint32_t n_all = L.lpre[nch];
  const bool ok = x.octave == x.octave && L.lovf == 0u && n_all > 0u && n_all <= (uint32_t)kNCap;
  const uint32_t n = min(n_all, (uint32_t)kNCap);
  float v[kGatherSteps];
  float* src[kGatherSteps];
  int c = 0;
#pragma unroll
  for (int j = 0; j < kGatherSteps; ++j) {  // every load first, then every use
    const uint32_t i = (uint32_t)(tid + j * kLTT);
    src[j] = nullptr;
    v[j] = 0.f;
    if (i < n) {
      while (L.lpre[c + 1] <= i) ++c;  // i grows, so the chunk only advances
      src[j] = lvals + ((size_t)r * nch + c) * kChunkCap + (i - L.lpre[c]);
      v[j] = *src[j];
    }
  }
  uint32_t my_n = 0;
#pragma unroll
  for (int j = 0; j < kGatherSteps; ++j) {
    if (src[j]) {
      *src[j] = 0.f;
      if (ok) {
        L.cand[j * kLTT + tid] = v[j];
        ++my_n;
      }
    }
  }
  // entries past the kNCap gathered ones (a row marked for listing too many):
  // cleared too
  {
    int c2 = 0;
    for (uint32_t i = (uint32_t)kNCap + tid; i < n_all; i += kLTT) {
      while (L.lpre[c2 + 1] <= i) ++c2;
      lvals[((size_t)r * nch + c2) * kChunkCap + (i - L.lpre[c2])] = 0.f;
    }
  }
  __syncthreads();  // every thread has read the row's record and counts
  if (tid < nch) cnt[tid] = 0u;
  if (tid == 0) rc[r] = RowCross{0.f, 0.f, 0.f, 0.f, 0.0, 0.0};
  if (!ok) {
    if (tid == 0) f.thr[r] = __uint_as_float(kMarkedBits);
    return;
  }
  const float C = x.C, k = f.k;
  const float tau = list_pick<E, kLTT, true>(L, L.cand, my_n, -INFINITY, x.base, x.target,
                                             [&](float w) { return fast_exp2(fmaf(w, k, -C)); }, f.top_p);
  if (tid == 0) f.thr[r] = tau;
}
}  // namespace

namespace {
// Layout of the streaming nucleus path in the filter workspace: row records,
// chunk records, row lists.
struct NucleusLayout {
  int nch;
  size_t off_stats, off_counts, off_lists, total;
};
NucleusLayout nucleus_layout(size_t rows, int V) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  NucleusLayout L{};
  L.nch = (V + kNChunk - 1) / kNChunk;
  const size_t nq = rows * (size_t)L.nch;
  L.off_stats = up(rows * sizeof(RowCross));
  L.off_counts = L.off_stats + up(nq * sizeof(ChunkStat));
  L.off_lists = L.off_counts + up(nq * sizeof(uint32_t));
  L.total = L.off_lists + up(nq * (size_t)kChunkCap * sizeof(float));
  return L;
}

}  // namespace

size_t filter_list_bytes(int B, int gamma, int V) {
  const size_t rows = (size_t)B * (2 * gamma + 1), nch = ((size_t)V + kLChunk - 1) / kLChunk;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  // the chunk lists of a small top-k and the nucleus path share the region
  return std::max(up(rows * nch * sizeof(uint32_t)) + up(rows * nch * kListCap * sizeof(float)),
                  nucleus_layout(rows, V).total);
}

hipError_t filter_thresholds(const VerifyArgs& a, int top_k, float top_p, float* thr, void* lists, hipStream_t s) {
  FilterArgs f{a.target, a.draft, a.B * (a.gamma + 1), a.V, a.k, top_k, top_p, thr, 0, nullptr, nullptr, 0};
  const int rows = a.B * (2 * a.gamma + 1);
  if (rows == 0) return hipSuccess;
  const size_t row_bytes = (size_t)a.V * (a.dtype == SPEC_BF16 ? 2 : 4);
  const bool aligned = row_bytes % 16 == 0 && (uintptr_t)a.target % 16 == 0 &&
                       (a.gamma == 0 || (uintptr_t)a.draft % 16 == 0);
  const bool topp_alone = !(top_k > 0 && top_k < a.V) && top_p < 1.f;
  // chunk lists for a small top-k (the lists region is zero on entry and is
  // left zero by the row kernel)
  // (rows of more than 256 chunks keep to the row path: the row kernel holds
  // at most 256 chunk offsets)
  if (lists != nullptr && aligned && topp_alone && (a.V + kNChunk - 1) / kNChunk <= 256) {
    // top-p alone: the streaming nucleus path (the region is zero on entry
    // and is left zero; the pick kernel holds at most 256 chunk offsets)
    const NucleusLayout NL = nucleus_layout((size_t)rows, a.V);
    char* base = static_cast<char*>(lists);
    RowCross* rc = reinterpret_cast<RowCross*>(base);
    ChunkStat* stats = reinterpret_cast<ChunkStat*>(base + NL.off_stats);
    uint32_t* lcnt = reinterpret_cast<uint32_t*>(base + NL.off_counts);
    float* lvals = reinterpret_cast<float*>(base + NL.off_lists);
    const int nq = rows * NL.nch;
    if (a.dtype == SPEC_BF16)
      nucleus_stats_kernel<BF16><<<dim3(nq), dim3(kNT), 0, s>>>(f, NL.nch, nq, stats);
    else
      nucleus_stats_kernel<F32><<<dim3(nq), dim3(kNT), 0, s>>>(f, NL.nch, nq, stats);
    nucleus_cross_kernel<<<dim3(rows), dim3(kWave), 0, s>>>(f, NL.nch, stats, rc);
    if (a.dtype == SPEC_BF16)
      nucleus_list_kernel<BF16><<<dim3(nq), dim3(kNT), 0, s>>>(f, NL.nch, nq, rc, lcnt, lvals);
    else
      nucleus_list_kernel<F32><<<dim3(nq), dim3(kNT), 0, s>>>(f, NL.nch, nq, rc, lcnt, lvals);
    if (a.dtype == SPEC_BF16)
      nucleus_pick_kernel<BF16><<<dim3(rows), dim3(kLTT), 0, s>>>(f, NL.nch, rc, lcnt, lvals);
    else
      nucleus_pick_kernel<F32><<<dim3(rows), dim3(kLTT), 0, s>>>(f, NL.nch, rc, lcnt, lvals);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the row kernel takes only the rows the nucleus path left to it
    f.marked_only = 1;
  } else if (lists != nullptr && top_k > 0 && top_k <= kListK && top_k < a.V && (a.V + kLChunk - 1) / kLChunk <= 256) {
    f.nch = (a.V + kLChunk - 1) / kLChunk;
    f.lcount = static_cast<uint32_t*>(lists);
    f.lvals = reinterpret_cast<float*>(static_cast<char*>(lists) +
                                       ((rows * (size_t)f.nch * sizeof(uint32_t) + 255) & ~(size_t)255));
    const dim3 lgrid((unsigned)(rows * f.nch)), lblock(kLT);
    if (a.dtype == SPEC_BF16) {
      if (aligned)
        chunk_list_kernel<BF16, true><<<lgrid, lblock, 0, s>>>(f);
      else
        chunk_list_kernel<BF16, false><<<lgrid, lblock, 0, s>>>(f);
    } else {
      if (aligned)
        chunk_list_kernel<F32, true><<<lgrid, lblock, 0, s>>>(f);
      else
        chunk_list_kernel<F32, false><<<lgrid, lblock, 0, s>>>(f);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.dtype == SPEC_BF16)
      list_threshold_kernel<BF16><<<dim3(rows), dim3(kLTT), 0, s>>>(f);
    else
      list_threshold_kernel<F32><<<dim3(rows), dim3(kLTT), 0, s>>>(f);
    const hipError_t e2 = hipGetLastError();
    if (e2 != hipSuccess) return e2;
    // the row kernel takes only the rows the lists left to it
    f.marked_only = 1;
    f.lcount = nullptr;
    f.lvals = nullptr;
  }
  const dim3 grid(rows), block(kFT);
  if (a.dtype == SPEC_BF16) {
    if (aligned)
      row_threshold_kernel<BF16, true><<<grid, block, 0, s>>>(f);
    else
      row_threshold_kernel<BF16, false><<<grid, block, 0, s>>>(f);
  } else {
    if (aligned)
      row_threshold_kernel<F32, true><<<grid, block, 0, s>>>(f);
    else
      row_threshold_kernel<F32, false><<<grid, block, 0, s>>>(f);
  }
  return hipGetLastError();
}

}  // namespace specv
