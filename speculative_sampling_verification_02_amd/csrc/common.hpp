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
  // The empty asm pins each value to a register: without it a run of these
  // copies is merged into one memcpy out of the raw buffer, which then has to
  // live in scratch memory instead of registers.
  __device__ static inline void unpack(const u32x4& v, float* out) {
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      asm("" : "+v"(w[k]));
      out[k] = __uint_as_float(w[k]);
    }
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

// Ordinary cached 16-byte load (for data read again shortly after).
__device__ inline u32x4 load_cached(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------- cross-workgroup words
//
// Naturally aligned 64-bit relaxed agent-scope atomic stores and loads: single-
// copy atomic and, on gfx950, device-coherent across XCDs (the SC1 scope bit),
// with no cache writeback or invalidate.  A reader polls a word until it is
// published (nonzero low half) and the poll returns the data itself.

__device__ inline void st_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint64_t ld_u64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------ wave reductions
//
// All-reduce across a wave64 with DPP lane moves inside each 16-lane row
// (xor 1, xor 2, half-row mirror, row mirror), after which every lane of row j
// holds the row's result r_j; then two row broadcasts (lane 15 of rows 0 and 2
// into rows 1 and 3, lane 31 into rows 2 and 3) leave (r3 . r2) . (r1 . r0) in
// lane 63, which readlane returns to every lane.  Every step combines two
// values with a commutative operation, so the result equals
// (r0 . r1) . (r2 . r3) bit for bit and the order of operations is fixed:
// results are reproducible run to run.

constexpr int kDppXor1 = 0xB1;         // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i within each 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i within each 16 lanes
constexpr int kDppBcast15 = 0x142;     // lane 15 of each row to all of the next row
constexpr int kDppBcast31 = 0x143;     // lane 31 to all of rows 2 and 3

template <int CTRL>
__device__ inline int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}
template <int CTRL>
__device__ inline double dpp_d(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = dpp_i<CTRL>((int)(b & 0xffffffffll)), hi = dpp_i<CTRL>((int)(b >> 32));
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}
__device__ inline float lane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ inline double lane_d(double v, int lane) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffffll), lane);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), lane);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// A row broadcast into the rows of ROWS; the other rows read `old`.
template <int CTRL, int ROWS>
__device__ inline float bcast_f(float old, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROWS, 0xF, false));
}
template <int CTRL, int ROWS>
__device__ inline double bcast_d(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(b & 0xffffffffll), CTRL, ROWS, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, ROWS, 0xF, false);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

__device__ inline float wave_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  v = fmaxf(v, bcast_f<kDppBcast15, 0xA>(v, v));
  v = fmaxf(v, bcast_f<kDppBcast31, 0xC>(v, v));
  return lane_f(v, kWave - 1);
}

__device__ inline float wave_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  v += bcast_f<kDppBcast15, 0xA>(0.f, v);  // rows 0 and 2 add 0 (lane 63 never reads them again)
  v += bcast_f<kDppBcast31, 0xC>(0.f, v);
  return lane_f(v, kWave - 1);
}

__device__ inline double wave_sum(double v) {
  v += dpp_d<kDppXor1>(v);
  v += dpp_d<kDppXor2>(v);
  v += dpp_d<kDppHalfMirror>(v);
  v += dpp_d<kDppMirror>(v);
  v += bcast_d<kDppBcast15, 0xA>(v);
  v += bcast_d<kDppBcast31, 0xC>(v);
  return lane_d(v, kWave - 1);
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

// Argmax of a thread's N values visited in increasing token order (token(t)
// increasing in t): the maximum by a tree of three-input maxima, then the
// first value equal to it, found backwards.  About two instructions per value
// instead of a compare-and-select of the (value, index) pair for each.  Equal
// values include -0 and +0 and, for a thread of -inf only, every value: the
// lowest index wins, as argmax_better would choose.
template <int N, class TokenFn>
__device__ inline ArgMax thread_argmax_first(const float (&x)[N], TokenFn token) {
  static_assert(N % 2 == 0, "pairs of values");
  float m0 = x[0], m1 = x[1];
#pragma unroll
  for (int t = 2; t + 3 < N; t += 4) {
    m0 = __builtin_fmaxf(m0, __builtin_fmaxf(x[t], x[t + 1]));
    m1 = __builtin_fmaxf(m1, __builtin_fmaxf(x[t + 2], x[t + 3]));
  }
  if constexpr (N % 4 == 0) m0 = __builtin_fmaxf(m0, __builtin_fmaxf(x[N - 2], x[N - 1]));
  const float m = __builtin_fmaxf(m0, m1);
  int first = 0;  // (some value equals m, so the last assignment is to the first of them)
#pragma unroll
  for (int t = N - 1; t >= 0; --t) first = x[t] == m ? t : first;
  return ArgMax{m, token(first)};
}

template <int CTRL>
__device__ inline ArgMax dpp_argmax(ArgMax a) {
  return argmax_better(a, ArgMax{dpp_f<CTRL>(a.v), dpp_i<CTRL>(a.i)});
}

__device__ inline ArgMax wave_argmax(ArgMax a) {
  a = dpp_argmax<kDppXor1>(a);
  a = dpp_argmax<kDppXor2>(a);
  a = dpp_argmax<kDppHalfMirror>(a);
  a = dpp_argmax<kDppMirror>(a);
  ArgMax r{lane_f(a.v, 0), __builtin_amdgcn_readlane(a.i, 0)};
  r = argmax_better(r, ArgMax{lane_f(a.v, 16), __builtin_amdgcn_readlane(a.i, 16)});
  r = argmax_better(r, ArgMax{lane_f(a.v, 32), __builtin_amdgcn_readlane(a.i, 32)});
  r = argmax_better(r, ArgMax{lane_f(a.v, 48), __builtin_amdgcn_readlane(a.i, 48)});
  return r;
}

// Inclusive scan across the wave in lane order: Kogge-Stone with DPP row
// shifts inside each 16-lane row (lanes shifted in from outside the row read
// 0), then the totals of the earlier rows, read with readlane, added in row
// order.
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;

template <int CTRL>
__device__ inline float dpp_shr_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ inline double dpp_shr_d(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(b & 0xffffffffll), CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, 0xF, 0xF, true);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

__device__ inline float wave_inclusive_scan(float v) {
  const int lane = threadIdx.x & (kWave - 1);
  v += dpp_shr_f<kDppShr1>(v);
  v += dpp_shr_f<kDppShr2>(v);
  v += dpp_shr_f<kDppShr4>(v);
  v += dpp_shr_f<kDppShr8>(v);
  const float t0 = lane_f(v, 15), t1 = lane_f(v, 31), t2 = lane_f(v, 47);
  const float before = lane < 16 ? 0.f : lane < 32 ? t0 : lane < 48 ? t0 + t1 : (t0 + t1) + t2;
  return lane < 16 ? v : before + v;
}

__device__ inline double wave_inclusive_scan(double v) {
  const int lane = threadIdx.x & (kWave - 1);
  v += dpp_shr_d<kDppShr1>(v);
  v += dpp_shr_d<kDppShr2>(v);
  v += dpp_shr_d<kDppShr4>(v);
  v += dpp_shr_d<kDppShr8>(v);
  const double t0 = lane_d(v, 15), t1 = lane_d(v, 31), t2 = lane_d(v, 47);
  const double before = lane < 16 ? 0.0 : lane < 32 ? t0 : lane < 48 ? t0 + t1 : (t0 + t1) + t2;
  return lane < 16 ? v : before + v;
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

// Two independent reductions sharing one pair of barriers.  `lds` must hold
// 2 * kMaxWaves entries.
__device__ inline float2 block_max2(float a, float b, float* lds) {
  const int wid = threadIdx.x / kWave, nw = blockDim.x / kWave;
  a = wave_max(a);
  b = wave_max(b);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) {
    lds[wid] = a;
    lds[kMaxWaves + wid] = b;
  }
  __syncthreads();
  float ra = lds[0], rb = lds[kMaxWaves];
  for (int w = 1; w < nw; ++w) {
    ra = fmaxf(ra, lds[w]);
    rb = fmaxf(rb, lds[kMaxWaves + w]);
  }
  return make_float2(ra, rb);
}

__device__ inline float2 block_sum2(float a, float b, float* lds) {
  const int wid = threadIdx.x / kWave, nw = blockDim.x / kWave;
  a = wave_sum(a);
  b = wave_sum(b);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) {
    lds[wid] = a;
    lds[kMaxWaves + wid] = b;
  }
  __syncthreads();
  float ra = lds[0], rb = lds[kMaxWaves];
  for (int w = 1; w < nw; ++w) {
    ra += lds[w];
    rb += lds[kMaxWaves + w];
  }
  return make_float2(ra, rb);
}

__device__ inline double block_sum(double v, double* lds) {
  const int wid = threadIdx.x / kWave, nw = blockDim.x / kWave;
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) lds[wid] = v;
  __syncthreads();
  double r = lds[0];
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
  // previous lane's inclusive value (DPP wave_shr:1; lane 0 reads 0)
  float prev = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(inc), 0x138, 0xF, 0xF, true));
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

// ------------------------------------------------------ inverse-CDF search

// Inverse-CDF search over a token range: the first token j in [lo, hi) whose
// running weight (from 0 at lo) exceeds theta.  `weight(j, x)` gives the
// weight of token j with logit x in row `r0` (and `x1` from row `r1` for the
// residual).  If rounding leaves the whole chunk at or below theta, the last
// token with positive weight is returned.  Called by the whole workgroup.
template <class E, bool VEC, int kThreads, class W>
__device__ int range_search(const typename E::storage* r0, const typename E::storage* r1, int lo,
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
        E::unpack(load_cached(r0 + j0), x0);
        if (r1) E::unpack(load_cached(r1 + j0), x1);
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
  // (callers keep hi - lo below 2^24, so offsets compare exactly as floats)
  ArgMax lp{last_pos >= 0 ? (float)(last_pos - lo) : -1.f, last_pos};
  lp = block_argmax(lp, lds_f, lds_i);
  return lp.i;
}

// Inverse-CDF search over one tile of kThreads * PER tokens starting at
// tile_lo (16-byte aligned rows, V a multiple of kVec).  Thread t owns the PER
// consecutive tokens from tile_lo + t * PER.  All loads are issued before the
// scan, and one workgroup scan over the thread sums locates the owner of
// theta, so the search costs one memory round trip and one scan.  Returns the
// first token whose running weight (from 0 at tile_lo, in token order)
// exceeds theta.  If rounding leaves the whole tile at or below theta, the last
// token with positive weight is returned.  Called by the whole workgroup
// (blockDim.x == kThreads).
template <class E, int PER, int kThreads, class W>
__device__ int tile_search(const typename E::storage* r0, const typename E::storage* r1, int tile_lo, int V,
                           float theta, W&& weight, float* lds_f, int* lds_i) {
  constexpr int NS = PER / E::kVec;
  __shared__ int found;
  const int base = tile_lo + (int)threadIdx.x * PER;
  u32x4 raw0[NS], raw1[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int j0 = base + s * E::kVec;
    raw0[s] = j0 < V ? load_cached(r0 + j0) : u32x4{0u, 0u, 0u, 0u};
    raw1[s] = (r1 && j0 < V) ? load_cached(r1 + j0) : u32x4{0u, 0u, 0u, 0u};
  }
  if (threadIdx.x == 0) found = -1;
  float w[PER];
  float sum = 0.f;
  int last_pos = -1;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int j0 = base + s * E::kVec;
    float x0[E::kVec], x1[E::kVec];
    E::unpack(raw0[s], x0);
    E::unpack(raw1[s], x1);
#pragma unroll
    for (int v = 0; v < E::kVec; ++v) {
      const float wv = j0 < V ? weight(x0[v], x1[v]) : 0.f;
      w[s * E::kVec + v] = wv;
      if (wv > 0.f) last_pos = j0 + v;
      sum += wv;
    }
  }
  float excl, total;
  const float incl = block_scan(sum, lds_f, &excl, &total);
  if (excl <= theta && theta < incl) {  // exactly one thread owns theta
    float run = excl;
    int pick = -1, lastp = -1;
#pragma unroll
    for (int v = 0; v < PER; ++v) {
      if (w[v] > 0.f) lastp = base + v;
      run += w[v];
      if (pick < 0 && run > theta) pick = base + v;
    }
    found = pick >= 0 ? pick : lastp;
  }
  __syncthreads();
  const int f = found;
  __syncthreads();
  if (f >= 0) return f;
  // rounding guard: the last positive-weight token of the tile (offsets inside
  // the tile are small, so they compare exactly as floats)
  ArgMax lp{last_pos >= 0 ? (float)(last_pos - tile_lo) : -1.f, last_pos};
  lp = block_argmax(lp, lds_f, lds_i);
  return lp.i;
}

// Inverse-CDF draw over a whole row [0, V) from per-token weights: their total
// first (fp32 per thread, fp64 across the workgroup), then the first token
// whose running weight exceeds u * total (range_search).  Returns -1 when no
// token of the row has positive weight.  A fall-back for a search whose chunk
// or tile turned out to hold no positive weight; called by the whole
// workgroup.  VEC needs 16-byte aligned rows and V a multiple of kVec.
template <class E, bool VEC, int kThreads, class W>
__device__ int row_search(const typename E::storage* r0, const typename E::storage* r1, int V, double u,
                          W&& weight, float* lds_f, int* lds_i, double* lds_d) {
  constexpr int kPer = VEC ? E::kVec : 1;
  float s = 0.f;
  for (int j0 = (int)threadIdx.x * kPer; j0 < V; j0 += kThreads * kPer) {
    float x0[kPer], x1[kPer];
    if constexpr (VEC) {
      E::unpack(load_cached(r0 + j0), x0);
      if (r1) E::unpack(load_cached(r1 + j0), x1);
    } else {
      x0[0] = E::at(r0, j0);
      if (r1) x1[0] = E::at(r1, j0);
    }
#pragma unroll
    for (int t = 0; t < kPer; ++t) s += weight(x0[t], r1 ? x1[t] : 0.f);
  }
  const double total = block_sum((double)s, lds_d);
  if (!(total > 0.0)) return -1;
  return range_search<E, VEC, kThreads>(r0, r1, 0, V, (float)(u * total), weight, lds_f, lds_i);
}

// Bytes [o, o + 16) of the 32 bytes a || b (o < 16, the same in every lane
// of the workgroup): each output word is one v_alignbyte of two input words.
__device__ inline u32x4 cut_vector(const u32x4& a, const u32x4& b, int o) {
  const uint32_t c[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  const uint32_t r = (uint32_t)o & 3u;
  auto w = [&](int k) { return __builtin_amdgcn_alignbyte(c[k + 1], c[k], r); };
  switch (o >> 2) {
    case 0: return u32x4{w(0), w(1), w(2), w(3)};
    case 1: return u32x4{w(1), w(2), w(3), w(4)};
    case 2: return u32x4{w(2), w(3), w(4), w(5)};
    default: return u32x4{w(3), w(4), w(5), w(6)};
  }
}

// Tokens [j0, j0 + kVec) of a row that need not start on 16 bytes (its tensor
// does), as floats; tokens at or past V read as -inf.  Cut from the two
// aligned vectors that cover them when both lie in the row, else token by token.
template <class E>
__device__ inline void shifted_vector(const typename E::storage* row, int j0, int V, float* out) {
  const int sh = (int)(((uintptr_t)row & 15u) / sizeof(typename E::storage));
  if (j0 + 2 * E::kVec - sh <= V) {
    const auto* ra = row - sh;
    E::unpack(cut_vector(load_cached(ra + j0), load_cached(ra + j0 + E::kVec), sh * (int)sizeof(typename E::storage)),
              out);
  } else {
#pragma unroll
    for (int v = 0; v < E::kVec; ++v) out[v] = j0 + v < V ? E::at(row, j0 + v) : -INFINITY;
  }
}

// tile_search (inverse-CDF draw over one tile of kThreads * PER tokens, one
// memory round trip and one workgroup scan) for rows that need not start on
// 16 bytes: thread t owns the PER tokens from tile_lo + t * PER, each vector
// from shifted_vector.  Tokens at or past V have weight 0.  Returns the first
// token whose running weight exceeds theta, or the tile's last positive-weight
// token if rounding leaves the whole tile at or below theta, or -1 if no
// token has positive weight.  Called by the whole workgroup.
template <class E, int PER, class W>
__device__ int shifted_tile_search(const typename E::storage* r0, const typename E::storage* r1, int tile_lo, int V,
                                   float theta, W&& weight, float* lds_f, int* lds_i) {
  constexpr int NS = PER / E::kVec;
  __shared__ int found;
  const int base = tile_lo + (int)threadIdx.x * PER;
  float x0[PER], x1[PER];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    shifted_vector<E>(r0, base + s * E::kVec, V, x0 + s * E::kVec);
    if (r1) shifted_vector<E>(r1, base + s * E::kVec, V, x1 + s * E::kVec);
  }
  if (threadIdx.x == 0) found = -1;
  float w[PER];
  float sum = 0.f;
  int last_pos = -1;
#pragma unroll
  for (int t = 0; t < PER; ++t) {
    const float wv = base + t < V ? weight(x0[t], r1 ? x1[t] : 0.f) : 0.f;
    w[t] = wv;
    if (wv > 0.f) last_pos = base + t;
    sum += wv;
  }
  float excl, total;
  const float incl = block_scan(sum, lds_f, &excl, &total);
  if (excl <= theta && theta < incl) {  // exactly one thread owns theta
    float run = excl;
    int pick = -1, lastp = -1;
#pragma unroll
    for (int t = 0; t < PER; ++t) {
      if (w[t] > 0.f) lastp = base + t;
      run += w[t];
      if (pick < 0 && run > theta) pick = base + t;
    }
    found = pick >= 0 ? pick : lastp;
  }
  __syncthreads();
  const int f = found;
  __syncthreads();
  if (f >= 0) return f;
  ArgMax lp{last_pos >= 0 ? (float)(last_pos - tile_lo) : -1.f, last_pos};
  lp = block_argmax(lp, lds_f, lds_i);
  return lp.i;
}

// Row normaliser from nch chunk partials (max m_c, sum S_c relative to m_c),
// computed by one wave in a fixed order: M = max m_c and
// S = sum_c S_c exp2((m_c - M) k) accumulated in fp64.  Call from all 64
// lanes of one wave; every lane gets the result.
struct WaveNorm {
  float M;
  double S;
};

__device__ inline WaveNorm wave_row_norm(const float2* st, int nch, float k) {
  const int lane = threadIdx.x & (kWave - 1);
  float M = -INFINITY;
  for (int c = lane; c < nch; c += kWave) M = fmaxf(M, st[c].x);
  M = wave_max(M);
  double S = 0.0;
  for (int c = lane; c < nch; c += kWave) {
    const float2 v = st[c];
    if (v.x != -INFINITY) S += (double)v.y * (double)fast_exp2((v.x - M) * k);
  }
  return WaveNorm{M, wave_sum(S)};
}

}  // namespace specv
