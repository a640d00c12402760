// LM-head skinny GEMM for gfx950: logits[m][v] = sum_k hidden[m][k] * W[k][v]
// with bf16 inputs, fp32 accumulation and fp32 output, for the few rows a
// verification step needs (B * (gamma + 1) target positions, B * gamma draft
// positions).
//
// During decoding the product reads every weight once and uses it once, so it
// is bound by HBM, not by arithmetic ([FI] "Decoding waits on memory, not
// arithmetic").  The design follows from that: W streams through once, in
// 16-byte loads, and everything else stays on chip.
//
// Work split.  One wave owns a slab of 128 vocabulary columns and walks the
// whole hidden dimension in steps of 32.  A workgroup is 4 waves on 4
// adjacent slabs, so one workgroup reads 1 KiB contiguous of each W row.  The
// two heads of a verification step (target and draft) run in one launch:
// blockIdx.y selects the head.
//
// Per step a lane loads 8 rows x 8 columns of W (rows k0 + 8g .. +7, columns
// v0 + 8c .. +7, with g = lane / 16 and c = lane % 16), which is the natural
// coalesced order: lanes 0..15 cover 256 contiguous bytes of one row.  The
// matrix cores want each lane's operand as 8 consecutive k of ONE column, so
// the lane transposes its 8x8 block in registers with byte permutes (one
// v_perm_b32 per output dword), giving 8 operands: column v0 + 8c + j for
// j = 0..7.  Each is the B operand (32 k x 16 columns, column c of the tile)
// of one v_mfma_f32_16x16x32_bf16 whose A operand is a 16-row tile of hidden
// (16 rows x 32 k, lane holds row c, k = 8g .. 8g + 7, read from L2 as one
// 16-byte load).  Lane (g, c) ends with D rows 4g .. 4g + 3 of column c in
// each of the 8 tiles: for one row, that is 8 consecutive columns, written as
// two 16-byte stores.
//
// The next step's W loads are issued before the current step's matrix work,
// so each wave keeps 16 KiB of W in flight.

#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.hpp"
#include "specverify.h"
#include "verify_internal.hpp"

namespace specv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kSlab = 128;          // columns per wave
constexpr int kWaves = 4;           // waves per workgroup
constexpr int kKStep = 32;          // hidden dimension per matrix-core step
constexpr int kMaxTiles = 4;        // 16-row tiles per pass: up to 64 rows

struct HeadArgs {
  const uint16_t* hidden;  // bf16 bits [rows][d]
  const uint16_t* W;       // bf16 bits [d][V]
  float* out;              // [M][V]
  int M;                   // output rows of this head
  int group_in, group_out; // output row m reads hidden row (m / group_out) * group_in + m % group_out
  int row0;                // first output row of this pass
};

struct LMHeadParams {
  HeadArgs head[2];
  int d, V;
};

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Operand j (column v0 + 8c + j) from the 8 loaded row segments: dword t holds
// rows 2t (low half) and 2t + 1 (high half) of that column.
template <int J>
__device__ inline u32x4 column_operand(const u32x4 (&r)[8]) {
  constexpr uint32_t sel = (J & 1) ? 0x07060302u : 0x05040100u;
  u32x4 o;
  o.x = __builtin_amdgcn_perm(r[1][J >> 1], r[0][J >> 1], sel);
  o.y = __builtin_amdgcn_perm(r[3][J >> 1], r[2][J >> 1], sel);
  o.z = __builtin_amdgcn_perm(r[5][J >> 1], r[4][J >> 1], sel);
  o.w = __builtin_amdgcn_perm(r[7][J >> 1], r[6][J >> 1], sel);
  return o;
}

template <int MT>
__device__ inline void step_mfma(const u32x4 (&r)[8], const u32x4 (&a)[MT], f32x4 (&acc)[MT][8]) {
#define SPECV_LMHEAD_COL(J)                                                           \
  {                                                                                   \
    const bf16x8 bj = as_bf16x8(column_operand<J>(r));                                \
    _Pragma("unroll") for (int t = 0; t < MT; ++t)                                    \
      acc[t][J] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[t]), bj, acc[t][J], 0, 0, 0); \
  }
  SPECV_LMHEAD_COL(0)
  SPECV_LMHEAD_COL(1)
  SPECV_LMHEAD_COL(2)
  SPECV_LMHEAD_COL(3)
  SPECV_LMHEAD_COL(4)
  SPECV_LMHEAD_COL(5)
  SPECV_LMHEAD_COL(6)
  SPECV_LMHEAD_COL(7)
#undef SPECV_LMHEAD_COL
}

template <int MT>
__global__ __launch_bounds__(kWaves * kWave) void lmhead_kernel(LMHeadParams P) {
  const HeadArgs& h = P.head[blockIdx.y];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int g = lane >> 4, c = lane & 15;
  const int v0 = (blockIdx.x * kWaves + wave) * kSlab + 8 * c;  // this lane's 8 columns
  const int d = P.d, V = P.V;
  const bool live = v0 < V;  // V is a multiple of 8: all 8 columns or none

  // hidden rows of this lane's A operands (row c of each 16-row tile)
  const uint16_t* arow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = h.row0 + 16 * t + c;
    arow[t] = m < h.M ? h.hidden + (size_t)((m / h.group_out) * h.group_in + m % h.group_out) * d + 8 * g
                      : nullptr;
  }
  const uint16_t* wcol = h.W + (size_t)(8 * g) * V + (live ? v0 : 0);

  f32x4 acc[MT][8];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load_w = [&](int k0, u32x4 (&r)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      r[i] = live ? load_stream(wcol + (size_t)(k0 + i) * V) : u32x4{0u, 0u, 0u, 0u};
  };
  auto load_a = [&](int k0, u32x4 (&a)[MT]) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
      a[t] = arow[t] ? load_cached(arow[t] + k0) : u32x4{0u, 0u, 0u, 0u};
  };

  // two register stages: the loads of step s + 1 are in flight during step s
  u32x4 r0[8], r1[8], a0[MT], a1[MT];
  load_w(0, r0);
  load_a(0, a0);
  int k0 = 0;
  while (true) {
    const bool more1 = k0 + kKStep < d;
    if (more1) {
      load_w(k0 + kKStep, r1);
      load_a(k0 + kKStep, a1);
    }
    step_mfma<MT>(r0, a0, acc);
    if (!more1) break;
    k0 += kKStep;
    const bool more0 = k0 + kKStep < d;
    if (more0) {
      load_w(k0 + kKStep, r0);
      load_a(k0 + kKStep, a0);
    }
    step_mfma<MT>(r1, a1, acc);
    if (!more0) break;
    k0 += kKStep;
  }

  if (!live) return;
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = h.row0 + 16 * t + 4 * g + i;
      if (m < h.M) {
        float* o = h.out + (size_t)m * V + v0;
        *reinterpret_cast<float4*>(o) = make_float4(acc[t][0][i], acc[t][1][i], acc[t][2][i], acc[t][3][i]);
        *reinterpret_cast<float4*>(o + 4) = make_float4(acc[t][4][i], acc[t][5][i], acc[t][6][i], acc[t][7][i]);
      }
    }
}

template <int MT>
void launch_tiles(const LMHeadParams& P, int nheads, hipStream_t s) {
  const int cols_per_block = kWaves * kSlab;
  const dim3 grid((P.V + cols_per_block - 1) / cols_per_block, nheads);
  lmhead_kernel<MT><<<grid, dim3(kWaves * kWave), 0, s>>>(P);
}

}  // namespace

bool lmhead_shape_ok(int d, int V) { return d >= kKStep && d % kKStep == 0 && V >= 8 && V % 8 == 0; }

hipError_t lmhead_launch(const LMHeadJob* jobs, int njobs, int d, int V, hipStream_t s) {
  if (njobs < 1 || njobs > 2 || !lmhead_shape_ok(d, V)) return hipErrorInvalidValue;
  int maxM = 0;
  for (int j = 0; j < njobs; ++j) maxM = std::max(maxM, jobs[j].M);
  // one pass covers 64 output rows of every head; more rows take more passes
  // over W
  for (int row0 = 0; row0 < maxM; row0 += 16 * kMaxTiles) {
    LMHeadParams P{};
    P.d = d;
    P.V = V;
    int rows = 0;
    for (int j = 0; j < njobs; ++j) {
      HeadArgs& h = P.head[j];
      h.hidden = static_cast<const uint16_t*>(jobs[j].hidden);
      h.W = static_cast<const uint16_t*>(jobs[j].W);
      h.out = jobs[j].out;
      h.M = jobs[j].M;
      h.group_in = jobs[j].group_in;
      h.group_out = jobs[j].group_out;
      h.row0 = row0;
      rows = std::max(rows, std::min(jobs[j].M - row0, 16 * kMaxTiles));
    }
    const int tiles = (rows + 15) / 16;
    switch (tiles) {
      case 1: launch_tiles<1>(P, njobs, s); break;
      case 2: launch_tiles<2>(P, njobs, s); break;
      case 3: launch_tiles<3>(P, njobs, s); break;
      default: launch_tiles<4>(P, njobs, s); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace specv
