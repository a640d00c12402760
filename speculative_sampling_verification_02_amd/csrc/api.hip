// C ABI of the verification library: argument validation, workspace sizing and
// dispatch to the kernel paths.  The declarations and the contract of every
// entry point are in include/specverify.h.

#include <float.h>
#include <math.h>

#include <algorithm>

#include "specverify.h"
#include "verify_internal.hpp"

using specv::VerifyArgs;

namespace {

constexpr float kLog2e = 1.4426950408889634f;

bool valid_shape(int B, int gamma, int V) {
  if (B < 0 || gamma < 0 || gamma > SPEC_MAX_GAMMA || V < 1) return false;
  // every kernel indexes blocks and rows with 32-bit grid sizes
  const size_t rows = (size_t)B * (2 * (size_t)gamma + 1);
  return rows * (((size_t)V + 8191) / 8192) < (size_t)INT32_MAX;
}

bool valid_temperature(float T) {
  if (!std::isfinite(T) || T < 0.f) return false;
  if (T == 0.f) return true;
  return T >= FLT_MIN && std::isfinite(kLog2e / T);
}

int map_hip(hipError_t e) {
  if (e == hipSuccess) return SPEC_OK;
  return e == hipErrorNotSupported ? SPEC_EUNSUPPORTED : SPEC_EHIP;
}

// Both paths start their scratch at the workspace's base and both leave all
// of it zero when they complete (the fused path needs zero slots on entry).
// The top-k / top-p keep thresholds (one float per row) follow, and are
// zeroed again after the verification that reads them; then the threshold
// kernel's chunk lists, which it leaves zero.
size_t paths_bytes(int B, int gamma, int V) {
  const size_t b = std::max(specv::fused_workspace_bytes(B, gamma, V), specv::multipass_workspace_bytes(B, gamma, V));
  return (std::max<size_t>(b, 256) + 255) & ~(size_t)255;
}

size_t thr_bytes(int B, int gamma) {
  return ((size_t)B * (2 * gamma + 1) * sizeof(float) + 255) & ~(size_t)255;
}

VerifyArgs make_args(const void* target_logits, const void* draft_logits, int dtype, const int32_t* draft_tokens,
                     const float* uniforms, int B, int gamma, int V, float temperature, int32_t* n_accepted,
                     int32_t* next_token, float* alpha, float* p_draft, float* q_draft, void* workspace,
                     size_t workspace_bytes) {
  VerifyArgs a{};
  a.target = target_logits;
  a.draft = draft_logits;
  a.dtype = dtype;
  a.tokens = draft_tokens;
  a.uniforms = uniforms;
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.temperature = temperature;
  a.k = temperature > 0.f ? kLog2e / temperature : 0.f;
  a.n_out = n_accepted;
  a.t_out = next_token;
  a.alpha = gamma > 0 ? alpha : nullptr;
  a.p_draft = gamma > 0 ? p_draft : nullptr;
  a.q_draft = gamma > 0 ? q_draft : nullptr;
  a.ws = workspace;
  a.ws_bytes = workspace_bytes;
  a.lenience = 1.f;
  return a;
}

// The verification proper on the chosen path.
int launch_paths(int algo, const VerifyArgs& a, hipStream_t s) {
  if (algo == SPEC_ALGO_FUSED) return map_hip(specv::fused_launch(a, s));
  // In argmax mode (T = 0) there is no team exchange for the persistent
  // kernel to hide, and the multipass path's per-chunk argmax kernel streams
  // the rows faster: 30.4 against 36.4 us at B = 64, gamma = 4, V = 128256
  // bf16, and 345 against 407 us at B = 256, gamma = 8, V = 256000.
  if (algo == SPEC_ALGO_AUTO && a.temperature > 0.f && specv::fused_supported(a.B, a.gamma, a.V, a.dtype)) {
    // the fused path declines unaligned rows and teams that cannot be resident
    const hipError_t e = specv::fused_launch(a, s);
    if (e != hipErrorNotSupported) return map_hip(e);
  }
  return map_hip(specv::multipass_launch(a, s));
}

}  // namespace

size_t specv::verify_scratch_bytes(int B, int gamma, int V) {
  if (!valid_shape(B, gamma, V)) return 0;
  return paths_bytes(B, gamma, V);
}

int specv::verify_check(const void* target_logits, const void* draft_logits, int dtype,
                        const int32_t* draft_tokens, const float* uniforms, int B, int gamma, int V,
                        float temperature, const int32_t* n_accepted, const int32_t* next_token) {
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_EUNSUPPORTED;
  if (!valid_shape(B, gamma, V) || !valid_temperature(temperature)) return SPEC_EINVAL;
  if (B == 0) return SPEC_OK;
  if (!target_logits || !uniforms || !n_accepted || !next_token) return SPEC_EINVAL;
  if (gamma > 0 && (!draft_logits || !draft_tokens)) return SPEC_EINVAL;
  return SPEC_OK;
}

int specv::verify_in_scratch(const void* target_logits, const void* draft_logits, int dtype,
                             const int32_t* draft_tokens, const float* uniforms, int B, int gamma, int V,
                             float temperature, int32_t* n_accepted, int32_t* next_token, float* alpha,
                             float* p_draft, float* q_draft, void* scratch, size_t scratch_bytes, hipStream_t s) {
  const int st = verify_check(target_logits, draft_logits, dtype, draft_tokens, uniforms, B, gamma, V, temperature,
                              n_accepted, next_token);
  if (st != SPEC_OK || B == 0) return st;
  if (scratch_bytes < paths_bytes(B, gamma, V) || !scratch) return SPEC_ENOSPACE;
  const VerifyArgs a = make_args(target_logits, draft_logits, dtype, draft_tokens, uniforms, B, gamma, V,
                                 temperature, n_accepted, next_token, alpha, p_draft, q_draft, scratch,
                                 scratch_bytes);
  return launch_paths(SPEC_ALGO_AUTO, a, s);
}

extern "C" {

const char* spec_status_string(int status) {
  switch (status) {
    case SPEC_OK: return "ok";
    case SPEC_EINVAL: return "invalid argument";
    case SPEC_EUNSUPPORTED: return "unsupported dtype, algorithm or shape";
    case SPEC_ENOSPACE: return "workspace too small";
    case SPEC_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

size_t spec_verify_workspace_size(int B, int gamma, int V, int dtype) {
  if (!valid_shape(B, gamma, V) || (dtype != SPEC_F32 && dtype != SPEC_BF16)) return 0;
  return paths_bytes(B, gamma, V) + thr_bytes(B, gamma) + specv::filter_list_bytes(B, gamma, V);
}

size_t spec_filter_workspace_size(int B, int gamma, int V) {
  if (!valid_shape(B, gamma, V)) return 0;
  return specv::filter_list_bytes(B, gamma, V);
}

int spec_verify_ex(int algo, const void* target_logits, const void* draft_logits, int dtype,
                   const int32_t* draft_tokens, const float* uniforms, int B, int gamma, int V,
                   float temperature, int top_k, float top_p, float lenience, const int32_t* gamma_seq,
                   int32_t* n_accepted,
                   int32_t* next_token, float* alpha, float* p_draft, float* q_draft, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (algo != SPEC_ALGO_AUTO && algo != SPEC_ALGO_MULTIPASS && algo != SPEC_ALGO_FUSED)
    return SPEC_EUNSUPPORTED;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_EUNSUPPORTED;
  if (!valid_shape(B, gamma, V) || !valid_temperature(temperature)) return SPEC_EINVAL;
  if (!(lenience > 0.f && lenience <= 1.f)) return SPEC_EINVAL;  // also rejects NaN
  if (!(top_p > 0.f)) return SPEC_EINVAL;                          // also rejects NaN
  if (B == 0) return SPEC_OK;
  if (!target_logits || !uniforms || !n_accepted || !next_token) return SPEC_EINVAL;
  if (gamma > 0 && (!draft_logits || !draft_tokens)) return SPEC_EINVAL;
  if (workspace_bytes < spec_verify_workspace_size(B, gamma, V, dtype) || !workspace)
    return SPEC_ENOSPACE;

  VerifyArgs a = make_args(target_logits, draft_logits, dtype, draft_tokens, uniforms, B, gamma, V, temperature,
                           n_accepted, next_token, alpha, p_draft, q_draft, workspace, workspace_bytes);
  a.lenience = lenience;
  a.gamma_seq = gamma > 0 ? gamma_seq : nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);

  // Top-k / top-p (T > 0 only: they leave the argmax unchanged): the keep
  // thresholds first, then the verification that reads them (on either path
  // the last reader of each threshold zeroes it).
  const bool filtered = temperature > 0.f && ((top_k > 0 && top_k < V) || top_p < 1.f);
  if (filtered) {
    char* base = static_cast<char*>(workspace) + paths_bytes(B, gamma, V);
    float* thr = reinterpret_cast<float*>(base);
    const hipError_t e = specv::filter_thresholds(a, top_k, top_p, thr, base + thr_bytes(B, gamma), s);
    if (e != hipSuccess) return map_hip(e);
    a.thr = thr;
  }
  return launch_paths(algo, a, s);
}

int spec_verify_algo(int algo, const void* target_logits, const void* draft_logits, int dtype,
                     const int32_t* draft_tokens, const float* uniforms, int B, int gamma, int V,
                     float temperature, int32_t* n_accepted, int32_t* next_token, float* alpha,
                     float* p_draft, float* q_draft, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return spec_verify_ex(algo, target_logits, draft_logits, dtype, draft_tokens, uniforms, B, gamma, V,
                        temperature, 0, 1.f, 1.f, nullptr, n_accepted, next_token, alpha, p_draft, q_draft,
                        workspace, workspace_bytes, stream);
}

int spec_verify(const void* target_logits, const void* draft_logits, int dtype,
                const int32_t* draft_tokens, const float* uniforms, int B, int gamma, int V,
                float temperature, int32_t* n_accepted, int32_t* next_token, float* alpha,
                float* p_draft, float* q_draft, void* workspace, size_t workspace_bytes,
                void* stream) {
  return spec_verify_algo(SPEC_ALGO_AUTO, target_logits, draft_logits, dtype, draft_tokens, uniforms,
                          B, gamma, V, temperature, n_accepted, next_token, alpha, p_draft, q_draft,
                          workspace, workspace_bytes, stream);
}

void spec_set_wait_limit(unsigned polls) { specv::set_wait_limit(polls); }

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int spec_lmhead_logits(const void* hidden, const void* W, int M, int d, int V, float* logits,
                       void* stream) {
  if (!hidden || !W || !logits) return SPEC_EINVAL;
  if (M < 1 || M > 256 || !specv::lmhead_shape_ok(d, V)) return SPEC_EINVAL;
  if (!aligned16(hidden) || !aligned16(W) || !aligned16(logits)) return SPEC_EINVAL;
  const specv::LMHeadJob job{hidden, W, logits, M, 1, 1};
  return map_hip(specv::lmhead_launch(&job, 1, d, V, static_cast<hipStream_t>(stream)));
}

int spec_filter_thresholds(const void* target_logits, const void* draft_logits, int dtype, int B, int gamma,
                           int V, float temperature, int top_k, float top_p, float* thresholds, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_EUNSUPPORTED;
  if (!valid_shape(B, gamma, V) || !valid_temperature(temperature) || !(temperature > 0.f)) return SPEC_EINVAL;
  if (!(top_p > 0.f)) return SPEC_EINVAL;  // also rejects NaN
  if (B == 0) return SPEC_OK;
  if (!target_logits || !thresholds || (gamma > 0 && !draft_logits)) return SPEC_EINVAL;
  if (workspace && workspace_bytes < spec_filter_workspace_size(B, gamma, V)) return SPEC_ENOSPACE;
  VerifyArgs a{};
  a.target = target_logits;
  a.draft = draft_logits;
  a.dtype = dtype;
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.temperature = temperature;
  a.k = kLog2e / temperature;
  return map_hip(specv::filter_thresholds(a, top_k, top_p, thresholds, workspace, static_cast<hipStream_t>(stream)));
}

size_t spec_lmhead_workspace_size(int B, int gamma, int d, int V) {
  if (!specv::lmhead_shape_ok(d, V)) return 0;
  return spec_verify_workspace_size(B, gamma, V, SPEC_F32);
}

int spec_lmhead_verify(const void* hidden, const void* hidden_draft, const void* W_target,
                       const void* W_draft, int B, int gamma, int d, int V,
                       const int32_t* draft_tokens, const float* uniforms, float temperature,
                       float* target_logits, float* draft_logits, int32_t* n_accepted,
                       int32_t* next_token, float* alpha, float* p_draft, float* q_draft,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_shape(B, gamma, V) || !valid_temperature(temperature)) return SPEC_EINVAL;
  if (B == 0) return SPEC_OK;
  const int M = B * (gamma + 1);
  if (M > 256 || !specv::lmhead_shape_ok(d, V)) return SPEC_EINVAL;
  if (!hidden || !W_target || !target_logits || (gamma > 0 && (!W_draft || !draft_logits)))
    return SPEC_EINVAL;
  if (!aligned16(hidden) || !aligned16(W_target) || !aligned16(target_logits) ||
      (gamma > 0 && (!aligned16(W_draft) || !aligned16(draft_logits) ||
                     (hidden_draft && !aligned16(hidden_draft)))))
    return SPEC_EINVAL;
  if (workspace_bytes < spec_lmhead_workspace_size(B, gamma, d, V) || !workspace) return SPEC_ENOSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Both heads in one launch.  Draft rows are either a dense [B*gamma][d]
  // tensor, or rows 0..gamma-1 of each sequence's gamma+1 block of `hidden`.
  specv::LMHeadJob jobs[2] = {{hidden, W_target, target_logits, M, 1, 1}, {}};
  int njobs = 1;
  if (gamma > 0) {
    jobs[1] = hidden_draft ? specv::LMHeadJob{hidden_draft, W_draft, draft_logits, B * gamma, 1, 1}
                           : specv::LMHeadJob{hidden, W_draft, draft_logits, B * gamma, gamma + 1, gamma};
    njobs = 2;
  }
  const hipError_t e = specv::lmhead_launch(jobs, njobs, d, V, s);
  if (e != hipSuccess) return map_hip(e);
  return spec_verify(target_logits, draft_logits, SPEC_F32, draft_tokens, uniforms, B, gamma, V,
                     temperature, n_accepted, next_token, alpha, p_draft, q_draft, workspace,
                     workspace_bytes, stream);
}

}  // extern "C"
