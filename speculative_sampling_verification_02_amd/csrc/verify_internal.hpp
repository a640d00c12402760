// Internal interface between the C ABI layer and the verification kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace specv {

// Everything one verification call needs, validated by the ABI layer.
struct VerifyArgs {
  const void* target;      // [B][gamma+1][V]
  const void* draft;       // [B][gamma][V]
  int dtype;               // SPEC_F32 / SPEC_BF16
  const int32_t* tokens;   // [B][gamma]
  const float* uniforms;   // [B][gamma+1]
  int B, gamma, V;
  float temperature;       // 0 = argmax mode
  float k;                 // log2(e) / T in fp32 (unused in argmax mode)
  int32_t* n_out;
  int32_t* t_out;
  float* alpha;            // may be null
  float* p_draft;          // may be null
  float* q_draft;          // may be null
  void* ws;
  size_t ws_bytes;
  float lenience;              // l in (0, 1]; 1 = exact speculative sampling
  const int32_t* gamma_seq;    // [B] per-sequence draft counts, or null (all gamma)
  float* thr;                  // top-k / top-p keep thresholds per row, or null:
                               // [B(gamma+1)] target rows, then [B gamma] draft rows;
                               // each is zeroed by its last reader in the fused kernel
};

// A logit below its row's keep threshold counts as -inf (probability 0).
__device__ inline float thr_target(const VerifyArgs& a, int b, int i) {
  return a.thr[(size_t)b * (a.gamma + 1) + i];
}
__device__ inline float thr_draft(const VerifyArgs& a, int b, int i) {
  return a.thr[(size_t)a.B * (a.gamma + 1) + (size_t)b * a.gamma + i];
}

// Draft count of sequence b: gamma_seq[b] clamped into [0, gamma], or gamma.
__device__ inline int seq_gamma(const VerifyArgs& a, int b) {
  if (!a.gamma_seq) return a.gamma;
  const int g = a.gamma_seq[b];
  return g < 0 ? 0 : (g > a.gamma ? a.gamma : g);
}

// ---- scratch of a verification without top-k / top-p (both paths): the
// bytes a workspace needs for it, 0 for an invalid shape
size_t verify_scratch_bytes(int B, int gamma, int V);
// The host-side argument checks of spec_verify (SPEC_OK or its status code)
int verify_check(const void* target_logits, const void* draft_logits, int dtype, const int32_t* draft_tokens,
                 const float* uniforms, int B, int gamma, int V, float temperature, const int32_t* n_accepted,
                 const int32_t* next_token);
// spec_verify on a zeroed scratch of at least verify_scratch_bytes(), with
// the argument checks of spec_verify (its status codes)
int verify_in_scratch(const void* target_logits, const void* draft_logits, int dtype, const int32_t* draft_tokens,
                      const float* uniforms, int B, int gamma, int V, float temperature, int32_t* n_accepted,
                      int32_t* next_token, float* alpha, float* p_draft, float* q_draft, void* scratch,
                      size_t scratch_bytes, hipStream_t stream);

// ---- multi-pass path
size_t multipass_workspace_bytes(int B, int gamma, int V);
hipError_t multipass_launch(const VerifyArgs& a, hipStream_t stream);

// ---- fused read-once path
// Exchange slots of the fused path: all zero before a call, and all zero again
// after a call that completes.  A multiple of 256 bytes.
size_t fused_workspace_bytes(int B, int gamma, int V);
// Returns hipErrorNotSupported when the shape does not fit the fused design.
hipError_t fused_launch(const VerifyArgs& a, hipStream_t stream);
bool fused_supported(int B, int gamma, int V, int dtype);
// Bound (polls) of every cross-workgroup wait of later launches (the fused
// path; the multipass path's argmax finishing); 0 restores the default.
void set_wait_limit(unsigned polls);
unsigned wait_limit();

// ---- top-k / top-p keep thresholds (filter.hip): one float per row into thr,
// and a fill kernel that zeroes them again after the verification
// Workspace of the chunk candidate lists for a top-k of at most 64 (zero on
// entry, left zero).
size_t filter_list_bytes(int B, int gamma, int V);
hipError_t filter_thresholds(const VerifyArgs& a, int top_k, float top_p, float* thr, void* lists,
                             hipStream_t stream);

// ---- LM head
// One head of the product: out[m][v] = sum_k hidden[r(m)][k] W[k][v] for
// m < M, with hidden row r(m) = (m / group_out) * group_in + m % group_out
// (group_in = group_out = 1 reads the rows in order).
struct LMHeadJob {
  const void* hidden;  // bf16 [rows][d], 16-byte aligned
  const void* W;       // bf16 [d][V], 16-byte aligned
  float* out;          // [M][V], 16-byte aligned
  int M, group_in, group_out;
};
// d a multiple of 32, V a multiple of 8.
bool lmhead_shape_ok(int d, int V);
// One launch per 64 output rows computes one or two heads (sharing d and V).
hipError_t lmhead_launch(const LMHeadJob* jobs, int njobs, int d, int V, hipStream_t stream);

}  // namespace specv
