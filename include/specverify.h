/*
 * specverify.h -- C ABI of the speculative-sampling verification library for
 * AMD Instinct MI355X (gfx950).
 *
 * Pages cited:
 *   [FI] intuitivepapers.ai, "Fast Inference from Transformers via Speculative Decoding"
 *   [SD] nonconvexcard course page, "Speculative Decoding"
 *   [LH] lihaoran.work article on speculative decoding
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA tensors),
 *     row-major, owned by the caller.  They must stay valid until the work
 *     queued on `stream` has run.  The library keeps no pointer after a call
 *     returns, allocates no device memory, and holds no global state besides
 *     the kernels; calls are thread-safe.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls are asynchronous: they queue kernels on `stream` and return.
 *   - Argument errors are detected on the host before anything is queued.
 *     Nothing is written in that case.  A HIP launch failure returns SPEC_EHIP.
 *   - Logits must be finite or -inf (-inf means probability 0, for example a
 *     token masked out before sampling), and at T > 0 every finite logit l
 *     must keep l * log2(e) / T finite in fp32 (the scaled logit the softmax
 *     is taken of).  Every row needs at least one finite logit.  +inf or NaN
 *     logits, scaled logits that overflow, and rows with no finite logit are
 *     caller errors.  The results are then undefined but the kernels still
 *     terminate.
 *   - Outputs are deterministic: the same inputs give bit-identical outputs.
 *   - Workspace: the caller zero-fills it once before its first use (for
 *     example torch.zeros).  Every call that completes leaves it all-zero
 *     again, so it can be reused for any later call, of any shape up to its
 *     size, without clearing.  Two calls that may run at the same time need
 *     two workspaces.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum {
  SPEC_OK = 0,
  SPEC_EINVAL = -1,       /* bad argument: NULL pointer, size out of range, bad temperature */
  SPEC_EUNSUPPORTED = -2, /* unsupported dtype or algorithm */
  SPEC_ENOSPACE = -3,     /* workspace smaller than the *_workspace_size() query */
  SPEC_EHIP = -4          /* HIP runtime error while queueing work */
};

/* Element type of logit tensors. */
enum { SPEC_F32 = 0, SPEC_BF16 = 1 };

/* Algorithm selector for spec_verify_algo(). */
enum {
  SPEC_ALGO_AUTO = 0,      /* the faster path: fused at T > 0 where it takes the shape, else multipass */
  SPEC_ALGO_MULTIPASS = 1, /* row statistics, then pair overlap, then a per-sequence finish */
  SPEC_ALGO_FUSED = 2      /* one persistent kernel; every logit is read from HBM once */
};

#define SPEC_MAX_GAMMA 32

/* Human-readable text for a status code (static storage, never NULL). */
const char* spec_status_string(int status);

/*
 * Bytes of device workspace spec_verify() / spec_verify_algo() need for this
 * shape, for any algorithm and either dtype.  Returns 0 for invalid arguments.
 */
size_t spec_verify_workspace_size(int B, int gamma, int V, int dtype);

/*
 * spec_verify -- one verification step for a batch of B independent sequences
 * ([FI] "The loop: draft, verify in one pass, keep a prefix", Algorithm 1
 * steps 3-4; [SD] "The algorithm").
 *
 * For each sequence b, with positions i counted from 0:
 *   p_i = softmax(target_logits[b][i] / T), i = 0..gamma;
 *   q_i = softmax(draft_logits[b][i] / T),  i = 0..gamma-1.
 * The same temperature applies to both models ([FI] "The loop"; nazmi.tech
 * "5. Sampling and evaluation").
 *   alpha[b][i] = sum_x min(p_i(x), q_i(x)) = 1 - TV(p_i, q_i) for every i < gamma
 *     ([SD] "How often do we accept?").
 *   Drafts are walked left to right.  Draft x_i is kept iff
 *     uniforms[b][i] <= min(1, p_i(x_i) / q_i(x_i)); the walk stops at the first
 *     failure.  n_accepted[b] = number kept, in [0, gamma].
 *   next_token[b] is drawn with uniforms[b][gamma] by inverse CDF in token order
 *     (the first token whose cumulative weight exceeds u * total).  The weights
 *     are max(0, p_n - q_n) when n < gamma (the residual, [FI] "Speculative
 *     sampling: the accept/reject rule", eq. (2)), and p_gamma when every draft
 *     was kept (the bonus token).  Only a residual with no mass at all is not
 *     sampled: next_token is then drawn from p_n itself ([LH] "Three candidates
 *     explain the acceptance rule").  The weights are computed in fp32, so a
 *     residual whose true mass is within fp32 rounding of zero may be found
 *     empty, and a uniform within that rounding of a step of the CDF may pick
 *     the neighbouring token.
 *   T == 0 is argmax mode: p_i and q_i are one-hot at the row argmax, with ties
 *     going to the lowest index.  A draft is kept iff it equals the target
 *     argmax.  next_token is the target argmax at position n.  alpha is 1 where
 *     the two argmaxes agree, else 0 ([FI] "Speculative sampling", the
 *     temperature-to-zero limit; [LH] "What does 'unchanged output' mean?").
 *     The uniforms are not read.
 *   A ratio with q_i(x_i) = 0 follows IEEE rules: p > 0 keeps the draft, 0/0 rejects.
 *   A draft token outside [0, V) is rejected (it has p = q = 0).
 *   n_accepted[b] = next_token[b] = -1 reports that a workgroup gave up
 *     waiting on a partner workgroup (the fused path, and in argmax mode the
 *     multipass path's finishing workgroups; 2^20 polls by default, see
 *     spec_set_wait_limit; only possible when another kernel occupies the
 *     device's compute units at the same time).  That sequence has no result,
 *     and the waits that gave up may leave words in the workspace: it must be
 *     zero-filled again before its next use.
 *
 * Arguments:
 *   target_logits  [B][gamma+1][V], dtype
 *   draft_logits   [B][gamma][V],   dtype (may be NULL when gamma == 0)
 *   dtype          SPEC_F32 or SPEC_BF16
 *   draft_tokens   int32 [B][gamma], each in [0, V) (may be NULL when gamma == 0)
 *   uniforms       float32 [B][gamma+1], each in (0, 1)
 *   B >= 0, 0 <= gamma <= SPEC_MAX_GAMMA, 1 <= V <= 2^31 - 1
 *   temperature    0 (argmax) or finite with temperature >= FLT_MIN
 *   n_accepted     int32 [B] out
 *   next_token     int32 [B] out
 *   alpha          float32 [B][gamma] out, or NULL
 *   p_draft        float32 [B][gamma] out, p_i(x_i), or NULL
 *   q_draft        float32 [B][gamma] out, q_i(x_i), or NULL
 *   workspace      device scratch of at least spec_verify_workspace_size() bytes,
 *                  all-zero on entry (see the conventions above); all-zero on
 *                  return of the queued work.
 * Returns SPEC_OK or an error status.  B == 0 returns SPEC_OK and queues nothing.
 */
int spec_verify(const void* target_logits, const void* draft_logits, int dtype,
                const int32_t* draft_tokens, const float* uniforms,
                int B, int gamma, int V, float temperature,
                int32_t* n_accepted, int32_t* next_token, float* alpha,
                float* p_draft, float* q_draft,
                void* workspace, size_t workspace_bytes, void* stream);

/* spec_verify with an explicit algorithm (SPEC_ALGO_*).  All algorithms give the
 * same outputs up to the floating-point rounding of their reductions.
 * SPEC_ALGO_FUSED returns SPEC_EUNSUPPORTED, with nothing queued, for logit
 * tensors that do not start on 16 bytes, rows longer than 256 * 64 * 32
 * tokens, fp32 rows with V % 4 != 0, bf16 rows with V % 8 != 0 (rows that
 * do not all start on 16 bytes) in argmax mode, and per-sequence draft counts
 * (spec_verify_ex) with B > 2048; SPEC_ALGO_AUTO runs the multipass path for
 * those. */
int spec_verify_algo(int algo,
                     const void* target_logits, const void* draft_logits, int dtype,
                     const int32_t* draft_tokens, const float* uniforms,
                     int B, int gamma, int V, float temperature,
                     int32_t* n_accepted, int32_t* next_token, float* alpha,
                     float* p_draft, float* q_draft,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_verify_ex -- spec_verify_algo with optional extensions of the step.
 * With top_k == 0, top_p == 1, lenience == 1 and gamma_seq == NULL it is
 * spec_verify_algo exactly.
 *
 *   top_k, top_p  top-k and nucleus filtering of both models' rows before the
 *              step ([FI] "The loop: draft, verify in one pass, keep a prefix":
 *              the method runs on p and q as the sampling method adjusted them;
 *              [NZ] "5. Sampling and evaluation": the same settings for both).
 *              After the temperature, top-k keeps every token whose logit is at
 *              least the row's k-th largest (ties kept); then top-p keeps, of
 *              those, the smallest set of whole tie groups, most likely first,
 *              that holds at least top_p of their probability mass.  Every other
 *              token has probability 0, in alpha, the ratio tests and the
 *              samples.  top_k <= 0 or >= V, and top_p >= 1, disable a filter;
 *              top_p must be > 0 (else SPEC_EINVAL).  In argmax mode (T == 0)
 *              the filters change nothing and are skipped.  Both paths take
 *              filters, for any shape.  A filtered call launches the
 *              threshold kernel of spec_filter_thresholds (into the
 *              workspace), then the verification, whose last reader of each
 *              threshold zeroes it (the workspace is left zero).
 *
 *   lenience   l in (0, 1] ([FI] "The acceptance rate is the overlap of p and q",
 *              the lenience factor): draft i is kept when
 *              u_i <= min(1, p_i(x_i) / (l q_i(x_i))), and after the first
 *              rejection n the token is drawn from max(0, p_n - l q_n) (the page
 *              does not give the residual under l; this one is built from the
 *              same scaled comparison, and no token is then emitted more than
 *              1/l times as often as under p).  The output is exact only for
 *              l = 1.  alpha stays sum_x min(p_i, q_i).  Argmax mode (T == 0)
 *              is unaffected.  A value outside (0, 1] (or NaN) is SPEC_EINVAL.
 *   gamma_seq  NULL, or a device int32 [B]: gamma_b, the number of drafts of
 *              sequence b, for a batch of sequences with different draft counts
 *              ([LH] "A longer draft is not always faster": a draft may stop
 *              early) padded to gamma.  Sequence b's data sit in positions
 *              0..gamma_b of the padded arrays: draft rows and tokens
 *              0..gamma_b-1, target rows 0..gamma_b (row gamma_b is its
 *              bonus row), accept uniforms 0..gamma_b-1 and the final-sample
 *              uniform u[b][gamma_b].  Positions past gamma_b are padding: never
 *              read, and alpha / p_draft / q_draft there are set to NaN.
 *              n_accepted[b] <= gamma_b.  gamma_b = 0 is a plain decoding step
 *              (the token is drawn from target row 0).  The values are read on
 *              the device, so they are not checked here: a value below 0 or
 *              above gamma is taken as 0 or gamma.
 * All other arguments, the workspace and the return values are as for
 * spec_verify / spec_verify_algo.
 */
int spec_verify_ex(int algo,
                   const void* target_logits, const void* draft_logits, int dtype,
                   const int32_t* draft_tokens, const float* uniforms,
                   int B, int gamma, int V, float temperature,
                   int top_k, float top_p, float lenience, const int32_t* gamma_seq,
                   int32_t* n_accepted, int32_t* next_token, float* alpha,
                   float* p_draft, float* q_draft,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_filter_thresholds -- the per-row keep thresholds of top-k / top-p, as
 * spec_verify_ex applies them ([FI] "The loop: draft, verify in one pass, keep
 * a prefix"; [NZ] "5. Sampling and evaluation"), for callers that mask or
 * sample rows themselves.
 *   target_logits [B][gamma+1][V], draft_logits [B][gamma][V] (NULL when
 *   gamma == 0), dtype SPEC_F32 or SPEC_BF16, any V and alignment (16-byte
 *   aligned rows of whole 16-byte vectors take vector loads, other rows
 *   element loads).  temperature > 0 and finite (the top-p mass is that of
 *   softmax(logit / T)); top_k and top_p as for spec_verify_ex.
 *   thresholds  device float32 [B*(gamma+1) + B*gamma] out: first the target
 *               rows in order (b, i), then the draft rows.  Row r keeps the
 *               tokens whose logit is >= thresholds[r]; the value is one of the
 *               row's logits, or -inf when the row keeps everything (no filter
 *               active, or fewer finite logits than top_k).
 *   workspace   NULL, or device scratch of at least
 *               spec_filter_workspace_size() bytes, all-zero on entry and
 *               all-zero on return of the queued work.  With a workspace, a
 *               top-k of at most 64 first lists each 8192-token chunk's
 *               candidates (the values at or above a pivot the chunk has k
 *               values above) and selects from their union, without holding
 *               the row; the thresholds are the same either way.  A smaller
 *               non-NULL workspace is SPEC_ENOSPACE.
 *   Ties are kept.  Masses are fp32 exp2((logit - max) log2(e) / T), summed in
 *   fp64 and 2^-40 fixed point; a nucleus boundary within the fp32 rounding of
 *   those weights (a few 1e-7 of the total for the rows of the B=64, V=128256
 *   workload) of top_p may fall on either side of that tie group.
 *   Returns SPEC_EINVAL for a bad shape, temperature or top_p.
 */
int spec_filter_thresholds(const void* target_logits, const void* draft_logits, int dtype,
                           int B, int gamma, int V, float temperature, int top_k, float top_p,
                           float* thresholds, void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_verify_noalloc -- spec_verify for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  The same verification as spec_verify (the same kernels,
 * outputs bit-identical to spec_verify's for the same inputs), with its scratch
 * in a device array the library holds instead of a workspace argument.  The
 * caller still passes every input and output.
 *   Arguments, outputs and status codes as for spec_verify, without
 *   workspace / workspace_bytes.
 *   The array is spec_verify_noalloc_limit() bytes (16 MiB) on each device the
 *   library runs on, kept until the process ends and zero-filled on the first
 *   call on that device.  A shape whose scratch would exceed it returns
 *   SPEC_ENOSPACE before anything is queued (B=256, gamma=8, V=256000 needs
 *   6.8 MB).  No call allocates device or host memory.
 *   Every call on a device uses that device's one array: calls that may run at
 *   the same time on one device (two streams, two threads) race and must not
 *   overlap.  A call that completes leaves the array zero again.  A sequence
 *   that reports -1 (a wait gave up, see spec_verify) may leave stale words
 *   in it: a call with B == 0 (and any valid gamma, V and temperature) queues a
 *   kernel that zero-fills the whole array on `stream`, to run before the next
 *   verification.
 */
int spec_verify_noalloc(const void* target_logits, const void* draft_logits, int dtype,
                        const int32_t* draft_tokens, const float* uniforms,
                        int B, int gamma, int V, float temperature,
                        int32_t* n_accepted, int32_t* next_token, float* alpha,
                        float* p_draft, float* q_draft, void* stream);

/* Bytes of the device array spec_verify_noalloc uses on each device. */
size_t spec_verify_noalloc_limit(void);

/*
 * spec_set_wait_limit -- the number of polls after which every cross-workgroup
 * wait of a later launch in this process gives up (the fused path, and the
 * multipass path's argmax finishing; the sequence
 * then reports -1, see spec_verify).  0 restores the default, 2^20.  It exists
 * for callers and tests that exercise the give-up path: a small limit makes
 * waits give up whenever their data is late, and every kernel still exits
 * normally.  A process-wide setting, read when a launch is queued; not for use
 * while other threads queue launches.
 */
void spec_set_wait_limit(unsigned polls);

/* Bytes of the optional spec_filter_thresholds() workspace; 0 for a bad shape. */
size_t spec_filter_workspace_size(int B, int gamma, int V);

/*
 * spec_lmhead_logits -- the target pass's final matrix product for the positions
 * being verified ([FI] "Decoding waits on memory, not arithmetic": every weight
 * is read once per pass).
 *   logits[m][v] = sum_k hidden[m][k] * W[k][v], with bf16 inputs, products
 *   exact in fp32, fp32 accumulation (matrix cores), written as fp32.
 *   hidden  bf16 [M][d];  W  bf16 [d][V];  logits  float32 [M][V] out.
 *   1 <= M <= 256; d >= 32 and a multiple of 32; V >= 8 and a multiple of 8.
 *   All three pointers 16-byte aligned.  W is read once per 64 rows of M.
 *   Returns SPEC_EINVAL for any other shape or alignment.
 */
int spec_lmhead_logits(const void* hidden, const void* W, int M, int d, int V,
                       float* logits, void* stream);

/*
 * spec_lmhead_verify -- LM heads of both models over the verified positions,
 * followed by spec_verify at `temperature`.
 *   hidden           bf16 [B*(gamma+1)][d], the target's hidden states at the
 *                    gamma+1 positions of each sequence
 *   hidden_draft     bf16 [B*gamma][d], or NULL to use rows 0..gamma-1 of each
 *                    sequence's block of `hidden`
 *   W_target, W_draft  bf16 [d][V]
 *   target_logits    float32 [B][gamma+1][V] out (caller-owned; feeds the verify)
 *   draft_logits     float32 [B][gamma][V]   out
 *   other arguments as for spec_verify (the logits are fp32).
 * Both products run in one launch (for B*(gamma+1) <= 64), then the verification
 * on the fp32 logits.  Limits and alignment as spec_lmhead_logits for d, V and
 * every pointer; B*(gamma+1) <= 256.  The workspace is that of spec_verify for
 * SPEC_F32 (spec_lmhead_workspace_size), zero on entry as there.
 */
size_t spec_lmhead_workspace_size(int B, int gamma, int d, int V);
int spec_lmhead_verify(const void* hidden, const void* hidden_draft,
                       const void* W_target, const void* W_draft,
                       int B, int gamma, int d, int V,
                       const int32_t* draft_tokens, const float* uniforms, float temperature,
                       float* target_logits, float* draft_logits,
                       int32_t* n_accepted, int32_t* next_token, float* alpha,
                       float* p_draft, float* q_draft,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_kv_crop -- the KV-cache crop that follows a verification step ([FI]
 * "The loop: draft, verify in one pass, keep a prefix", the KV-cache paragraph:
 * after the accept test the cache entries past the accepted prefix are
 * discarded, one crop after the sampling function; [LH] "Fix the benchmark
 * conditions first": the cache follows the committed prefix).  Contiguous
 * caches, each [B][H][S_max][entry_bytes] (entry_bytes = head size times the
 * element size), for example the K and V caches of every layer.
 *   caches       HOST array of n_caches device pointers (1..SPEC_KV_MAX_CACHES,
 *                16-byte aligned); may be NULL when clear == 0
 *   seq_len      device int32 [B], in and out: on entry the committed length
 *                of each sequence before the verification pass; the pass
 *                wrote `appended` entries after it (seq_len .. seq_len +
 *                appended - 1).  On return of the queued work: seq_len +
 *                keep_extra + n_accepted.
 *   n_accepted   device int32 [B], as spec_verify wrote it (read on the
 *                device: queue this after the verification on the same stream,
 *                no synchronisation needed).  A sequence with -1 is left as
 *                it was.
 *   keep_extra   entries kept besides the accepted drafts (0..appended; 1 when
 *                the pass also wrote the entry of the previous step's final
 *                token).  The new token of this step is not in the cache.
 *   clear        nonzero: zero-fill the discarded entries [new length, seq_len
 *                + appended) of every cache and head (positions at or past
 *                S_max are never touched); zero: only the lengths change.
 *   entry_bytes  a multiple of 16.
 * Two launches on `stream` (the fill, then the lengths).  Returns SPEC_EINVAL
 * for a bad argument; B == 0 returns SPEC_OK and queues nothing.
 */
#define SPEC_KV_MAX_CACHES 256
#define SPEC_KV_MAX_APPENDED 1024
int spec_kv_crop(void* const* caches, int n_caches, int B, int H, int S_max, int entry_bytes,
                 int32_t* seq_len, const int32_t* n_accepted, int appended, int keep_extra, int clear,
                 void* stream);

/*
 * spec_kv_crop_paged -- spec_kv_crop for a paged cache ([LH] "Fix the
 * benchmark conditions first": with paged storage the rejected state is whole
 * pages).  Each cache is [num_pages][page_size][token_bytes] (token_bytes =
 * heads x head size x element size, a multiple of 16); sequence b's position s
 * lives in page block_table[b][s / page_size] at slot s % page_size
 * (an entry outside [0, num_pages), e.g. -1, is no page).
 *   block_table  device int32 [B][max_blocks], in and out
 *   seq_len, n_accepted, appended, keep_extra, clear  as for spec_kv_crop
 *                (clear zero-fills the discarded slots of every cache);
 *                appended <= SPEC_KV_MAX_APPENDED
 *   free_pages   device int32 [free_capacity] (free_capacity >= num_pages),
 *   free_count   device int32 [1]: the pool's free list.  Every page of a
 *                cropped sequence at block index >= ceil(new length /
 *                page_size) is released: its id is written to
 *                free_pages[free_count++] -- sequences in order, blocks in
 *                ascending order -- and its table entry becomes -1.  Pages past
 *                a sequence's crop point must belong to that sequence alone.
 * Two launches on `stream`, the second a single workgroup.  Returns SPEC_EINVAL
 * for a bad argument; B == 0 returns SPEC_OK and queues nothing.
 */
int spec_kv_crop_paged(void* const* caches, int n_caches, int num_pages, int page_size, int token_bytes,
                       int32_t* block_table, int B, int max_blocks, int32_t* seq_len,
                       const int32_t* n_accepted, int appended, int keep_extra, int clear,
                       int32_t* free_pages, int32_t* free_count, int free_capacity, void* stream);

/*
 * spec_stream_read -- a plain streaming read of a device buffer, for the HBM
 * read rate the device sustains (the context the verification's bandwidth
 * is judged against; not part of the method).
 *   buffer  device pointer, 16-byte aligned; bytes a multiple of 16 (read once)
 *   sink    device uint32 [blocks] out: the XOR of each workgroup's words (it
 *           keeps the reads from being dropped; the values mean nothing)
 *   blocks  workgroups of 256 threads (a few per compute unit fill the device)
 * Returns SPEC_EINVAL for a null pointer, misalignment or blocks < 1.
 */
int spec_stream_read(const void* buffer, size_t bytes, uint32_t* sink, int blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
