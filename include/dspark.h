/*
 * libdspark: DSpark's per-round token path on one AMD Instinct MI355X (gfx950).
 *
 * Sources (page titles; sections, equations):
 *   [R] "DSpark: Confidence-Scheduled Speculative Decoding with
 *       Semi-Autoregressive Generation", technical review (zhongzhuzhou.org):
 *       "Speculative Decoding: Draft, Then Verify" (step 3), "The Sequential
 *       Correction" (Eq. 4), "Instantiation 1: The Markov Head" (Eq. 5),
 *       "The Confidence Head" (Eq. 8), "Deriving the Acceptance-Rate Identity
 *       Behind Equation 8" (Eq. 8a-8c), "The Hardware-Aware Prefix Scheduler"
 *       (cumulative products, Algorithm 1), "The Non-Anticipating Property"
 *       (Eq. 9-10), "Common Questions Answered" (greedy decoding, ties),
 *       "Putting It All Together: The Full Decode Loop as Pseudocode".
 *   [E] "Speculative decoding, from zero to DSpark", section 2 "The loop, and
 *       why it's lossless" (residual rule, bonus token).
 *   [Z] "DSpark：置信度调度的半自回归投机解码" (robotworld.top review),
 *       confidence-head paragraph (accept-rate label clamped to [0, 1]).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Symbols: B requests, gamma draft positions, V vocabulary size, r Markov
 * rank, T temperature.  Position k runs 1..gamma (stored 0-based).
 *
 * Memory.  Every array pointer is a DEVICE pointer to contiguous row-major
 * memory, aligned to 16 bytes, owned by the caller.  The library allocates
 * nothing and keeps no state between calls; scratch memory is the caller's
 * `workspace` of at least dspark_workspace_size(op, ...) bytes, which must not
 * be shared by calls that may run concurrently.  The one exception is
 * dspark_markov_draft_noalloc, whose scratch is a static device array.
 *
 * Layouts.
 *   U       float32 [B][gamma][V]      base logits U_k of the parallel backbone
 *   W1      [V][r]                     Markov embedding (bf16 or float32)
 *   W2      [r][V]                     Markov projection (same dtype as W1)
 *   x0      int32 [B]                  anchors (the previous round's last token)
 *   target  float32 [B][gamma+1][V]    target logits; row gamma+1 is the bonus
 *                                      position after the block
 *   seeds   uint64 [B]                 per-request Philox4x64-10 keys
 *
 * Random numbers.  Each draw is word w of Philox4x64-10 (Salmon, Moraes,
 * Dror, Shaw, SC'11) under key (seeds[b], 0) at counter (round, k, stream, i),
 * mapped to the double ((w >> 12) + 0.5) * 2^-52 in (0, 1).  Streams: 0 draft
 * sample, 1 acceptance test, 2 residual proposals (word 0 proposal, word 1
 * keep test, index i = proposal number) and the bonus token (k = gamma+1,
 * i = 0), 3 exact residual fallback.  `round` is the caller's round counter:
 * the same (seeds, round, inputs) give bit-identical outputs.
 *
 * Sampling.  A categorical draw with uniform u takes the first token v, in
 * ascending vocabulary order, whose cumulative probability exceeds u.  At
 * T == 0 every draw becomes an argmax, lowest index on ties, and no random
 * numbers are used.
 *
 * Streams and errors.  Every call is asynchronous on `stream` and returns once
 * its kernels are enqueued; outputs are valid after the stream is
 * synchronised.  Arguments are validated on the host before any HIP call:
 * DSPARK_ERR_INVALID_ARGUMENT for sizes out of range (1 <= B <= 65536,
 * 1 <= gamma <= 32, 2 <= V < 2^31, 16 <= r <= 512 with r % 16 == 0, T finite
 * and >= 0), a NULL required pointer or a misaligned one;
 * DSPARK_ERR_UNSUPPORTED for an unknown weight dtype; DSPARK_ERR_WORKSPACE for
 * a workspace smaller than dspark_workspace_size; DSPARK_ERR_HIP when a
 * launch fails.  On error the outputs are unspecified.  Logits must be finite
 * or -inf, and no row may be all -inf.  A token id outside [0, V) in x0 or
 * draft_tokens is detected on the device: that request's outputs become -1
 * (tokens, accept_len) and NaN (probabilities); the other requests are
 * unaffected.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSPARK_OK = 0,
  DSPARK_ERR_INVALID_ARGUMENT = -1,
  DSPARK_ERR_UNSUPPORTED = -2,
  DSPARK_ERR_WORKSPACE = -3,
  DSPARK_ERR_HIP = -4,
  DSPARK_ERR_SCRATCH_LIMIT = -5
} dspark_status;

/* Storage type of W1 and W2. */
typedef enum { DSPARK_F32 = 0, DSPARK_BF16 = 1 } dspark_dtype;

/* Admission rule of dspark_schedule. */
typedef enum {
  DSPARK_SCHEDULE_EARLY_STOP = 0,
  DSPARK_SCHEDULE_CAPACITY = 1,
  DSPARK_SCHEDULE_TOP_K = 2
} dspark_schedule_mode;

/* Which entry point a workspace is sized for. */
typedef enum {
  DSPARK_OP_DRAFT = 0,
  DSPARK_OP_VERIFY = 1,
  DSPARK_OP_SURVIVAL = 2,
  DSPARK_OP_RNN_DRAFT = 3
} dspark_op;

/* Maximum number of residual proposals drawn against p_t before the exact
 * residual inverse CDF (stream 3) is used. */
#define DSPARK_MAX_RESIDUAL_PROPOSALS 64

/* Library version as major * 10000 + minor * 100 + patch. */
int dspark_version(void);

/* Static, NUL-terminated description of a status code. */
const char* dspark_status_string(dspark_status s);

/* Bytes of device workspace that `op` needs for these sizes; 0 when the sizes
 * are out of range.  The workspace needs no initialisation. */
size_t dspark_workspace_size(dspark_op op, int B, int gamma, int V, int r);

/*
 * dspark_markov_bias -- rows of the rank-r bigram bias, Eq. 5 of [R]
 * ("Instantiation 1: The Markov Head"):  out[i][v] = sum_j W1[tokens[i]][j] W2[j][v].
 *
 *   tokens  int32 [n]           previous tokens, 0 <= tokens[i] < V
 *   out     float32 [n][V]      fp32 accumulation of the exact products; a row
 *                               whose token is out of range is all NaN
 * n >= 1.  Needs no workspace.
 */
dspark_status dspark_markov_bias(const void* W1, const void* W2, dspark_dtype wdtype,
                                 const int32_t* tokens, int n, int V, int r,
                                 float* out, hipStream_t stream);

/*
 * dspark_markov_draft -- semi-autoregressive block sampling of [R]
 * "The Sequential Correction" (Eq. 4) with the Markov head (Eq. 5).
 *
 * For every request b and k = 1..gamma, left to right:
 *   l_k(v)  = U[b][k][v] + W1[x_{k-1}] . W2[:, v]      (x_0 = x0[b])
 *   p_d^k   = softmax(l_k / T)  over the whole vocabulary
 *   x_k     = categorical draw from p_d^k with the stream-0 uniform at (round, k)
 * At T == 0, x_k = argmax l_k, draft_prob = 1 and draft_lse = 0.
 *
 * W2T is optional (NULL to skip): W2 transposed, [V][r] in the weight dtype,
 * as dspark_transpose_w2 writes it.  When it is given, the weights are bf16,
 * r == 256, V % 16 == 0, V <= 80 * 8 * (compute units - 16) (153600 on
 * MI355X), B <= 512, 4 B gamma V < 2^32 and no confidence output is asked
 * for, all gamma positions run in one cooperative launch that keeps W2 on
 * chip (the "device-resident" loop); otherwise, or when the device cannot
 * hold that launch, each position is its own pair of launches.  Both give the same draws up to the
 * summation order of float32 sums.  If a grid-wide wait of the resident loop
 * ever times out (it cannot while the launch is co-resident), every request's
 * outputs are -1 / NaN.
 *
 * Outputs:
 *   draft_tokens  int32   [B][gamma]  x_1..x_gamma
 *   draft_prob    float32 [B][gamma]  p_d^k(x_k)
 *   draft_lse     float32 [B][gamma]  log sum_v exp(l_k(v) / T), the log
 *                                     normaliser of p_d^k (used by
 *                                     dspark_survival)
 *
 * Confidence head (optional; conf == NULL skips it and conf_h, conf_w,
 * conf_sts, conf_d are not read): the per-position confidence of [R] "The
 * Confidence Head" (Eq. 7; the decode round of "Putting It All Together"
 * computes it inside the draft loop, step 6) with the temperatures of
 * Sequential Temperature Scaling (same section), computed by the selection
 * that draws x_{k-1}, where that token's W1 row is read anyway:
 *   c_{b,k} = sigma(z / t_k),  z = w . [h_{b,k} ; W1[x_{k-1}]]   (x_0 = x0[b])
 *   conf_h    float32 [B][gamma][conf_d]  hidden states h_k (16-byte aligned)
 *   conf_w    float32 [conf_d + r]        head weights: hidden part, then
 *                                         embedding part (16-byte aligned)
 *   conf_sts  float32 [gamma]             calibrated temperatures t_k > 0
 *                                         (NULL: 1, the raw head)
 *   conf      float32 [B][gamma]          out: c_{b,k}; NaN where x_{k-1} is
 *                                         outside [0, V)
 * 1 <= conf_d <= 2^20; z is summed in float64 from the float32 products, as
 * dspark_confidence computes it for given tokens.
 * Workspace: dspark_workspace_size(DSPARK_OP_DRAFT, B, gamma, V, r).
 */
dspark_status dspark_markov_draft(const float* U, const void* W1, const void* W2, const void* W2T,
                                  dspark_dtype wdtype, const int32_t* x0,
                                  int B, int gamma, int V, int r, float temperature,
                                  const uint64_t* seeds, uint64_t round,
                                  int32_t* draft_tokens, float* draft_prob, float* draft_lse,
                                  const float* conf_h, const float* conf_w, const float* conf_sts, int conf_d,
                                  float* conf, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dspark_markov_draft_noalloc -- dspark_markov_draft without a workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).
 *
 * Arguments, outputs and results are exactly those of dspark_markov_draft
 * (the same kernels run).  Its scratch memory is a static device array of
 * dspark_static_scratch_bytes() bytes (32 MiB) inside the library, one per
 * GPU, held until the process ends; the call allocates nothing (no hipMalloc,
 * hipFree or allocating routine; the per-kernel event timing records nothing
 * for it).  Sizes whose dspark_workspace_size(DSPARK_OP_DRAFT, ...) exceeds
 * that array return DSPARK_ERR_SCRATCH_LIMIT before any HIP call.  Every call
 * on a GPU shares that GPU's array: calls that overlap on one GPU (other
 * streams, other threads) race on it and must be serialised by the caller.
 * The array is that of the device current at the call, which must be the
 * device of `stream`.
 */
dspark_status dspark_markov_draft_noalloc(const float* U, const void* W1, const void* W2, const void* W2T,
                                          dspark_dtype wdtype, const int32_t* x0,
                                          int B, int gamma, int V, int r, float temperature,
                                          const uint64_t* seeds, uint64_t round,
                                          int32_t* draft_tokens, float* draft_prob, float* draft_lse,
                                          const float* conf_h, const float* conf_w, const float* conf_sts,
                                          int conf_d, float* conf, hipStream_t stream);

/* Bytes of the static scratch array of dspark_markov_draft_noalloc. */
size_t dspark_static_scratch_bytes(void);

/*
 * dspark_rnn_draft -- the same block sampling with the RNN head of [R]
 * "Instantiation 2: The RNN Head" (Eq. 6) in place of the Markov bias.
 *
 * For every request b, s_0 = 0 and for k = 1..gamma, left to right:
 *   (g, c, o) = Wp [s_{k-1} ; W1[x_{k-1}]] + hp[b][k-1]     (x_0 = x0[b])
 *   s_k       = sigmoid(g) s_{k-1} + (1 - sigmoid(g)) tanh(c)
 *   e_k       = tanh(o)
 *   l_k(v)    = U[b][k][v] + e_k . W2[:, v]
 * then x_k, draft_prob and draft_lse exactly as dspark_markov_draft (same
 * stream-0 uniforms, same greedy rule at T == 0).
 *
 *   W1, W2  bf16 only (wdtype must be DSPARK_BF16)
 *   Wp      float32 [3r][2r]   rows: gate, candidate, output; columns: the
 *                              state s_{k-1}, then the token embedding
 *   hp      float32 [B][gamma][3r]  the hidden-state part of the projection,
 *                              W_p[:, 2r:] h_k, computed by the caller (it
 *                              depends on no drafted token)
 *   e_out   float32 [B][gamma][r] or NULL: the e_k used
 * The cell computes in float32 (the precision of Wp and hp); e_k enters the
 * bf16 tile pass as two bf16 parts (e_k to about 2^-18 relative).  A position after an invalid anchor or
 * token is -1 / NaN as in dspark_markov_draft.
 * The hidden state enters only through hp: the library takes the product
 * W_p[:, 2r:] h_k, not h_k and that block of W_p, because it depends on no
 * drafted token and is one dense GEMM of the backbone's parallel stage.
 * To verify an RNN draft or take its survival products, pass e_out as the
 * draft_rows argument of dspark_verify and dspark_survival: without it they
 * rebuild p_d from the Markov head, which is not the law these tokens were
 * drawn from.
 * Workspace: dspark_workspace_size(DSPARK_OP_RNN_DRAFT, B, gamma, V, r).
 * Errors: DSPARK_ERR_UNSUPPORTED for float32 weights, otherwise as
 * dspark_markov_draft.
 */
dspark_status dspark_rnn_draft(const float* U, const void* W1, const void* W2, dspark_dtype wdtype,
                               const float* Wp, const float* hp, const int32_t* x0,
                               int B, int gamma, int V, int r, float temperature,
                               const uint64_t* seeds, uint64_t round,
                               int32_t* draft_tokens, float* draft_prob, float* draft_lse, float* e_out,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dspark_verify -- lossless rejection-sampling verification of the drafted
 * blocks: [R] "Speculative Decoding: Draft, Then Verify" step 3 and [E]
 * section 2.
 *
 * For every request b, k = 1..gamma left to right, with p_t^k = softmax(target[b][k] / T):
 *   alpha_k = min(1, p_t^k(x_k) / p_d^k(x_k))   (p_d^k(x_k) = draft_prob[b][k])
 *   accept x_k iff the stream-1 uniform at (round, k) is < alpha_k.
 * At the first rejection j, one token is drawn from norm(max(0, p_t^j - p_d^j))
 * and the block ends (n = j - 1): proposals v ~ p_t^j (stream 2, word 0,
 * index i) are kept with probability max(0, 1 - p_d^j(v) / p_t^j(v)) (stream 2,
 * word 1); after DSPARK_MAX_RESIDUAL_PROPOSALS misses the residual itself is
 * drawn by inverse CDF with the stream-3 uniform at (round, j).  p_d^j(v) is
 * rebuilt from U, W2 and the draft's operand row: W1[x_{j-1}] of the Markov
 * head, or e_j of an RNN draft when draft_rows is given.  If all gamma
 * positions pass (n = gamma)
 * a bonus token is drawn from p_t^{gamma+1} with the stream-2 uniform at
 * (round, gamma+1, index 0).
 * At T == 0 acceptance is the exact match x_k == argmax target[b][k] and the
 * correction or bonus token is argmax target[b][n+1] ([R] "Common Questions
 * Answered").
 *
 * lengths is optional (NULL: every request verifies its whole block): int32
 * [B], the scheduled verification lengths l_b of [R] "The Hardware-Aware
 * Prefix Scheduler" (as dspark_schedule writes them).  Only x_1..x_l are
 * offered to the target: n <= l, and if all l pass, the bonus token is drawn
 * from p_t^{l+1} (target row l+1) with the stream-2 uniform at (round, l+1,
 * index 0), so l = 0 emits one token drawn from p_t^1 and l = gamma is the
 * full block.  A length outside [0, gamma] invalidates that request like a
 * bad token id.  The lengths must be fixed before the drafted tokens are
 * seen (non-anticipating, [R] "The Non-Anticipating Property"): a schedule
 * that depends on them changes the output law.
 *
 * W2T is optional (NULL to skip): W2 transposed, [V][r] in the weight dtype,
 * as written by dspark_transpose_w2.  When given, p_d at a single token reads
 * one contiguous row of W2T instead of r elements spread over W2; the results
 * differ from the W2-only path only by the summation order of float64 sums.
 * Inputs draft_tokens / draft_prob are the draft's outputs (dspark_markov_draft
 * or dspark_rnn_draft).
 * draft_rows is optional: NULL for a Markov-head draft; for a draft of the RNN
 * head ([R] "Instantiation 2: The RNN Head", Eq. 6, which the decode round of
 * [R] "Putting It All Together" verifies like the Markov head's), float32
 * [B][gamma][r], the e_k rows dspark_rnn_draft writes to e_out, so that p_d^k
 * = softmax((U_k + e_k W2) / T) is the law x_k was drawn from.  Not read at
 * T == 0.
 * Outputs:
 *   accept_len   int32   [B]          n in 0..l (l = gamma without lengths)
 *   out_tokens   int32   [B][gamma+1] x_1..x_n, then the correction or bonus
 *                                     token, then -1
 *   accept_prob  float32 [B][gamma]   alpha_k for the tested positions
 *                                     k <= min(n+1, l), NaN after; NULL to skip
 * Workspace: dspark_workspace_size(DSPARK_OP_VERIFY, B, gamma, V, r).
 */
dspark_status dspark_verify(const float* U, const void* W1, const void* W2, const void* W2T, dspark_dtype wdtype,
                            const int32_t* x0, const int32_t* draft_tokens,
                            const float* draft_prob, const float* draft_rows, const float* target_logits,
                            const int32_t* lengths,
                            int B, int gamma, int V, int r, float temperature,
                            const uint64_t* seeds, uint64_t round,
                            int32_t* accept_len, int32_t* out_tokens, float* accept_prob,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dspark_transpose_w2 -- W2T[v][j] = W2[j][v]: the Markov projection of [R]
 * Eq. 5 stored vocabulary-major, for the single-token p_d evaluations of
 * dspark_verify.  The weights are constant across rounds, so the copy is made
 * once per model.
 *
 *   W2   [r][V] (bf16 or float32, per wdtype)
 *   W2T  out, [V][r], same dtype; must not overlap W2
 * 2 <= V < 2^31, 16 <= r <= 512 with r % 16 == 0.  Needs no workspace.
 */
dspark_status dspark_transpose_w2(const void* W2, dspark_dtype wdtype, int r, int V, void* W2T, hipStream_t stream);

/*
 * dspark_survival -- prefix survival products a_{b,k} = prod_{i<=k} c_{b,i}
 * of [R] "The Hardware-Aware Prefix Scheduler".
 *
 * Confidence mode (conf != NULL, float32 [B][gamma]): c = conf; U, W1, W2,
 * x0, draft_tokens, draft_lse and target_logits are not read and may be NULL,
 * and c_star is not written.
 * Analytical mode (conf == NULL): c_{b,k} = c*_k = clamp(sum_v min(p_d^k(v),
 * p_t^k(v)), 0, 1), the acceptance probability of Eq. 8a / 8c with the
 * clamp of [Z], at every block position k = 1..gamma along the drafted prefix;
 * p_d^k(v) = exp(l_k(v) / T - draft_lse[b][k]).  At T == 0, c*_k is the
 * indicator x_k == argmax target[b][k].
 * draft_rows as for dspark_verify: NULL for a Markov-head draft (l_k = U_k +
 * W1[x_{k-1}] W2), or float32 [B][gamma][r], the e_k rows of an RNN draft
 * (l_k = U_k + e_k W2; finite values; with bf16 weights e_k enters the tile
 * pass as two bf16 parts, as in dspark_rnn_draft).
 *
 * Outputs: c_star float32 [B][gamma] (analytical mode; NULL to skip) and
 * survival float32 [B][gamma].
 * Workspace: dspark_workspace_size(DSPARK_OP_SURVIVAL, B, gamma, V, r); 0
 * bytes are needed in confidence mode.
 */
dspark_status dspark_survival(const float* U, const void* W1, const void* W2, dspark_dtype wdtype,
                              const int32_t* x0, const int32_t* draft_tokens,
                              const float* draft_lse, const float* draft_rows, const float* target_logits,
                              const float* conf, int B, int gamma, int V, int r,
                              float temperature, float* c_star, float* survival,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dspark_confidence -- the confidence head of [R] "The Confidence Head"
 * (Eq. 7) with the per-position temperatures of Sequential Temperature
 * Scaling (same section):
 *   c_{b,k} = sigma(z / t_k),  z = w . [h_{b,k} ; W1[x_{k-1}]]   (x_0 = x0[b])
 * for k = 1..gamma, the scalar the scheduler's survival products are built
 * from (dspark_survival in confidence mode, then dspark_schedule) before the
 * target runs.  A Markov-head draft gets the same values from
 * dspark_markov_draft's own confidence output with no launch of its own;
 * this entry point serves tokens drafted elsewhere (an RNN-head draft).
 *
 *   h             float32 [B][gamma][d]  backbone hidden states h_k
 *   w             float32 [d + r]        head weights: hidden part, then
 *                                        embedding part (no bias term)
 *   W1            [V][r]                 the Markov embedding of the draft
 *   x0            int32 [B]              anchors
 *   draft_tokens  int32 [B][gamma]       dspark_markov_draft's tokens (x_k
 *                                        feeds position k+1; x_gamma is unused)
 *   sts           float32 [gamma]        calibrated temperatures t_k > 0
 *                                        (NULL: 1, the raw head)
 *   conf          float32 [B][gamma]     out: c_{b,k}; NaN where the previous
 *                                        token is outside [0, V)
 * z is summed in float64 from the float32 products.  1 <= d <= 2^20; the
 * other sizes as for dspark_markov_draft.  Asynchronous on `stream`; needs
 * no workspace.
 */
dspark_status dspark_confidence(const float* h, const float* w, const void* W1, dspark_dtype wdtype,
                                const int32_t* x0, const int32_t* draft_tokens, const float* sts, int B, int gamma,
                                int d, int V, int r, float* conf, hipStream_t stream);

/*
 * dspark_schedule -- the hardware-aware prefix scheduler, Algorithm 1 of [R]
 * "The Hardware-Aware Prefix Scheduler": per-request verification lengths
 * that maximise the expected token throughput Theta = tau * SPS(n).
 *
 *   survival  float32 [B][gamma]  a_{b,j}, the prefix survival products (as
 *                                 dspark_survival writes them); entries <= 0
 *                                 or NaN are not candidates
 *   sps       float64 [sps_len]   sps[n] = SPS(n), the profiled target
 *                                 throughput at n verified tokens;
 *                                 sps_len >= B (gamma + 1) + 1
 *   lengths   int32 [B]           out: l*_b in 0..gamma
 *   theta     float64 [1]         out: Theta_best (NULL to skip)
 *
 * The candidates (b, j) are admitted in descending a_{b,j}, ties to the
 * lowest request and then the lowest position ([R] "Common Questions
 * Answered").  Starting from n = B verified tokens and tau = B, the m-th
 * admission adds one token and a_{b,j} to tau; the scan keeps the admission
 * while Theta = tau * sps[n] improves on the previous value and stops at the
 * first one that does not (the early stop that keeps the schedule
 * non-anticipating, [R] "The Non-Anticipating Property", Eq. 9-10).  l*_b is
 * the largest position admitted for b; with survivals that do not increase
 * along a block, the admitted positions of b are exactly 1..l*_b (Lemma 1).
 * tau is summed in float64; decisions whose two Theta values agree to
 * rounding may resolve either way.
 *
 * mode selects the admission rule:
 *   DSPARK_SCHEDULE_EARLY_STOP  Algorithm 1 as above (capacity_in and
 *                               capacity_out are not used).
 *   DSPARK_SCHEDULE_CAPACITY    the unconstrained search of [R] "The
 *                               Asynchronous Fix, and Why It Stays Lossless":
 *                               the admission count m* at the first maximum of
 *                               Theta over the whole sorted scan (0..all
 *                               candidates), written to capacity_out[0]
 *                               (nullable) with the lengths and Theta of that
 *                               admission.  Run on survival products from two
 *                               steps earlier, m* is the capacity K.
 *   DSPARK_SCHEDULE_TOP_K       the first min(K, candidates) sorted candidates
 *                               of the current products are admitted, K =
 *                               capacity_in[0] (device int32, decided
 *                               earlier; negative counts as 0); theta is
 *                               Theta at that admission.
 * In every mode the lengths depend on the drafted tokens only through the
 * survival products of positions that are admitted before them, which keeps
 * verification lossless; a capacity computed from the current round's
 * products would not.
 * 1 <= gamma <= 32, 1 <= B * gamma <= 16384.  Asynchronous on `stream`; needs
 * no workspace.
 */
dspark_status dspark_schedule(const float* survival, const double* sps, int sps_len, int B, int gamma,
                              dspark_schedule_mode mode, const int32_t* capacity_in, int32_t* capacity_out,
                              int32_t* lengths, double* theta, hipStream_t stream);

/*
 * Per-kernel timing (tracing).  dspark_profile_enable(1) clears earlier
 * records and makes every later kernel launch of the library record a HIP
 * event before and after it on its stream; dspark_profile_enable(0) stops
 * recording.  dspark_profile_get(kind, ...) waits for the recorded events of
 * one kernel kind (0 <= kind < dspark_profile_kinds()) and returns its name (a
 * static string), the number of launches recorded and their summed elapsed
 * milliseconds.  Events are host-side objects created on first use and
 * reused; no device memory is allocated.
 */
dspark_status dspark_profile_enable(int on);
int dspark_profile_kinds(void);
dspark_status dspark_profile_get(int kind, const char** name, long long* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
