/*
 * gdn_oracle.h -- reference (test-infrastructure) implementation of the gated
 * delta-rule recurrence, in plain C and IEEE double.
 *
 * TEST INFRASTRUCTURE ONLY.  This code is the slow, obviously-correct CPU
 * definition that the HIP library is checked against.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it; the
 * library's own path never does.  It shares no source with the HIP library.
 *
 * Sources (web pages; cited by page and section, no line numbers):
 *   [P1] onnxruntime-ep-mlx 0.31.1, src/ops/ssm.rs
 *        -- `linear_attention_op` (stable unroll, T = 0 handling),
 *           `linear_attention_gate_op`, the wide-BF16 working-state test,
 *           `causal_conv_op` (CausalConvWithState), `gated_rms_norm_op`.
 *   [P3] nuvec-core 0.6.1, fast/imp.rs -- `gated_delta_graph`, the
 *        `causal_conv1d_slots` fallback graph.
 *   [P4] onnx-runtime-ep-cuda 0.1.0-dev.6, src/kernels/linear_attention.rs
 *        -- module doc "Parallelization", `linear_attention_core` steps
 *           1-4, the gate helpers `la_sigmoid` / `la_softplus`,
 *           `LinearAttentionFactory::create` (default scale),
 *           `UpdateRule` (rule family).
 *
 * Layouts (all row-major, contiguous, double):
 *   q, k          [T_total, h_qk, d_k]
 *   v, out        [T_total, h_v,  d_v]
 *   g, beta       [T_total, h_v]          g is the log-decay, alpha = exp(g)
 *   a, b          [T_total, h_v]          raw gate inputs
 *   A_log,dt_bias [h_v]
 *   states        [num_seqs, h_v, d_k, d_v]
 * Sequence n owns tokens cu_seqlens[n] .. cu_seqlens[n+1]-1 (host int32).
 * Value head h reads query/key head h / (h_v / h_qk): each q/k head serves a
 * run of consecutive value heads ([P4] `linear_attention_core`, inverse-GQA
 * branch; [P3] `gated_delta_graph`).
 *
 * Parity status: every function here is pinned by the CPU test suite
 * (tests/test_oracle_*.py) against brute force, closed forms, library
 * routines or values printed on [P1]; none is "parity unpinned".
 */
#ifndef GDN_ORACLE_H
#define GDN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Update-rule family of [P4] `UpdateRule` / [P1] `is_known_rule`. */
enum {
  GDNREF_RULE_LINEAR = 0,      /* S += k v^T                     */
  GDNREF_RULE_GATED = 1,       /* S = exp(g) S + k v^T           */
  GDNREF_RULE_DELTA = 2,       /* S += k (beta (v - S^T k))^T    */
  GDNREF_RULE_GATED_DELTA = 3  /* decay, then the delta update   */
};

/* Logistic function, evaluated so that exp never sees a large positive
 * argument ([P4] `la_sigmoid`). */
double gdnref_sigmoid(double x);

/* softplus(x) = log(1 + e^x) in the overflow-free form
 * max(x, 0) + log1p(exp(-|x|)) ([P4] `la_softplus`). */
double gdnref_softplus(double x);

/* Gate prologue ([P4] `linear_attention_core` fused decay/beta branch;
 * [P1] `linear_attention_gate_op`):
 *   g[r,h]    = -exp(A_log[h]) * softplus(a[r,h] + dt_bias[h])
 *   beta[r,h] = sigmoid(b[r,h])
 * for r < rows, h < h_v.  Either output pointer may be NULL. */
void gdnref_gates(int64_t rows, int32_t h_v, const double* a, const double* b,
                  const double* A_log, const double* dt_bias, double* g,
                  double* beta);

/* Serial scan over packed sequences.  For each sequence n and value head h,
 * starting from initial_state[n,h] (zeros if NULL), every token t runs
 *   decay     S <- exp(g[t,h]) S                       (gated rules)
 *   retrieval r  = S^T k_t                             (delta rules)
 *   delta     d  = beta[t,h] (v_t - r)  (delta rules; v_t otherwise)
 *   update    S <- S + k_t d^T
 *   readout   out[t,h] = scale * S^T q_t   on the updated S
 * ([P4] `linear_attention_core` steps 1-4; [P1] stable unroll; [P3]
 * `gated_delta_graph`).  scale == 0 selects 1/sqrt(d_k) ([P4]
 * `LinearAttentionFactory::create`).  g / beta may be NULL when the rule does
 * not use them.  final_state may be NULL.  A sequence with no tokens leaves
 * its final state equal to its initial state ([P1] zero-length time axis).
 *
 * Returns 0, or -1 on an invalid argument (nothing written). */
int gdnref_prefill(int32_t rule, int32_t h_qk, int32_t h_v, int32_t d_k,
                   int32_t d_v, double scale, int32_t num_seqs,
                   const int32_t* cu_seqlens, const double* q,
                   const double* k, const double* v, const double* g,
                   const double* beta, const double* initial_state,
                   double* out, double* final_state);

/* gdnref_prefill with the variants the pages define:
 *   decay_per_key  g is [T_total, h_v, d_k]: row i of the state decays by
 *                  exp(g[t,h,i]) ([P4] `linear_attention_core` per-key-dim
 *                  decay; [P1] per-head-per-key-dim decay form)
 *   beta_shared    beta is [T_total]: one write strength per token, shared by
 *                  all value heads ([P4] beta layout [B, T, 1])
 *   window > 0     history [num_seqs, window, h_v, d_k, d_v] receives the
 *                  state after each of the last `window` tokens of every
 *                  sequence, oldest first; slots before the first token are
 *                  zero ([P1] `state_window`; window = T gives [P3]
 *                  `gated_delta_steps`). */
int gdnref_prefill_ex(int32_t rule, int32_t h_qk, int32_t h_v, int32_t d_k,
                      int32_t d_v, double scale, int32_t num_seqs,
                      const int32_t* cu_seqlens, const double* q,
                      const double* k, const double* v, const double* g,
                      const double* beta, int32_t decay_per_key,
                      int32_t beta_shared, const double* initial_state,
                      double* out, double* final_state, int32_t window,
                      double* history);

/* One token per sequence, state read and written in place:
 * identical to gdnref_prefill with cu_seqlens = {0, 1, ..., batch}. */
int gdnref_decode_step(int32_t rule, int32_t h_qk, int32_t h_v, int32_t d_k,
                       int32_t d_v, double scale, int32_t batch,
                       const double* q, const double* k, const double* v,
                       const double* g, const double* beta, double* state,
                       double* out);

/* Causal depthwise conv1d with a carried state ([P1] `causal_conv_op`,
 * channels-last layout; [P3] `causal_conv1d_slots` fallback graph).  With
 * carry = (ksize - 1) * dilation and, for sequence n of length L, the padded
 * input xp(p) = initial_state[n, carry + p, c] for -carry <= p < 0 (zeros
 * without an initial state) and x[cu[n] + p, c] for 0 <= p < L:
 *     z = bias[c] + sum_j weight[c, j] * xp(t - carry + j * dilation)
 *     y[cu[n] + t, c] = silu ? z * sigmoid(z) : z
 *     final_state[n, i, c] = xp(L - carry + i),  0 <= i < carry.
 * Layouts: x, y [T_total, channels]; weight [channels, ksize]; bias
 * [channels] or NULL; states [num_seqs, carry, channels] (either may be
 * NULL).  Returns 0, or -1 on an invalid argument. */
int gdnref_causal_conv(int32_t channels, int32_t ksize, int32_t dilation, int32_t silu,
                       int32_t num_seqs, const int32_t* cu_seqlens, const double* x,
                       const double* weight, const double* bias,
                       const double* initial_state, double* y, double* final_state);

/* Gated RMSNorm ([P1] `gated_rms_norm_op`): each row of `width` elements is
 * split into width / group groups of `group` consecutive elements; per group
 *     y = x / sqrt(mean(x^2) + eps) * scale * act(gate)
 * with scale [group] and act = silu (activation 1: gate * sigmoid(gate)) or
 * sigmoid (activation 2).  x, gate, y are [rows, width].  Returns 0, or -1 on
 * an invalid argument. */
int gdnref_gated_rmsnorm(int64_t rows, int32_t width, int32_t group, const double* x,
                         const double* gate, const double* scale, double eps,
                         int32_t activation, double* y);

/* The convolution over a state pool ([P3] `causal_conv1d_slots`): pool
 * [num_slots, carry, C]; sequence n's state is pool[slots[n]], read and
 * replaced by its new state; a slot outside [0, num_slots) starts from zeros
 * and is not written back.  Returns 0, or -1 on an invalid argument. */
int gdnref_causal_conv_slots(int32_t channels, int32_t ksize, int32_t dilation, int32_t silu,
                             int32_t num_seqs, const int32_t* cu_seqlens, const double* x,
                             const double* weight, const double* bias, double* pool,
                             int32_t num_slots, const int32_t* slots, double* y);

/* Threads the parallel loop over independent (sequence, head) units uses. */
int gdnref_max_threads(void);

/* Sets that thread count (n > 0) for later calls. */
void gdnref_set_threads(int32_t n);

/* Bytes of the working precision of the state and its accumulations: 8 in
 * the reference build (double), 4 in the float32 baseline build of the same
 * source (-DGDNREF_ACC=float). */
int32_t gdnref_acc_bytes(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_ORACLE_H */
