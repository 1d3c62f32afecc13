/*
 * gdn_oracle.c -- reference (test-infrastructure) implementation of the gated
 * delta-rule recurrence.  Plain C, IEEE double, one serial scan per
 * (sequence, value head).  See gdn_oracle.h for layouts and sources.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark; never by the library's own path.
 */
#include "gdn_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Working precision of the recurrence's state and accumulations.  The
 * reference build keeps double; a second build of this same source with
 * -DGDNREF_ACC=float is the timed CPU baseline (float32 working state, as the
 * pages' kernels keep), and is itself held to the double build by the tests.
 * Inputs and outputs stay double arrays either way: each input value is the
 * widened I/O value, exact in float as well. */
#ifndef GDNREF_ACC
#define GDNREF_ACC double
#endif
typedef GDNREF_ACC acc_t;

/* [P4] `la_sigmoid`: two branches so that exp only sees arguments <= 0. */
double gdnref_sigmoid(double x) {
  if (x >= 0.0) return 1.0 / (1.0 + exp(-x));
  const double e = exp(x);
  return e / (1.0 + e);
}

/* [P4] `la_softplus`: log(1 + e^x) = max(x, 0) + log1p(e^{-|x|}). */
double gdnref_softplus(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }

/* [P4] fused decay branch of `linear_attention_core` (neg_exp_A times the
 * softplus of a + dt_bias, with neg_exp_A = -exp(A_log) folded in) and the
 * fused beta = sigmoid(b); [P1] `linear_attention_gate_op` computes the same
 * decay as softplus(a + bias) times a per-head scale.  No intermediate
 * rounding: everything stays in double. */
void gdnref_gates(int64_t rows, int32_t h_v, const double* a, const double* b,
                  const double* A_log, const double* dt_bias, double* g,
                  double* beta) {
  for (int64_t r = 0; r < rows; ++r) {
    for (int32_t h = 0; h < h_v; ++h) {
      const int64_t idx = r * h_v + h;
      if (g) g[idx] = -exp(A_log[h]) * gdnref_softplus(a[idx] + dt_bias[h]);
      if (beta) beta[idx] = gdnref_sigmoid(b[idx]);
    }
  }
}

static int rule_decays(int32_t rule) {
  return rule == GDNREF_RULE_GATED || rule == GDNREF_RULE_GATED_DELTA;
}
static int rule_deltas(int32_t rule) {
  return rule == GDNREF_RULE_DELTA || rule == GDNREF_RULE_GATED_DELTA;
}

/* Scan of one (sequence, value head) unit over tokens [t0, t1).
 * S is the d_k x d_v state, row i / column j at S[i*d_v + j]; it holds the
 * initial state on entry and the final state on return.  r and d are
 * d_v-long scratch vectors.
 *
 * The four steps and their order follow [P4] `linear_attention_core`
 * (step 1 decay, step 2 retrieval, step 3 delta update, step 4 readout of the
 * UPDATED state), which [P1]'s stable unroll and [P3] `gated_delta_graph`
 * also take. */
static void scan_unit(int32_t rule, int32_t h_qk, int32_t h_v, int32_t d_k,
                      int32_t d_v, double scale, int64_t t0, int64_t t1,
                      int32_t h, const double* q, const double* k,
                      const double* v, const double* g, const double* beta,
                      int32_t decay_per_key, int32_t beta_shared, int32_t window,
                      double* history, acc_t* S, acc_t* r, acc_t* d, double* out) {
  const int32_t hq = h / (h_v / h_qk); /* consecutive value heads share q/k */
  const int64_t state_elems = (int64_t)d_k * d_v;
  /* history slots before the first token stay zero ([P1] state_window) */
  for (int64_t w = 0; window > 0 && w < window - (t1 - t0); ++w)
    memset(history + (w * h_v + h) * state_elems, 0, sizeof(double) * (size_t)state_elems);
  for (int64_t t = t0; t < t1; ++t) {
    const double* kt = k + (t * h_qk + hq) * d_k;
    const double* qt = q + (t * h_qk + hq) * d_k;
    const double* vt = v + (t * h_v + h) * d_v;

    /* decay: S <- exp(g) S; per-key-dim decay scales row i by exp(g_i) */
    if (rule_decays(rule)) {
      if (decay_per_key) {
        const double* gt = g + (t * h_v + h) * d_k;
        for (int32_t i = 0; i < d_k; ++i) {
          const acc_t alpha_i = (acc_t)exp(gt[i]);
          for (int32_t j = 0; j < d_v; ++j) S[i * d_v + j] *= alpha_i;
        }
      } else {
        const acc_t alpha = (acc_t)exp(g[t * h_v + h]);
        for (int32_t i = 0; i < d_k; ++i)
          for (int32_t j = 0; j < d_v; ++j) S[i * d_v + j] *= alpha;
      }
    }

    /* retrieval r = S^T k and delta d = beta (v - r); plain rules use d = v */
    if (rule_deltas(rule)) {
      const acc_t bt = (acc_t)(beta_shared ? beta[t] : beta[t * h_v + h]);
      for (int32_t j = 0; j < d_v; ++j) {
        acc_t acc = 0;
        for (int32_t i = 0; i < d_k; ++i) acc += S[i * d_v + j] * (acc_t)kt[i];
        r[j] = acc;
      }
      for (int32_t j = 0; j < d_v; ++j) d[j] = bt * ((acc_t)vt[j] - r[j]);
    } else {
      for (int32_t j = 0; j < d_v; ++j) d[j] = (acc_t)vt[j];
    }

    /* rank-1 update S <- S + k d^T */
    for (int32_t i = 0; i < d_k; ++i)
      for (int32_t j = 0; j < d_v; ++j) S[i * d_v + j] += (acc_t)kt[i] * d[j];

    /* readout of the updated state: out = scale * S^T q */
    if (out) {
      double* ot = out + (t * h_v + h) * d_v;
      for (int32_t j = 0; j < d_v; ++j) {
        acc_t acc = 0;
        for (int32_t i = 0; i < d_k; ++i) acc += S[i * d_v + j] * (acc_t)qt[i];
        ot[j] = (double)((acc_t)scale * acc);
      }
    }

    /* state after this token, for the last `window` tokens */
    const int64_t w = (t - t0) - ((t1 - t0) - window);
    if (window > 0 && w >= 0) {
      double* hw = history + (w * h_v + h) * state_elems;
      for (int64_t e = 0; e < state_elems; ++e) hw[e] = (double)S[e];
    }
  }
}

static int valid_geometry(int32_t rule, int32_t h_qk, int32_t h_v, int32_t d_k,
                          int32_t d_v) {
  if (rule < GDNREF_RULE_LINEAR || rule > GDNREF_RULE_GATED_DELTA) return 0;
  if (h_qk <= 0 || h_v <= 0 || d_k <= 0 || d_v <= 0) return 0;
  if (h_v % h_qk != 0) return 0;
  return 1;
}

int gdnref_prefill_ex(int32_t rule, int32_t h_qk, int32_t h_v, int32_t d_k,
                      int32_t d_v, double scale, int32_t num_seqs,
                      const int32_t* cu_seqlens, const double* q,
                      const double* k, const double* v, const double* g,
                      const double* beta, int32_t decay_per_key,
                      int32_t beta_shared, const double* initial_state,
                      double* out, double* final_state, int32_t window,
                      double* history) {
  if (!valid_geometry(rule, h_qk, h_v, d_k, d_v) || num_seqs < 0) return -1;
  if (num_seqs > 0 && !cu_seqlens) return -1;
  if (rule_decays(rule) && !g && num_seqs > 0) return -1;
  if (rule_deltas(rule) && !beta && num_seqs > 0) return -1;
  if (window < 0 || (window > 0 && !history)) return -1;
  if (num_seqs > 0 && cu_seqlens[0] != 0) return -1;
  for (int32_t n = 0; n < num_seqs; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;

  if (scale == 0.0) scale = 1.0 / sqrt((double)d_k);
  const int64_t state_elems = (int64_t)d_k * d_v;
  const int64_t units = (int64_t)num_seqs * h_v;
  int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < units; ++u) {
    const int32_t n = (int32_t)(u / h_v);
    const int32_t h = (int32_t)(u % h_v);
    acc_t* S = (acc_t*)malloc(sizeof(acc_t) * (size_t)(state_elems + 2 * d_v));
    if (!S) {
#pragma omp atomic write
      failed = 1;
      continue;
    }
    acc_t* r = S + state_elems;
    acc_t* d = r + d_v;
    for (int64_t e = 0; e < state_elems; ++e)
      S[e] = initial_state ? (acc_t)initial_state[u * state_elems + e] : (acc_t)0;
    scan_unit(rule, h_qk, h_v, d_k, d_v, scale, cu_seqlens[n], cu_seqlens[n + 1], h,
              q, k, v, g, beta, decay_per_key, beta_shared, window,
              window > 0 ? history + (int64_t)n * window * h_v * state_elems : NULL, S, r, d, out);
    if (final_state)
      for (int64_t e = 0; e < state_elems; ++e) final_state[u * state_elems + e] = (double)S[e];
    free(S);
  }
  return failed ? -1 : 0;
}

int gdnref_prefill(int32_t rule, int32_t h_qk, int32_t h_v, int32_t d_k,
                   int32_t d_v, double scale, int32_t num_seqs,
                   const int32_t* cu_seqlens, const double* q,
                   const double* k, const double* v, const double* g,
                   const double* beta, const double* initial_state,
                   double* out, double* final_state) {
  return gdnref_prefill_ex(rule, h_qk, h_v, d_k, d_v, scale, num_seqs, cu_seqlens, q, k, v, g,
                           beta, 0, 0, initial_state, out, final_state, 0, NULL);
}

int gdnref_decode_step(int32_t rule, int32_t h_qk, int32_t h_v, int32_t d_k,
                       int32_t d_v, double scale, int32_t batch,
                       const double* q, const double* k, const double* v,
                       const double* g, const double* beta, double* state,
                       double* out) {
  if (batch < 0 || !state) return -1;
  int32_t* cu = (int32_t*)malloc(sizeof(int32_t) * (size_t)(batch + 1));
  if (!cu) return -1;
  for (int32_t n = 0; n <= batch; ++n) cu[n] = n;
  /* initial and final state are the same buffer: each unit copies its slice
   * in before scanning and back out after, so the in-place call is safe. */
  const int rc = gdnref_prefill(rule, h_qk, h_v, d_k, d_v, scale, batch, cu, q, k,
                                v, g, beta, state, out, state);
  free(cu);
  return rc;
}

/* [P1] `causal_conv_op`: the past state is concatenated in front of the
 * input along time, a depthwise conv1d (a cross-correlation: tap j meets
 * input position t - carry + j * dilation) runs over it, the bias is added
 * and silu applied; the present state is the last `carry` positions of the
 * padded input.  [P3]'s fallback graph does the same with a pool. */
int gdnref_causal_conv(int32_t channels, int32_t ksize, int32_t dilation, int32_t silu,
                       int32_t num_seqs, const int32_t* cu_seqlens, const double* x,
                       const double* weight, const double* bias,
                       const double* initial_state, double* y, double* final_state) {
  if (channels <= 0 || ksize <= 0 || dilation <= 0 || num_seqs < 0) return -1;
  if (num_seqs > 0 && (!cu_seqlens || cu_seqlens[0] != 0)) return -1;
  for (int32_t n = 0; n < num_seqs; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
  const int64_t carry = (int64_t)(ksize - 1) * dilation;
  for (int32_t n = 0; n < num_seqs; ++n) {
    const int64_t t0 = cu_seqlens[n];
    const int64_t L = cu_seqlens[n + 1] - t0;
    const double* s0 = initial_state ? initial_state + (int64_t)n * carry * channels : NULL;
    for (int32_t c = 0; c < channels; ++c) {
      /* padded input at position p, -carry <= p < L */
#define XP(p) ((p) < 0 ? (s0 ? s0[(carry + (p)) * channels + c] : 0.0) : x[(t0 + (p)) * channels + c])
      for (int64_t t = 0; t < L && y; ++t) {
        double z = bias ? bias[c] : 0.0;
        for (int32_t j = 0; j < ksize; ++j)
          z += weight[(int64_t)c * ksize + j] * XP(t - carry + (int64_t)j * dilation);
        y[(t0 + t) * channels + c] = silu ? z * gdnref_sigmoid(z) : z;
      }
      if (final_state) {
        double* fs = final_state + (int64_t)n * carry * channels;
        for (int64_t i = 0; i < carry; ++i) fs[i * channels + c] = XP(L - carry + i);
      }
#undef XP
    }
  }
  return 0;
}

/* [P3] `causal_conv1d_slots`: the states of the sequences are gathered from
 * the pool at their slots (pool[slots[n]]), the convolution above runs on
 * them, and each new state is scattered back to its slot.  A slot outside
 * [0, num_slots) is a padding sequence: a zero state, nothing written back. */
int gdnref_causal_conv_slots(int32_t channels, int32_t ksize, int32_t dilation, int32_t silu,
                             int32_t num_seqs, const int32_t* cu_seqlens, const double* x,
                             const double* weight, const double* bias, double* pool,
                             int32_t num_slots, const int32_t* slots, double* y) {
  if (num_seqs < 0 || num_slots < 0 || (num_seqs > 0 && !slots)) return -1;
  const int64_t carry = (int64_t)(ksize - 1) * dilation;
  const int64_t per = carry * channels;
  double* states = (double*)calloc((size_t)(num_seqs * per + 1), sizeof(double));
  double* fresh = (double*)calloc((size_t)(num_seqs * per + 1), sizeof(double));
  if (!states || !fresh) {
    free(states);
    free(fresh);
    return -1;
  }
  for (int32_t n = 0; n < num_seqs; ++n) {
    const int32_t s = slots[n];
    if (s >= 0 && s < num_slots)
      for (int64_t e = 0; e < per; ++e) states[n * per + e] = pool[(int64_t)s * per + e];
  }
  const int rc = gdnref_causal_conv(channels, ksize, dilation, silu, num_seqs, cu_seqlens, x, weight,
                                    bias, states, y, fresh);
  if (rc == 0)
    for (int32_t n = 0; n < num_seqs; ++n) {
      const int32_t s = slots[n];
      if (s >= 0 && s < num_slots)
        for (int64_t e = 0; e < per; ++e) pool[(int64_t)s * per + e] = fresh[n * per + e];
    }
  free(states);
  free(fresh);
  return rc;
}

/* [P1] `gated_rms_norm_op`: rows of `group` elements in float, mean of the
 * squares plus epsilon, reciprocal square root, times the scale, times the
 * gate's activation (silu by default, or sigmoid). */
int gdnref_gated_rmsnorm(int64_t rows, int32_t width, int32_t group, const double* x,
                         const double* gate, const double* scale, double eps,
                         int32_t activation, double* y) {
  if (rows < 0 || width <= 0 || group <= 0 || width % group != 0) return -1;
  if (activation != 1 && activation != 2) return -1;
  const int64_t groups = rows * (width / group);
  for (int64_t r = 0; r < groups; ++r) {
    const double* xr = x + r * group;
    const double* gr = gate + r * group;
    double ss = 0.0;
    for (int32_t i = 0; i < group; ++i) ss += xr[i] * xr[i];
    const double inv = 1.0 / sqrt(ss / group + eps);
    for (int32_t i = 0; i < group; ++i) {
      const double s = gdnref_sigmoid(gr[i]);
      const double act = activation == 1 ? gr[i] * s : s;
      y[r * group + i] = xr[i] * inv * scale[i] * act;
    }
  }
  return 0;
}

/* Threads the OpenMP loop over (sequence, head) units uses from now on. */
void gdnref_set_threads(int32_t n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* sizeof the working precision: 8 for the reference build, 4 for the
 * float32 baseline build. */
int32_t gdnref_acc_bytes(void) { return (int32_t)sizeof(acc_t); }

int gdnref_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
