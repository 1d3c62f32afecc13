// gdn_api.cpp -- the C ABI of libgdn (include/gdn.h): host-side validation,
// error reporting and dispatch to the HIP kernels.
//
// Validation mirrors what the pages' execute paths check before a launch
// ([P4] onnx-runtime-ep-cuda, src/kernels/linear_attention.rs,
// `LinearAttentionKernel::execute`: head divisibility, d_k range, gate
// presence and shape, contiguous uniform-dtype tensors; [P1]
// onnxruntime-ep-mlx, src/ops/ssm.rs, `linear_attention_op` geometry checks),
// restated for this ABI's packed layout.  Nothing is enqueued unless every
// check passes.
#include "gdn.h"

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "gdn_launch.hpp"

#define GDN_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_last_error[512] = "";

gdn_status fail(gdn_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

gdn_status ok() {
  g_last_error[0] = '\0';
  return GDN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool aligned_to(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// [a, a + na) and [b, b + nb) share a byte.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

size_t io_size(int32_t dtype) { return dtype == GDN_F32 ? 4 : 2; }
bool io_known(int32_t dtype) { return dtype == GDN_F32 || dtype == GDN_BF16 || dtype == GDN_F16; }
const char* io_name(int32_t dtype) { return dtype == GDN_F32 ? "f32" : dtype == GDN_BF16 ? "bf16" : "f16"; }

bool rule_decays(int32_t rule) { return rule == GDN_RULE_GATED_DELTA || rule == GDN_RULE_GATED; }
bool rule_deltas(int32_t rule) { return rule == GDN_RULE_GATED_DELTA || rule == GDN_RULE_DELTA; }

// Shared checks of the geometry and the gate inputs.  The per-token gate
// tensors are required only when there are tokens to read them for.
gdn_status check_problem(const gdn_problem* p, const char* fn, bool has_tokens) {
  if (!p) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: problem is NULL", fn);
  if (p->h_qk <= 0 || p->h_v <= 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: head counts must be positive (h_qk=%d, h_v=%d)", fn,
                p->h_qk, p->h_v);
  if (p->h_v % p->h_qk != 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: h_v=%d is not a multiple of h_qk=%d", fn, p->h_v, p->h_qk);
  if (p->d_k <= 0 || p->d_v <= 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: head sizes must be positive (d_k=%d, d_v=%d)", fn, p->d_k,
                p->d_v);
  if (p->d_k > GDN_MAX_HEAD_DIM || p->d_v > GDN_MAX_HEAD_DIM)
    return fail(GDN_ERR_UNSUPPORTED, "%s: head sizes above %d are not supported (d_k=%d, d_v=%d)", fn,
                GDN_MAX_HEAD_DIM, p->d_k, p->d_v);
  if (!io_known(p->io_dtype))
    return fail(GDN_ERR_UNSUPPORTED, "%s: io_dtype %d is not supported (GDN_F32, GDN_BF16, GDN_F16)", fn,
                p->io_dtype);
  if (!std::isfinite(p->scale)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: scale is not finite", fn);
  const size_t es = io_size(p->io_dtype);
  if (p->rule < GDN_RULE_GATED_DELTA || p->rule > GDN_RULE_LINEAR)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: unknown rule %d", fn, p->rule);
  if ((p->decay_per_key != 0 && p->decay_per_key != 1) || (p->beta_shared != 0 && p->beta_shared != 1))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: decay_per_key and beta_shared must be 0 or 1", fn);
  const bool decays = rule_decays(p->rule), deltas = rule_deltas(p->rule);
  if (p->gate_mode == GDN_GATES_PRECOMPUTED) {
    if (has_tokens && ((decays && !p->g) || (deltas && !p->beta)))
      return fail(GDN_ERR_INVALID_ARGUMENT, "%s: precomputed gates need g and beta", fn);
    if (!aligned_to(p->g, es) || !aligned_to(p->beta, es))
      return fail(GDN_ERR_INVALID_ARGUMENT, "%s: g / beta are not aligned to their element size", fn);
  } else if (p->gate_mode == GDN_GATES_RAW) {
    if (has_tokens && ((decays && (!p->a || !p->A_log || !p->dt_bias)) || (deltas && !p->b)))
      return fail(GDN_ERR_INVALID_ARGUMENT, "%s: raw gates need a, b, A_log and dt_bias", fn);
    if (!aligned_to(p->a, es) || !aligned_to(p->b, es) || !aligned_to(p->A_log, 4) ||
        !aligned_to(p->dt_bias, 4))
      return fail(GDN_ERR_INVALID_ARGUMENT, "%s: gate inputs are not aligned to their element size", fn);
  } else {
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: unknown gate_mode %d", fn, p->gate_mode);
  }
  // a per-key-dim decay is read in row slices like k: 16-byte alignment
  if (p->decay_per_key && !aligned16(p->gate_mode == GDN_GATES_RAW ? p->a : p->g))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: a per-key-dim decay tensor must be 16-byte aligned", fn);
  if (p->algorithm != GDN_ALGO_AUTO && p->algorithm != GDN_ALGO_SERIAL && p->algorithm != GDN_ALGO_CHUNKED)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: unknown algorithm %d", fn, p->algorithm);
  if (p->norm_gate != nullptr) {
    if (!p->norm_scale) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: the output norm needs norm_scale", fn);
    if (!aligned16(p->norm_gate) || !aligned16(p->norm_scale))
      return fail(GDN_ERR_INVALID_ARGUMENT, "%s: norm_gate and norm_scale must be 16-byte aligned", fn);
    if (!(p->norm_eps >= 0.0f) || !std::isfinite(p->norm_eps))
      return fail(GDN_ERR_INVALID_ARGUMENT, "%s: norm_eps must be finite and >= 0", fn);
    if (p->norm_activation != GDN_ACT_SILU && p->norm_activation != GDN_ACT_SIGMOID)
      return fail(GDN_ERR_INVALID_ARGUMENT, "%s: norm_activation %d is not GDN_ACT_SILU or GDN_ACT_SIGMOID", fn,
                  p->norm_activation);
    if (!gdn::gated_rmsnorm_supported(p->io_dtype, p->d_v))
      return fail(GDN_ERR_UNSUPPORTED, "%s: the output norm does not serve d_v=%d", fn, p->d_v);
  }
  return GDN_OK;
}

gdn::NormEpilogue norm_epilogue(const gdn_problem* p) {
  gdn::NormEpilogue n{};
  n.gate = p->norm_gate;
  n.scale = p->norm_scale;
  n.eps = p->norm_eps;
  n.inv_n = 1.0f / static_cast<float>(p->d_v);
  n.silu = p->norm_activation == GDN_ACT_SILU ? 1 : 0;
  return n;
}

// The output norm as its own pass over out, in place: rows x h_v groups of d_v.
gdn_status norm_pass(const gdn_problem* p, int64_t rows, void* out, const char* fn, hipStream_t stream) {
  if (rows == 0 || out == nullptr) return GDN_OK;
  gdn::NormParams np{};
  np.x = out;
  np.gate = p->norm_gate;
  np.scale = p->norm_scale;
  np.y = out;
  np.groups = rows * p->h_v;
  np.group = p->d_v;
  np.eps = p->norm_eps;
  np.activation = p->norm_activation;
  const hipError_t e = gdn::launch_gated_rmsnorm(np, p->io_dtype, stream);
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "%s: norm launch failed: %s", fn, hipGetErrorString(e));
  return GDN_OK;
}

gdn::GateArgs gate_args(const gdn_problem* p) {
  gdn::GateArgs g{};
  g.raw = p->gate_mode == GDN_GATES_RAW ? 1 : 0;
  g.decays = rule_decays(p->rule) ? 1 : 0;
  g.deltas = rule_deltas(p->rule) ? 1 : 0;
  g.per_key = p->decay_per_key;
  g.beta_shared = p->beta_shared;
  g.g = p->g;
  g.beta = p->beta;
  g.a = p->a;
  g.b = p->b;
  g.A_log = p->A_log;
  g.dt_bias = p->dt_bias;
  return g;
}

float resolved_scale(const gdn_problem* p) {
  return p->scale != 0.0f ? p->scale : 1.0f / std::sqrt(static_cast<float>(p->d_k));
}

// Slot-pool arguments shared by the *_slots entry points.
struct SlotArgs {
  const int32_t* slots = nullptr;       // device [n] or null (no pool)
  const int32_t* slots_host = nullptr;  // optional host copy
  int32_t num_slots = 0;
};

// Slots in [0, num_slots) must be distinct (each names one sequence's state);
// anything else marks a padding sequence.  Checked through the host copy.
gdn_status check_slots(const SlotArgs& sl, int32_t n, const char* fn) {
  if (sl.num_slots < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: num_slots=%d is negative", fn, sl.num_slots);
  if (n > 0 && !sl.slots) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: slots is NULL", fn);
  if (!aligned_to(sl.slots, 4)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: slots is misaligned", fn);
  if (sl.slots_host && sl.num_slots > 0) {
    std::vector<int32_t> owner(static_cast<size_t>(sl.num_slots), -1);
    for (int32_t i = 0; i < n; ++i) {
      const int32_t sidx = sl.slots_host[i];
      if (sidx < 0 || sidx >= sl.num_slots) continue;  // padding
      if (owner[static_cast<size_t>(sidx)] >= 0)
        return fail(GDN_ERR_INVALID_ARGUMENT, "%s: slot %d is used by sequences %d and %d", fn, sidx,
                    owner[static_cast<size_t>(sidx)], i);
      owner[static_cast<size_t>(sidx)] = i;
    }
  }
  return GDN_OK;
}

// The prefill formulation a call takes, and the state columns one workgroup
// (serial: one wave) of its sequential kernel owns.  The single place where
// GDN_ALGO_AUTO is resolved: gdn_prefill and gdn_prefill_query_plan both ask it.
struct Plan {
  int form = GDN_FORM_SERIAL;
  int cols = 1;
  int norm = 0;  // 0 none, 1 fused into the output store, 2 a separate in-place pass
};

gdn::ScanParams plan_params(const gdn_problem& p, int32_t num_seqs, int32_t total_tokens) {
  gdn::ScanParams sp{};
  sp.gates = gate_args(&p);
  sp.num_seqs = num_seqs;
  sp.total_tokens = total_tokens;
  sp.h_qk = p.h_qk;
  sp.h_v = p.h_v;
  sp.d_k = p.d_k;
  sp.d_v = p.d_v;
  sp.ratio = p.h_v / p.h_qk;
  sp.window = p.state_window;
  return sp;
}

gdn_status plan_prefill(const gdn_problem& p, int32_t num_seqs, int32_t total_tokens, const char* fn, Plan* plan) {
  const gdn::ScanParams sp = plan_params(p, num_seqs, total_tokens);
  const int window = p.state_window;
  const int io_bf16 = p.io_dtype == GDN_BF16;
  // float32 I/O: the chunked form exists in two passes only, through a workspace
  const bool wide_ok = gdn::wide_supported(p.io_dtype, p.d_k, p.d_v, sp.gates, window);
  const bool wide_ws = wide_ok && p.workspace != nullptr &&
                       p.workspace_bytes >= gdn::wide_workspace_bytes(num_seqs, total_tokens, p.h_v, p.d_k, p.d_v);
  // bfloat16 I/O in two passes: any rule (the gated and linear rules only there)
  const bool split_ok = gdn::split_supported(io_bf16, p.d_k, p.d_v, sp.gates, window);
  const bool split_ws = split_ok && p.workspace != nullptr &&
                        p.workspace_bytes >= gdn::split_workspace_bytes(num_seqs, total_tokens, p.h_v, p.d_k, p.d_v,
                                                                        sp.gates.deltas != 0);
  const bool can_chunk = gdn::chunked_supported(io_bf16, p.d_k, p.d_v, sp.gates, window) || wide_ws || split_ws;
  if (p.algorithm == GDN_ALGO_CHUNKED && !can_chunk)
    return fail(GDN_ERR_UNSUPPORTED,
                "%s: the chunked algorithm needs bfloat16 I/O with d_k 64 or 128 and d_v a multiple of 8, or "
                "float32 I/O with d_k 128 or 256, d_v a multiple of 16 up to 256 and a workspace; and a per-head "
                "decay and no state history (got %s, d_k=%d, d_v=%d, rule=%d, "
                "decay_per_key=%d, state_window=%d%s)",
                fn, io_name(p.io_dtype), p.d_k, p.d_v, p.rule, p.decay_per_key, window,
                (wide_ok && !wide_ws) || (split_ok && !split_ws) ? ", no or too small a workspace" : "");
  const bool chunked = p.algorithm == GDN_ALGO_CHUNKED ||
                       (p.algorithm == GDN_ALGO_AUTO && can_chunk && (!wide_ws || gdn::wide_auto(p.d_k)) &&
                        static_cast<int64_t>(total_tokens) >= 64 * static_cast<int64_t>(num_seqs));
  const bool wide = chunked && wide_ws;
  // the two-pass chunked form when the caller's workspace holds it
  const bool split = chunked && !wide && split_ws;
  const bool norm = p.norm_gate != nullptr;
  plan->norm = norm ? 2 : 0;
  if (wide) {
    plan->form = GDN_FORM_CHUNKED_F32;
    plan->cols = 16;
  } else if (split) {
    plan->form = GDN_FORM_CHUNKED_TWO_PASS;
    if (norm && gdn::split_fuses_norm(p.d_v, num_seqs * p.h_v)) {
      plan->cols = 128;
      plan->norm = 1;
    } else {
      plan->cols = gdn::split_takes_rows_kernel(p.d_k, p.d_v, num_seqs * p.h_v, sp.gates.deltas != 0)
                       ? 16
                       : gdn::split_columns_per_block(p.d_v, num_seqs * p.h_v);
    }
  } else if (chunked) {
    plan->form = GDN_FORM_CHUNKED_ONE_PASS;
    plan->cols = gdn::chunked_columns_per_block(p.d_k, p.d_v);
  } else {
    plan->form = GDN_FORM_SERIAL;
    plan->cols = gdn::scan_columns_per_wave(sp);
  }
  return GDN_OK;
}

// The column-block state pass holds two workgroups per compute unit, and the
// two halves of its grid fill the two slots.  A sequence takes its chunk count
// times the time of a chunk, which is longer while its compute unit is shared.
// Ordering the sequences so that the first half of the positions takes the
// longest ones (longest first) and the second half the rest (shortest first)
// pairs a long sequence with a short one, which leaves it alone sooner (8
// packed sequences of 43 to 107 chunks: the state pass 376 -> 364 us).
// Sequences of one length keep the identity order.  Any order is correct:
// each workgroup carries one sequence's state from its first chunk to its last.
void order_sequences(const int32_t* cu, int32_t num_seqs, gdn::ScanParams* sp) {
  if (num_seqs < 2 || num_seqs > static_cast<int32_t>(sizeof(sp->seq_order))) return;
  int chunks[sizeof(sp->seq_order)];
  bool one_length = true;
  for (int n = 0; n < num_seqs; ++n) {
    chunks[n] = (cu[n + 1] - cu[n] + 63) / 64;
    one_length = one_length && chunks[n] == chunks[0];
  }
  if (one_length) return;
  const int half = (num_seqs + 1) / 2;
  for (int n = 0; n < num_seqs; ++n) {
    int rank = 0;  // by chunk count, longest first, ties by index: a permutation
    for (int m = 0; m < num_seqs; ++m) rank += (chunks[m] > chunks[n] || (chunks[m] == chunks[n] && m < n)) ? 1 : 0;
    sp->seq_order[rank < half ? rank : num_seqs - 1 - (rank - half)] = static_cast<uint8_t>(n);
  }
  sp->num_ordered = num_seqs;
}

gdn_status prefill_impl(const char* fn, const gdn_problem* problem, int32_t num_seqs, const int32_t* cu_seqlens,
                        const int32_t* cu_seqlens_host, int32_t total_tokens, const void* q, const void* k,
                        const void* v, const float* initial_state, void* out, float* final_state,
                        const SlotArgs* pool, hipStream_t stream) {
  gdn_status st = check_problem(problem, fn, total_tokens > 0);
  if (st != GDN_OK) return st;
  if (num_seqs < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: num_seqs=%d is negative", fn, num_seqs);
  if (total_tokens < 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: total_tokens=%d is negative", fn, total_tokens);
  if (num_seqs == 0 && total_tokens != 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: %d tokens but no sequences", fn, total_tokens);
  if (num_seqs > 0 && !cu_seqlens) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: cu_seqlens is NULL", fn);
  if (total_tokens > 0 && (!q || !k || !v))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: q, k and v are required when total_tokens > 0", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(initial_state) ||
      !aligned16(final_state))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: q, k, v, out and the states must be 16-byte aligned", fn);
  if (!aligned_to(cu_seqlens, 4)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: cu_seqlens is misaligned", fn);
  if (problem->state_window < 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: state_window=%d is negative", fn, problem->state_window);
  if (problem->state_window > 0 && num_seqs > 0 && !problem->state_history)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: state_window > 0 needs state_history", fn);
  if (!aligned16(problem->state_history))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: state_history must be 16-byte aligned", fn);
  if (!aligned16(problem->workspace))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: workspace must be 16-byte aligned", fn);
  if (cu_seqlens_host) {
    if (cu_seqlens_host[0] != 0)
      return fail(GDN_ERR_INVALID_ARGUMENT, "%s: cu_seqlens[0]=%d, expected 0", fn, cu_seqlens_host[0]);
    for (int32_t n = 0; n < num_seqs; ++n)
      if (cu_seqlens_host[n + 1] < cu_seqlens_host[n])
        return fail(GDN_ERR_INVALID_ARGUMENT, "%s: cu_seqlens decreases at %d (%d -> %d)", fn, n,
                    cu_seqlens_host[n], cu_seqlens_host[n + 1]);
    if (cu_seqlens_host[num_seqs] != total_tokens)
      return fail(GDN_ERR_INVALID_ARGUMENT, "%s: cu_seqlens[%d]=%d but total_tokens=%d", fn, num_seqs,
                  cu_seqlens_host[num_seqs], total_tokens);
  }
  const gdn_problem& p = *problem;
  if (pool) {
    st = check_slots(*pool, num_seqs, fn);
    if (st != GDN_OK) return st;
  }
  const size_t es = io_size(p.io_dtype);
  const int64_t state_count = pool ? pool->num_slots : num_seqs;
  const size_t state_bytes = static_cast<size_t>(state_count) * p.h_v * p.d_k * p.d_v * sizeof(float);
  const size_t out_bytes = static_cast<size_t>(total_tokens) * p.h_v * p.d_v * es;
  if (final_state && initial_state && final_state != initial_state &&
      overlaps(final_state, state_bytes, initial_state, state_bytes))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: final_state partially overlaps initial_state", fn);
  const size_t qk_bytes = static_cast<size_t>(total_tokens) * p.h_qk * p.d_k * es;
  const size_t v_bytes = static_cast<size_t>(total_tokens) * p.h_v * p.d_v * es;
  if (overlaps(out, out_bytes, q, qk_bytes) || overlaps(out, out_bytes, k, qk_bytes) ||
      overlaps(out, out_bytes, v, v_bytes) || overlaps(out, out_bytes, final_state, state_bytes))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: out overlaps an input or the final state", fn);
  if (overlaps(p.norm_gate, out_bytes, out, out_bytes) || overlaps(p.norm_scale, p.d_v * es, out, out_bytes))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: out overlaps norm_gate or norm_scale", fn);
  const int32_t window = problem->state_window;
  const size_t hist_bytes = static_cast<size_t>(num_seqs) * window * p.h_v * p.d_k * p.d_v * sizeof(float);
  if (window > 0 && (overlaps(problem->state_history, hist_bytes, out, out_bytes) ||
                     overlaps(problem->state_history, hist_bytes, final_state, state_bytes) ||
                     overlaps(problem->state_history, hist_bytes, initial_state, state_bytes)))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: state_history overlaps out or a state", fn);

  if (num_seqs == 0 || (total_tokens == 0 && !final_state && window == 0)) return ok();  // nothing to write

  gdn::ScanParams sp{};
  sp.q = q;
  sp.k = k;
  sp.v = v;
  sp.gates = gate_args(problem);
  sp.s0 = initial_state;
  sp.out = out;
  sp.sN = final_state;
  sp.cu = cu_seqlens;
  sp.slots = pool ? pool->slots : nullptr;
  sp.num_slots = pool ? pool->num_slots : 0;
  sp.num_seqs = num_seqs;
  sp.total_tokens = total_tokens;
  sp.h_qk = p.h_qk;
  sp.h_v = p.h_v;
  sp.d_k = p.d_k;
  sp.d_v = p.d_v;
  sp.ratio = p.h_v / p.h_qk;
  sp.scale = resolved_scale(problem);
  const int io_bf16 = p.io_dtype == GDN_BF16;
  sp.window = window;
  sp.history = window > 0 ? problem->state_history : nullptr;
  Plan plan;
  st = plan_prefill(p, num_seqs, total_tokens, fn, &plan);
  if (st != GDN_OK) return st;
  sp.col_blocks = (p.d_v + plan.cols - 1) / plan.cols;
  const uint64_t blocks = static_cast<uint64_t>(num_seqs) * p.h_v * sp.col_blocks;
  if (blocks > 0x7fffffffull)
    return fail(GDN_ERR_UNSUPPORTED, "%s: %llu workgroups exceed the grid limit", fn,
                static_cast<unsigned long long>(blocks));
  const bool wide = plan.form == GDN_FORM_CHUNKED_F32, split = plan.form == GDN_FORM_CHUNKED_TWO_PASS,
             chunked = plan.form == GDN_FORM_CHUNKED_ONE_PASS;
  if (plan.norm == 1) sp.norm = norm_epilogue(problem);
  if (split && cu_seqlens_host) order_sequences(cu_seqlens_host, num_seqs, &sp);
  const hipError_t e = wide      ? gdn::launch_prefill_wide(sp, p.workspace, stream)
                       : split   ? gdn::launch_prefill_split(sp, p.workspace, stream)
                       : chunked ? gdn::launch_prefill_chunked(sp, io_bf16, stream)
                                 : gdn::launch_prefill_scan(sp, p.io_dtype, stream);
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  if (plan.norm == 2) {
    st = norm_pass(problem, total_tokens, out, fn, stream);
    if (st != GDN_OK) return st;
  }
  return ok();
}

}  // namespace

GDN_EXPORT gdn_status gdn_prefill(const gdn_problem* problem, int32_t num_seqs, const int32_t* cu_seqlens,
                                  const int32_t* cu_seqlens_host, int32_t total_tokens, const void* q,
                                  const void* k, const void* v, const float* initial_state, void* out,
                                  float* final_state, hipStream_t stream) {
  return prefill_impl("gdn_prefill", problem, num_seqs, cu_seqlens, cu_seqlens_host, total_tokens, q, k, v,
                      initial_state, out, final_state, nullptr, stream);
}

GDN_EXPORT gdn_status gdn_prefill_slots(const gdn_problem* problem, int32_t num_seqs, const int32_t* cu_seqlens,
                                        const int32_t* cu_seqlens_host, int32_t total_tokens, const void* q,
                                        const void* k, const void* v, float* state_pool, int32_t num_slots,
                                        const int32_t* slots, const int32_t* slots_host, void* out,
                                        hipStream_t stream) {
  const char* fn = "gdn_prefill_slots";
  if (num_slots > 0 && !state_pool) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: state_pool is NULL", fn);
  SlotArgs sl;
  sl.slots = slots;
  sl.slots_host = slots_host;
  sl.num_slots = num_slots;
  return prefill_impl(fn, problem, num_seqs, cu_seqlens, cu_seqlens_host, total_tokens, q, k, v, state_pool, out,
                      state_pool, &sl, stream);
}

namespace {

// conv: the conv prologue (its x, states, taps and channels already checked
// by the caller; then q, k and v are NULL), or NULL.
gdn_status decode_impl(const char* fn, const gdn_problem* problem, int32_t batch, const void* q, const void* k,
                       const void* v, float* state, void* out, const SlotArgs* pool, hipStream_t stream,
                       const gdn::ConvPrologue* conv = nullptr) {
  gdn_status st = check_problem(problem, fn, batch > 0);
  if (st != GDN_OK) return st;
  if (batch < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: batch=%d is negative", fn, batch);
  if (batch == 0) return ok();
  if (pool) {
    st = check_slots(*pool, batch, fn);
    if (st != GDN_OK) return st;
  }
  // an empty pool (every sequence padding) needs no state buffer
  const bool needs_state = !(pool && pool->num_slots == 0);
  if (conv) {
    if (!out || !state) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: state and out are required", fn);
  } else if (!q || !k || !v || !out || (needs_state && !state)) {
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: q, k, v, state and out are required", fn);
  }
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(state) || !aligned16(out))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: q, k, v, state and out must be 16-byte aligned", fn);
  const gdn_problem& p = *problem;
  const size_t es = io_size(p.io_dtype);
  const int64_t state_count = pool ? pool->num_slots : batch;
  const size_t state_bytes = static_cast<size_t>(state_count) * p.h_v * p.d_k * p.d_v * sizeof(float);
  const size_t out_bytes = static_cast<size_t>(batch) * p.h_v * p.d_v * es;
  const size_t qk_bytes = static_cast<size_t>(batch) * p.h_qk * p.d_k * es;
  const size_t v_bytes = static_cast<size_t>(batch) * p.h_v * p.d_v * es;
  if (conv) {
    // every buffer the conv prologue reads or writes against out and the state
    const size_t x_bytes = static_cast<size_t>(batch) * conv->channels * es;
    const size_t cs_bytes = static_cast<size_t>(batch) * (conv->ksize - 1) * conv->channels * es;
    const size_t w_bytes = static_cast<size_t>(conv->channels) * conv->ksize * es;
    const size_t b_bytes = static_cast<size_t>(conv->channels) * es;
    const void* ins[4] = {conv->x, conv->state, conv->weight, conv->bias};
    const size_t in_bytes[4] = {x_bytes, cs_bytes, w_bytes, b_bytes};
    for (int i = 0; i < 4; ++i) {
      if (overlaps(out, out_bytes, ins[i], in_bytes[i]) || overlaps(state, state_bytes, ins[i], in_bytes[i]) ||
          overlaps(conv->state_out, cs_bytes, ins[i], in_bytes[i]))
        return fail(GDN_ERR_INVALID_ARGUMENT,
                    "%s: out, state and conv_state_out must not overlap x, conv_state, weight or bias", fn);
    }
    if (overlaps(conv->state_out, cs_bytes, out, out_bytes) || overlaps(conv->state_out, cs_bytes, state, state_bytes))
      return fail(GDN_ERR_INVALID_ARGUMENT, "%s: conv_state_out overlaps out or the state", fn);
  }
  if (overlaps(out, out_bytes, state, state_bytes) || overlaps(out, out_bytes, q, qk_bytes) ||
      overlaps(out, out_bytes, k, qk_bytes) || overlaps(out, out_bytes, v, v_bytes))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: out overlaps the state or an input", fn);
  if (overlaps(state, state_bytes, q, qk_bytes) || overlaps(state, state_bytes, k, qk_bytes) ||
      overlaps(state, state_bytes, v, v_bytes))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: state overlaps an input", fn);

  gdn::DecodeParams dp{};
  dp.q = q;
  dp.k = k;
  dp.v = v;
  dp.gates = gate_args(problem);
  dp.state = state;
  dp.out = out;
  dp.slots = pool ? pool->slots : nullptr;
  dp.num_slots = pool ? pool->num_slots : 0;
  dp.batch = batch;
  dp.h_qk = p.h_qk;
  dp.h_v = p.h_v;
  dp.d_k = p.d_k;
  dp.d_v = p.d_v;
  dp.ratio = p.h_v / p.h_qk;
  const bool per_key = dp.gates.per_key && dp.gates.decays;
  const int cpb = gdn::decode_columns_per_block(p.d_k, p.d_v, per_key);
  dp.col_blocks = (p.d_v + cpb - 1) / cpb;
  dp.scale = resolved_scale(problem);
  if (conv) {
    if (!gdn::decode_takes_conv(p.d_k, p.d_v, per_key))
      return fail(GDN_ERR_UNSUPPORTED,
                  "%s: the conv prologue serves d_k in {16, 32, 64, 128, 256}, d_v a multiple of %d and a "
                  "per-head decay (d_k=%d, d_v=%d%s); run gdn_causal_conv_step, then gdn_decode_step",
                  fn, cpb, p.d_k, p.d_v, per_key ? ", per-key decay" : "");
    dp.conv = *conv;
  }
  if (p.h_v > 65535)
    return fail(GDN_ERR_UNSUPPORTED, "%s: h_v = %d exceeds the grid's head axis (65535)", fn, p.h_v);
  if (overlaps(p.norm_gate, out_bytes, out, out_bytes) || overlaps(p.norm_scale, p.d_v * es, out, out_bytes))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: out overlaps norm_gate or norm_scale", fn);
  const bool norm = p.norm_gate != nullptr;
  const bool fused = norm && gdn::decode_fuses_norm(p.d_k, p.d_v, per_key);
  if (fused) dp.norm = norm_epilogue(problem);
  const hipError_t e = gdn::launch_decode_step(dp, p.io_dtype, stream);
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  if (norm && !fused) {
    st = norm_pass(problem, batch, out, fn, stream);
    if (st != GDN_OK) return st;
  }
  return ok();
}

}  // namespace

GDN_EXPORT gdn_status gdn_prefill_workspace_size(const gdn_problem* problem, int32_t num_seqs, int32_t total_tokens,
                                                 uint64_t* bytes) {
  const char* fn = "gdn_prefill_workspace_size";
  if (!bytes) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: bytes is NULL", fn);
  *bytes = 0;
  gdn_status st = check_problem(problem, fn, false);
  if (st != GDN_OK) return st;
  if (num_seqs < 0 || total_tokens < 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: num_seqs=%d and total_tokens=%d must be >= 0", fn, num_seqs,
                total_tokens);
  const gdn_problem& p = *problem;
  if (p.algorithm == GDN_ALGO_SERIAL) return ok();
  const gdn::GateArgs gates = gate_args(problem);
  if (gdn::wide_supported(p.io_dtype, p.d_k, p.d_v, gates, p.state_window)) {
    if (p.algorithm == GDN_ALGO_CHUNKED || gdn::wide_auto(p.d_k))
      *bytes = gdn::wide_workspace_bytes(num_seqs, total_tokens, p.h_v, p.d_k, p.d_v);
    return ok();
  }
  if (!gdn::split_supported(p.io_dtype == GDN_BF16, p.d_k, p.d_v, gates, p.state_window)) return ok();
  *bytes = gdn::split_workspace_bytes(num_seqs, total_tokens, p.h_v, p.d_k, p.d_v, gates.deltas != 0);
  return ok();
}

GDN_EXPORT gdn_status gdn_prefill_static_workspace(const gdn_problem* problem, int32_t num_seqs,
                                                   const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                                   int32_t total_tokens, const void* q, const void* k, const void* v,
                                                   const float* initial_state, void* out, float* final_state,
                                                   hipStream_t stream) {
  const char* fn = "gdn_prefill_static_workspace";
  gdn_status st = check_problem(problem, fn, total_tokens > 0);
  if (st != GDN_OK) return st;
  if (problem->workspace != nullptr || problem->workspace_bytes != 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: takes no workspace (the library's own is used)", fn);
  uint64_t need = 0;
  st = gdn_prefill_workspace_size(problem, num_seqs, total_tokens, &need);
  if (st != GDN_OK) return fail(st, "%s: %s", fn, g_last_error);
  if (need > GDN_STATIC_WORKSPACE_BYTES)
    return fail(GDN_ERR_UNSUPPORTED,
                "%s: %d sequences of %d tokens in all need %llu bytes of workspace, above the %llu bytes this "
                "entry point holds; call gdn_prefill with a workspace of gdn_prefill_workspace_size bytes, or "
                "fewer tokens per call",
                fn, num_seqs, total_tokens, static_cast<unsigned long long>(need),
                static_cast<unsigned long long>(GDN_STATIC_WORKSPACE_BYTES));
  if (need == 0)  // a form without a workspace: nothing to lend
    return prefill_impl(fn, problem, num_seqs, cu_seqlens, cu_seqlens_host, total_tokens, q, k, v, initial_state,
                        out, final_state, nullptr, stream);
  void* ws = nullptr;
  size_t ws_bytes = 0;
  const hipError_t e = gdn::static_workspace(&ws, &ws_bytes);
  if (e != hipSuccess)
    return fail(GDN_ERR_HIP, "%s: the static workspace's device address: %s", fn, hipGetErrorString(e));
  gdn_problem p = *problem;
  p.workspace = ws;
  p.workspace_bytes = ws_bytes;
  return prefill_impl(fn, &p, num_seqs, cu_seqlens, cu_seqlens_host, total_tokens, q, k, v, initial_state, out,
                      final_state, nullptr, stream);
}

GDN_EXPORT gdn_status gdn_prefill_query_plan(const gdn_problem* problem, int32_t num_seqs, int32_t total_tokens,
                                             gdn_prefill_plan* plan) {
  const char* fn = "gdn_prefill_query_plan";
  if (!plan) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: plan is NULL", fn);
  *plan = gdn_prefill_plan{};
  gdn_status st = check_problem(problem, fn, false);
  if (st != GDN_OK) return st;
  if (num_seqs < 0 || total_tokens < 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: num_seqs=%d and total_tokens=%d must be >= 0", fn, num_seqs,
                total_tokens);
  const gdn_problem& p = *problem;
  if (num_seqs == 0) {
    plan->form = GDN_FORM_NONE;
    return ok();
  }
  Plan pl;
  st = plan_prefill(p, num_seqs, total_tokens, fn, &pl);
  if (st != GDN_OK) return st;
  plan->form = pl.form;
  plan->columns_per_block = pl.cols;
  plan->norm = pl.norm;
  const int units = num_seqs * p.h_v;
  const int units8 = (units + 7) / 8 * 8;
  char* k = plan->kernels;
  const size_t kn = sizeof(plan->kernels);
  switch (pl.form) {
    case GDN_FORM_SERIAL: {
      const gdn::ScanParams sp = plan_params(p, num_seqs, total_tokens);
      const bool lean = gdn::scan_takes_plain_kernel(sp);
      const int blocks = (p.d_v + pl.cols - 1) / pl.cols;
      plan->state_workgroups = (lean ? units8 : units) * blocks;
      std::snprintf(k, kn, "%s", lean ? "scan_plain_kernel" : "scan_kernel");
      break;
    }
    case GDN_FORM_CHUNKED_ONE_PASS:
      plan->state_workgroups = units * ((p.d_v + pl.cols - 1) / pl.cols);
      std::snprintf(k, kn, "chunk_kernel");
      break;
    case GDN_FORM_CHUNKED_TWO_PASS:
      if (pl.norm == 1) {
        plan->state_workgroups = units8;
        std::snprintf(k, kn, "chunk_table_kernel + chunk_trec_kernel + chunk_state_kernel (gated RMSNorm fused)");
      } else if (gdn::split_takes_rows_kernel(p.d_k, p.d_v, units, gate_args(problem).deltas != 0)) {
        plan->state_workgroups = units8 * ((p.d_v + 15) / 16);
        std::snprintf(k, kn, "chunk_table_kernel + chunk_prep_kernel + chunk_rows_kernel");
      } else {
        plan->state_workgroups = units8 * ((p.d_v + pl.cols - 1) / pl.cols);
        std::snprintf(k, kn, "chunk_table_kernel + chunk_trec_kernel + chunk_state_kernel");
      }
      break;
    case GDN_FORM_CHUNKED_F32:
      plan->state_workgroups = units8 * (p.d_v / 16);
      std::snprintf(k, kn, "chunk_table_kernel + wide_prep_kernel + wide_state_kernel");
      break;
    default:
      break;
  }
  if (pl.norm == 2) {
    const size_t len = std::strlen(k);
    std::snprintf(k + len, kn - len, " + rmsnorm_kernel");
  }
  return ok();
}

GDN_EXPORT gdn_status gdn_decode_step(const gdn_problem* problem, int32_t batch, const void* q, const void* k,
                                      const void* v, float* state, void* out, hipStream_t stream) {
  return decode_impl("gdn_decode_step", problem, batch, q, k, v, state, out, nullptr, stream);
}

GDN_EXPORT gdn_status gdn_decode_step_slots(const gdn_problem* problem, int32_t batch, const void* q,
                                            const void* k, const void* v, float* state_pool, int32_t num_slots,
                                            const int32_t* slots, const int32_t* slots_host, void* out,
                                            hipStream_t stream) {
  const char* fn = "gdn_decode_step_slots";
  if (num_slots > 0 && !state_pool) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: state_pool is NULL", fn);
  SlotArgs sl;
  sl.slots = slots;
  sl.slots_host = slots_host;
  sl.num_slots = num_slots;
  return decode_impl(fn, problem, batch, q, k, v, num_slots > 0 ? state_pool : nullptr, out, &sl, stream);
}

GDN_EXPORT gdn_status gdn_gate_prologue(int32_t tokens, int32_t h_v, int32_t io_dtype, const void* a,
                                        const void* b, const float* A_log, const float* dt_bias, void* g,
                                        void* beta, hipStream_t stream) {
  const char* fn = "gdn_gate_prologue";
  if (tokens < 0 || h_v <= 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: tokens=%d must be >= 0 and h_v=%d > 0", fn, tokens, h_v);
  if (!io_known(io_dtype))
    return fail(GDN_ERR_UNSUPPORTED, "%s: io_dtype %d is not supported", fn, io_dtype);
  if (tokens == 0 || (!g && !beta)) return ok();
  if (g && (!a || !A_log || !dt_bias))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: g needs a, A_log and dt_bias", fn);
  if (beta && !b) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: beta needs b", fn);
  const size_t es = io_size(io_dtype);
  if (!aligned_to(a, es) || !aligned_to(b, es) || !aligned_to(g, es) || !aligned_to(beta, es) ||
      !aligned_to(A_log, 4) || !aligned_to(dt_bias, 4))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: pointers are not aligned to their element size", fn);
  gdn::GatePrologueParams gp{};
  gp.a = a;
  gp.b = b;
  gp.A_log = A_log;
  gp.dt_bias = dt_bias;
  gp.g = g;
  gp.beta = beta;
  gp.rows = tokens;
  gp.h_v = h_v;
  const hipError_t e = gdn::launch_gate_prologue(gp, io_dtype, stream);
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

namespace {

constexpr int32_t kMaxConvCarry = 4096;

gdn_status check_conv(const gdn_conv_problem* c, const char* fn) {
  if (!c) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: problem is NULL", fn);
  if (c->channels <= 0) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: channels=%d must be positive", fn, c->channels);
  if (c->kernel_size <= 0 || c->dilation <= 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: kernel_size=%d and dilation=%d must be positive", fn,
                c->kernel_size, c->dilation);
  if (c->kernel_size > GDN_MAX_CONV_KERNEL)
    return fail(GDN_ERR_UNSUPPORTED, "%s: kernel_size=%d is above %d", fn, c->kernel_size, GDN_MAX_CONV_KERNEL);
  if (static_cast<int64_t>(c->kernel_size - 1) * c->dilation > kMaxConvCarry)
    return fail(GDN_ERR_UNSUPPORTED, "%s: (kernel_size - 1) * dilation is above %d", fn, kMaxConvCarry);
  if (!io_known(c->io_dtype))
    return fail(GDN_ERR_UNSUPPORTED, "%s: io_dtype %d is not supported (GDN_F32, GDN_BF16, GDN_F16)", fn,
                c->io_dtype);
  if (c->activation != GDN_ACT_NONE && c->activation != GDN_ACT_SILU)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: activation %d is not GDN_ACT_NONE or GDN_ACT_SILU", fn,
                c->activation);
  if (!aligned16(c->weight) || !aligned16(c->bias))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: weight and bias must be 16-byte aligned", fn);
  return GDN_OK;
}

gdn::ConvParams conv_params(const gdn_conv_problem& c) {
  gdn::ConvParams cp{};
  cp.weight = c.weight;
  cp.bias = c.bias;
  cp.channels = c.channels;
  cp.ksize = c.kernel_size;
  cp.dilation = c.dilation;
  cp.carry = (c.kernel_size - 1) * c.dilation;
  cp.silu = c.activation == GDN_ACT_SILU;
  return cp;
}

}  // namespace

namespace {

gdn_status conv_impl(const char* fn, const gdn_conv_problem* problem, int32_t num_seqs, const int32_t* cu_seqlens,
                     const int32_t* cu_seqlens_host, int32_t total_tokens, const void* x, const void* initial_state,
                     void* y, void* final_state, const SlotArgs* pool, hipStream_t stream) {
  gdn_status st = check_conv(problem, fn);
  if (st != GDN_OK) return st;
  const gdn_conv_problem& c = *problem;
  if (num_seqs < 0 || total_tokens < 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: num_seqs=%d and total_tokens=%d must be >= 0", fn, num_seqs,
                total_tokens);
  if (num_seqs == 0 && total_tokens != 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: %d tokens but no sequences", fn, total_tokens);
  if (num_seqs > 0 && !cu_seqlens) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: cu_seqlens is NULL", fn);
  if (total_tokens > 0 && (!x || !y || !c.weight))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: x, y and weight are required when total_tokens > 0", fn);
  if (!aligned16(x) || !aligned16(y) || !aligned16(initial_state) || !aligned16(final_state))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: x, y and the states must be 16-byte aligned", fn);
  if (!aligned_to(cu_seqlens, 4)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: cu_seqlens is misaligned", fn);
  if (cu_seqlens_host) {
    if (cu_seqlens_host[0] != 0)
      return fail(GDN_ERR_INVALID_ARGUMENT, "%s: cu_seqlens[0]=%d, expected 0", fn, cu_seqlens_host[0]);
    for (int32_t n = 0; n < num_seqs; ++n)
      if (cu_seqlens_host[n + 1] < cu_seqlens_host[n])
        return fail(GDN_ERR_INVALID_ARGUMENT, "%s: cu_seqlens decreases at %d (%d -> %d)", fn, n,
                    cu_seqlens_host[n], cu_seqlens_host[n + 1]);
    if (cu_seqlens_host[num_seqs] != total_tokens)
      return fail(GDN_ERR_INVALID_ARGUMENT, "%s: cu_seqlens[%d]=%d but total_tokens=%d", fn, num_seqs,
                  cu_seqlens_host[num_seqs], total_tokens);
  }
  if (pool) {
    st = check_slots(*pool, num_seqs, fn);
    if (st != GDN_OK) return st;
  }
  const size_t es = io_size(c.io_dtype);
  const int32_t carry = (c.kernel_size - 1) * c.dilation;
  const size_t xy_bytes = static_cast<size_t>(total_tokens) * c.channels * es;
  const size_t st_bytes = static_cast<size_t>(pool ? pool->num_slots : num_seqs) * carry * c.channels * es;
  if (overlaps(y, xy_bytes, x, xy_bytes)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: y overlaps x", fn);
  if (overlaps(y, xy_bytes, initial_state, st_bytes) || overlaps(y, xy_bytes, final_state, st_bytes) ||
      overlaps(x, xy_bytes, final_state, st_bytes))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: a state overlaps x or y", fn);
  if (final_state && initial_state && final_state != initial_state &&
      overlaps(final_state, st_bytes, initial_state, st_bytes))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: final_state partially overlaps initial_state", fn);
  gdn::ConvParams cp = conv_params(c);
  cp.x = x;
  cp.s0 = carry > 0 ? initial_state : nullptr;
  cp.y = y;
  cp.sN = carry > 0 ? final_state : nullptr;
  cp.cu = cu_seqlens;
  cp.num_seqs = num_seqs;
  cp.total_tokens = total_tokens;
  cp.slots = pool ? pool->slots : nullptr;
  cp.num_slots = pool ? pool->num_slots : 0;
  const hipError_t e = gdn::launch_causal_conv(cp, c.io_dtype, stream);
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

gdn_status conv_step_impl(const char* fn, const gdn_conv_problem* problem, int32_t batch, const void* x, void* state,
                          void* y, const SlotArgs* pool, hipStream_t stream) {
  gdn_status st = check_conv(problem, fn);
  if (st != GDN_OK) return st;
  const gdn_conv_problem& c = *problem;
  if (batch < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: batch=%d is negative", fn, batch);
  if (batch == 0) return ok();
  if (pool) {
    st = check_slots(*pool, batch, fn);
    if (st != GDN_OK) return st;
  }
  const int32_t carry = (c.kernel_size - 1) * c.dilation;
  const bool needs_state = carry > 0 && !(pool && pool->num_slots == 0);
  if (!x || !y || !c.weight || (needs_state && !state))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: x, y, weight and the state are required", fn);
  if (!aligned16(x) || !aligned16(y) || !aligned16(state))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: x, y and the state must be 16-byte aligned", fn);
  const size_t es = io_size(c.io_dtype);
  const size_t xy_bytes = static_cast<size_t>(batch) * c.channels * es;
  const size_t st_bytes = static_cast<size_t>(pool ? pool->num_slots : batch) * carry * c.channels * es;
  if (overlaps(y, xy_bytes, x, xy_bytes) || overlaps(y, xy_bytes, state, st_bytes) ||
      overlaps(x, xy_bytes, state, st_bytes))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: x, y and the state must not overlap", fn);
  gdn::ConvParams cp = conv_params(c);
  cp.x = x;
  cp.s0 = state;
  cp.sN = state;
  cp.y = y;
  cp.num_seqs = batch;
  cp.total_tokens = batch;
  cp.slots = pool ? pool->slots : nullptr;
  cp.num_slots = pool ? pool->num_slots : 0;
  const hipError_t e = gdn::launch_causal_conv_step(cp, c.io_dtype, stream);
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

}  // namespace

GDN_EXPORT gdn_status gdn_causal_conv(const gdn_conv_problem* problem, int32_t num_seqs, const int32_t* cu_seqlens,
                                      const int32_t* cu_seqlens_host, int32_t total_tokens, const void* x,
                                      const void* initial_state, void* y, void* final_state, hipStream_t stream) {
  return conv_impl("gdn_causal_conv", problem, num_seqs, cu_seqlens, cu_seqlens_host, total_tokens, x,
                   initial_state, y, final_state, nullptr, stream);
}

GDN_EXPORT gdn_status gdn_causal_conv_slots(const gdn_conv_problem* problem, int32_t num_seqs,
                                            const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                            int32_t total_tokens, const void* x, void* state_pool, int32_t num_slots,
                                            const int32_t* slots, const int32_t* slots_host, void* y,
                                            hipStream_t stream) {
  const char* fn = "gdn_causal_conv_slots";
  if (num_slots > 0 && !state_pool && problem && problem->kernel_size > 1)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: state_pool is NULL", fn);
  SlotArgs sl;
  sl.slots = slots;
  sl.slots_host = slots_host;
  sl.num_slots = num_slots;
  return conv_impl(fn, problem, num_seqs, cu_seqlens, cu_seqlens_host, total_tokens, x, state_pool, y, state_pool,
                   &sl, stream);
}

GDN_EXPORT gdn_status gdn_causal_conv_step(const gdn_conv_problem* problem, int32_t batch, const void* x, void* state,
                                           void* y, hipStream_t stream) {
  return conv_step_impl("gdn_causal_conv_step", problem, batch, x, state, y, nullptr, stream);
}

GDN_EXPORT gdn_status gdn_causal_conv_step_slots(const gdn_conv_problem* problem, int32_t batch, const void* x,
                                                 void* state_pool, int32_t num_slots, const int32_t* slots,
                                                 const int32_t* slots_host, void* y, hipStream_t stream) {
  SlotArgs sl;
  sl.slots = slots;
  sl.slots_host = slots_host;
  sl.num_slots = num_slots;
  return conv_step_impl("gdn_causal_conv_step_slots", problem, batch, x, state_pool, y, &sl, stream);
}

GDN_EXPORT gdn_status gdn_decode_step_conv(const gdn_problem* problem, const gdn_conv_problem* conv, int32_t batch,
                                           const void* x, const void* conv_state, void* conv_state_out, float* state,
                                           void* out, hipStream_t stream) {
  const char* fn = "gdn_decode_step_conv";
  gdn_status st = check_conv(conv, fn);
  if (st != GDN_OK) return st;
  if (!problem) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: problem is NULL", fn);
  const gdn_conv_problem& c = *conv;
  if (c.io_dtype != problem->io_dtype)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: the conv's io_dtype %d differs from the problem's %d", fn, c.io_dtype,
                problem->io_dtype);
  const int64_t want = 2 * static_cast<int64_t>(problem->h_qk) * problem->d_k +
                       static_cast<int64_t>(problem->h_v) * problem->d_v;
  if (c.channels != want)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: channels=%d must be 2 h_qk d_k + h_v d_v = %lld", fn, c.channels,
                static_cast<long long>(want));
  if (c.dilation != 1 || c.kernel_size > 4)
    return fail(GDN_ERR_UNSUPPORTED,
                "%s: the conv prologue serves dilation 1 and kernel_size <= 4 (got %d, %d); run "
                "gdn_causal_conv_step, then gdn_decode_step",
                fn, c.dilation, c.kernel_size);
  if (batch < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: batch=%d is negative", fn, batch);
  const bool carries = c.kernel_size > 1;
  if (batch > 0 && (!x || !c.weight || (carries && (!conv_state || !conv_state_out))))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: x, weight, conv_state and conv_state_out are required", fn);
  if (!aligned16(x) || !aligned16(conv_state) || !aligned16(conv_state_out))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: x, conv_state and conv_state_out must be 16-byte aligned", fn);
  const size_t cs_bytes = static_cast<size_t>(batch) * (c.kernel_size - 1) * c.channels * io_size(c.io_dtype);
  if (overlaps(conv_state_out, cs_bytes, conv_state, cs_bytes))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: conv_state_out overlaps conv_state (it cannot be updated in place)", fn);
  gdn::ConvPrologue cp{};
  cp.x = x;
  cp.state = carries ? conv_state : nullptr;
  cp.state_out = carries ? conv_state_out : nullptr;
  cp.weight = c.weight;
  cp.bias = c.bias;
  cp.channels = c.channels;
  cp.ksize = c.kernel_size;
  cp.silu = c.activation == GDN_ACT_SILU;
  return decode_impl(fn, problem, batch, nullptr, nullptr, nullptr, state, out, nullptr, stream, &cp);
}

GDN_EXPORT gdn_status gdn_gated_rmsnorm(int64_t rows, int32_t width, int32_t group, int32_t io_dtype, const void* x,
                                        const void* gate, const void* scale, float eps, int32_t activation, void* y,
                                        hipStream_t stream) {
  const char* fn = "gdn_gated_rmsnorm";
  if (rows < 0 || width <= 0 || group <= 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: rows=%lld must be >= 0, width=%d and group=%d positive", fn,
                static_cast<long long>(rows), width, group);
  if (width % group != 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: width=%d is not a multiple of group=%d", fn, width, group);
  if (!io_known(io_dtype)) return fail(GDN_ERR_UNSUPPORTED, "%s: io_dtype %d is not supported", fn, io_dtype);
  if (activation != GDN_ACT_SILU && activation != GDN_ACT_SIGMOID)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: activation %d is not GDN_ACT_SILU or GDN_ACT_SIGMOID", fn,
                activation);
  if (!(eps >= 0.0f) || !std::isfinite(eps))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: eps must be finite and >= 0", fn);
  if (!gdn::gated_rmsnorm_supported(io_dtype, group))
    return fail(GDN_ERR_UNSUPPORTED, "%s: group=%d is larger than the kernel serves", fn, group);
  if (rows == 0) return ok();
  if (!x || !gate || !scale || !y) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: x, gate, scale and y are required", fn);
  if (!aligned16(x) || !aligned16(gate) || !aligned16(scale) || !aligned16(y))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: x, gate, scale and y must be 16-byte aligned", fn);
  const size_t bytes = static_cast<size_t>(rows) * width * io_size(io_dtype);
  if ((y != x && overlaps(y, bytes, x, bytes)) || overlaps(y, bytes, gate, bytes))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: y overlaps gate, or x other than exactly", fn);
  gdn::NormParams np{};
  np.x = x;
  np.gate = gate;
  np.scale = scale;
  np.y = y;
  np.groups = rows * (width / group);
  np.group = group;
  np.eps = eps;
  np.activation = activation;
  const hipError_t e = gdn::launch_gated_rmsnorm(np, io_dtype, stream);
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

GDN_EXPORT const char* gdn_last_error(void) { return g_last_error; }

GDN_EXPORT const char* gdn_status_string(gdn_status status) {
  switch (status) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_INVALID_ARGUMENT: return "GDN_ERR_INVALID_ARGUMENT";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
    case GDN_ERR_HIP: return "GDN_ERR_HIP";
  }
  return "GDN_STATUS_UNKNOWN";
}

GDN_EXPORT int32_t gdn_abi_version(void) { return GDN_ABI_VERSION; }
