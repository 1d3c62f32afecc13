/*
 * gdn.h -- C ABI of libgdn, the gated delta-rule (Gated DeltaNet) recurrence
 * on AMD Instinct MI355X (gfx950).
 *
 * The operation (per value head h, per token t of a sequence, state S of
 * d_k x d_v held in float32 whatever the I/O dtype):
 *     S   <- exp(g_t) S                         decay
 *     r    = S^T k_t                            retrieval
 *     S   <- S + k_t (beta_t (v_t - r))^T       delta update
 *     o_t  = scale S^T q_t                      readout of the UPDATED state
 * as defined on the pages
 *   [P4] onnx-runtime-ep-cuda 0.1.0-dev.6, src/kernels/linear_attention.rs:
 *        module doc "Parallelization" and `linear_attention_core` steps 1-4;
 *   [P1] onnxruntime-ep-mlx 0.31.1, src/ops/ssm.rs: `linear_attention_op`;
 *   [P3] nuvec-core 0.6.1, fast/imp.rs: `gated_delta` / `gated_delta_graph`.
 * The float32 working state follows [P4]'s module doc (widen on read, narrow
 * on write) and [P1]'s wide scan; narrowing to bfloat16 rounds to nearest
 * even, once per stored element.
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     keeps no pointer after a call returns and allocates no device memory.
 *   - Tensors are dense row-major with the layouts given below, and every
 *     tensor pointer is 16-byte aligned (GDN_ERR_INVALID_ARGUMENT otherwise).
 *   - Work is enqueued on `stream` and the call returns without waiting;
 *     nothing in the library synchronises the device, so calls may be
 *     captured into a HIP graph.
 *   - Arguments are validated on the host before anything is enqueued.  On a
 *     non-OK status nothing was enqueued and gdn_last_error() describes why.
 *   - Value head h reads query/key head h / (h_v / h_qk): each q/k head
 *     serves a run of consecutive value heads ([P4] inverse-GQA branch of
 *     `linear_attention_core`; [P3] `gated_delta_graph`).
 */
#ifndef GDN_H
#define GDN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 10

/* Largest supported head size ([P4] MAX_D_K; [P1] typed scan bound). */
#define GDN_MAX_HEAD_DIM 256

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARGUMENT = 1, /* shape, pointer, alignment or value error  */
  GDN_ERR_UNSUPPORTED = 2,      /* well-formed but outside what is built     */
  GDN_ERR_HIP = 3               /* a HIP runtime call failed (launch, attrs) */
} gdn_status;

/* I/O element types ([P4] module doc: half-precision inputs are widened to
 * float32 on read and narrowed on write; its `linear_attention_f16` and
 * `linear_attention_bf16` entry kernels).  Narrowing rounds to nearest even. */
typedef enum gdn_dtype {
  GDN_F32 = 0,
  GDN_BF16 = 1,
  GDN_F16 = 2
} gdn_dtype;

/* How the per-token gates reach the recurrence. */
typedef enum gdn_gate_mode {
  /* g (log-decay, alpha = exp(g)) and beta are given per token and value head. */
  GDN_GATES_PRECOMPUTED = 0,
  /* The gate prologue runs inside the kernel, in float32 with no intermediate
   * rounding ([P4] fused sigmoid / softplus branch of `linear_attention_core`;
   * [P1] `linear_attention_gate_op`):
   *     beta = sigmoid(b),   g = -exp(A_log) * softplus(a + dt_bias)        */
  GDN_GATES_RAW = 1
} gdn_gate_mode;

/* Which prefill formulation gdn_prefill runs.  Both compute the recurrence
 * above; they differ only in rounding. */
typedef enum gdn_algorithm {
  /* CHUNKED where it is supported and sequences average at least 64 tokens,
   * SERIAL otherwise.  For float32 I/O, CHUNKED is taken only with a
   * workspace (below). */
  GDN_ALGO_AUTO = 0,
  /* Token-by-token scan in float32 on the vector ALUs ([P4]'s order of
   * operations); any gates, any head size 1..256, float32, bfloat16 or
   * float16 I/O. */
  GDN_ALGO_SERIAL = 1,
  /* The same recurrence in chunks of 64 tokens on the matrix cores (f32
   * accumulation, f32 state carried between chunks).  bfloat16 I/O: bf16
   * operands, d_k of 64 or 128 and d_v a multiple of 8.  float32 I/O: every
   * operand split into two bf16 parts and each product formed as
   * hi.hi + hi.lo + lo.hi (float32-class accuracy), d_k of 128 or 256, d_v a
   * multiple of 16 up to 256, and a workspace (the two-pass form only).
   * Both need a per-head decay (or none), no state history and a true decay
   * (g <= 0, as the raw-gate prologue always gives).  The gated-delta and
   * delta rules run in every form, and so do the gated and linear rules (no
   * delta correction: T = I, D = V), with d_v up to 256 in the bfloat16
   * two-pass form.  Otherwise GDN_ERR_UNSUPPORTED when requested
   * explicitly. */
  GDN_ALGO_CHUNKED = 2
} gdn_algorithm;

/* Update rule ([P4] `UpdateRule`; [P1] `is_known_rule`).  The default (0) is
 * the gated delta rule; the others drop the decay, the delta correction, or
 * both:
 *   GATED_DELTA  S <- exp(g) S;  S <- S + k (beta (v - S^T k))^T
 *   DELTA        S <- S + k (beta (v - S^T k))^T          (g not read)
 *   GATED        S <- exp(g) S + k v^T                     (beta not read)
 *   LINEAR       S <- S + k v^T                            (neither read)  */
typedef enum gdn_rule {
  GDN_RULE_GATED_DELTA = 0,
  GDN_RULE_DELTA = 1,
  GDN_RULE_GATED = 2,
  GDN_RULE_LINEAR = 3
} gdn_rule;

/* Activation applied by the convolution and the norm. */
typedef enum gdn_activation {
  GDN_ACT_NONE = 0,    /* convolution only                        */
  GDN_ACT_SILU = 1,    /* x * sigmoid(x)                          */
  GDN_ACT_SIGMOID = 2  /* gated RMSNorm only: sigmoid(gate)       */
} gdn_activation;

/* Geometry and gate inputs of one call. */
typedef struct gdn_problem {
  int32_t h_qk;     /* query/key heads, >= 1                                  */
  int32_t h_v;      /* value (state, output) heads, a multiple of h_qk       */
  int32_t d_k;      /* key/query head size, 1 .. GDN_MAX_HEAD_DIM            */
  int32_t d_v;      /* value head size, 1 .. GDN_MAX_HEAD_DIM                */
  int32_t io_dtype; /* gdn_dtype of q, k, v, out, g, beta, a, b              */
  float scale;      /* readout scale; 0 selects 1/sqrt(d_k) ([P4] factory)   */
  int32_t gate_mode;    /* gdn_gate_mode                                     */
  const void* g;        /* PRECOMPUTED: [tokens, h_v] io_dtype, log-decay    */
  const void* beta;     /* PRECOMPUTED: [tokens, h_v] io_dtype               */
  const void* a;        /* RAW: [tokens, h_v] io_dtype                       */
  const void* b;        /* RAW: [tokens, h_v] io_dtype                       */
  const float* A_log;   /* RAW: [h_v] float32                                */
  const float* dt_bias; /* RAW: [h_v] float32                                */
  int32_t algorithm;    /* gdn_algorithm; gdn_prefill only (decode ignores it) */
  int32_t rule;         /* gdn_rule                                          */
  /* 1: the decay is per key dimension ([P4] decay layout [B, T, H_kv d_k]):
   * g (or a) is [tokens, h_v, d_k] and row i of the state decays by
   * exp(g[t,h,i]); with raw gates A_log and dt_bias are [h_v, d_k].       */
  int32_t decay_per_key;
  /* 1: one beta per token shared by all value heads ([P4] beta layout
   * [B, T, 1]): beta (or b) is [tokens].                                  */
  int32_t beta_shared;
  /* gdn_prefill / gdn_prefill_slots only: W > 0 writes the state after each
   * of the last W tokens of every sequence, oldest first, to state_history
   * [num_seqs, W, h_v, d_k, d_v] float32; slots before a sequence's first
   * token are zero ([P1] `state_window`; W = T gives every step, as [P3]
   * `gated_delta_steps`).  Decode ignores both fields.                    */
  int32_t state_window;
  float* state_history;
  /* Optional device workspace for the chunked prefill (gdn_prefill and
   * gdn_prefill_slots).  When the chunked form runs and workspace_bytes is at
   * least gdn_prefill_workspace_size(), it runs in two passes: every chunk's
   * factors are prepared in parallel into the workspace, then a sequential
   * pass carries the state from chunk to chunk.  Otherwise (bfloat16 I/O
   * only) one pass walks each sequence chunk by chunk.  Both give the same
   * result up to rounding.  The float32 form needs about 270 KiB per chunk
   * of 64 tokens and value head at d_k = d_v = 256.
   * The workspace is the caller's (16-byte aligned); its contents are
   * scratch, and calls that share it must not overlap in time. */
  void* workspace;
  uint64_t workspace_bytes;
  /* Optional gated RMSNorm of the output ([P1] `gated_rms_norm_op`), one
   * group per value head: with norm_gate non-NULL, out receives for every
   * (token, value head) row of d_v elements
   *     y = o / sqrt(mean(o^2) + norm_eps) * norm_scale * act(norm_gate)
   * in place of the readout o.  Where a workgroup owns whole output rows and
   * that pays (the decode step with d_v <= 128 at d_k <= 128, else d_v <= 64;
   * the bfloat16 two-pass chunked prefill with d_v <= 128 when its state pass
   * runs 128-column blocks, about 512 or more (sequence, value head) units)
   * the norm is applied to the float32 readout in the kernel that computes
   * it, and o never reaches memory; elsewhere out receives o and the norm then
   * runs over it in place, as gdn_gated_rmsnorm would.
   * gdn_prefill_query_plan reports which.                                   */
  const void* norm_gate;     /* [tokens, h_v, d_v] io_dtype, or NULL: no norm  */
  const void* norm_scale;    /* [d_v] io_dtype                                 */
  float norm_eps;            /* >= 0                                           */
  int32_t norm_activation;   /* GDN_ACT_SILU or GDN_ACT_SIGMOID                */
} gdn_problem;

/*
 * gdn_prefill -- the recurrence over packed variable-length sequences.
 *
 *   cu_seqlens      device int32 [num_seqs + 1]: sequence n owns tokens
 *                   cu_seqlens[n] .. cu_seqlens[n+1]-1.  Required:
 *                   cu_seqlens[0] = 0, non-decreasing, cu_seqlens[num_seqs]
 *                   = total_tokens.  The device copy is not read back, so
 *                   these are checked only through cu_seqlens_host.
 *   cu_seqlens_host optional host copy of the same values (NULL allowed).
 *                   When given it is validated and used to start the longest
 *                   sequences first.
 *   q, k            [total_tokens, h_qk, d_k] io_dtype
 *   v               [total_tokens, h_v, d_v] io_dtype
 *   initial_state   [num_seqs, h_v, d_k, d_v] float32, or NULL for zeros
 *   out             [total_tokens, h_v, d_v] io_dtype, or NULL (not written)
 *   final_state     [num_seqs, h_v, d_k, d_v] float32, or NULL (not
 *                   returned).  It may be the same pointer as initial_state
 *                   (each state slice is read before it is written) but must
 *                   not overlap it otherwise.
 * A sequence with no tokens returns its initial state (zeros without one)
 * ([P1] zero-length time axis).  total_tokens == 0 is valid.
 */
gdn_status gdn_prefill(const gdn_problem* problem, int32_t num_seqs,
                       const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                       int32_t total_tokens, const void* q, const void* k,
                       const void* v, const float* initial_state, void* out,
                       float* final_state, hipStream_t stream);

/*
 * gdn_decode_step -- one token for each of `batch` sequences, with the state
 * resident in device memory and updated in place: the recurrence above with a
 * time axis of length one, the present state written over the past one ([P4]
 * execute contract with T = 1, past_state -> present_state; [P1]
 * `linear_attention_op` with a one-step sequence; [P3] `gated_delta_slots` is
 * the same step over a state pool).
 *
 *   q, k   [batch, h_qk, d_k] io_dtype
 *   v      [batch, h_v, d_v] io_dtype
 *   state  [batch, h_v, d_k, d_v] float32, read and overwritten
 *   out    [batch, h_v, d_v] io_dtype
 * Gate tensors of `problem` are [batch, h_v].
 * Same result as gdn_prefill with cu_seqlens = {0, 1, ..., batch} and
 * final_state == initial_state == state.
 */
gdn_status gdn_decode_step(const gdn_problem* problem, int32_t batch,
                           const void* q, const void* k, const void* v,
                           float* state, void* out, hipStream_t stream);

/*
 * gdn_prefill_workspace_size -- bytes of workspace that let gdn_prefill (or
 * gdn_prefill_slots) with this problem, num_seqs sequences and total_tokens
 * tokens run the chunked form in two passes; 0 when that form does not apply
 * (the serial algorithm, or a geometry the chunked form does not serve).  The
 * size is a bound that holds for any split of the tokens into sequences.
 */
gdn_status gdn_prefill_workspace_size(const gdn_problem* problem, int32_t num_seqs,
                                      int32_t total_tokens, uint64_t* bytes);

/* The formulation gdn_prefill takes for a given problem ("plan"), as
 * resolved from problem->algorithm, the geometry, the workspace and the
 * device's compute-unit count.  Every form computes the recurrence above; they
 * differ in rounding only. */
typedef enum gdn_prefill_form {
  GDN_FORM_NONE = 0,              /* no sequences: nothing is launched          */
  GDN_FORM_SERIAL = 1,            /* token-by-token scan on the vector ALUs     */
  GDN_FORM_CHUNKED_ONE_PASS = 2,  /* bf16 chunks of 64, one pass per sequence   */
  GDN_FORM_CHUNKED_TWO_PASS = 3,  /* bf16 chunks, chunk-parallel preparation
                                     into the workspace, then a state pass     */
  GDN_FORM_CHUNKED_F32 = 4        /* float32 I/O chunks on split-bf16 products,
                                     two passes through the workspace          */
} gdn_prefill_form;

typedef struct gdn_prefill_plan {
  int32_t form;               /* gdn_prefill_form                              */
  int32_t columns_per_block;  /* state columns one workgroup of the sequential
                                 kernel owns (serial form: one wave)           */
  int32_t state_workgroups;   /* workgroups of the sequential kernel's grid    */
  int32_t norm;               /* 0: no norm; 1: fused into the output store;
                                 2: a separate in-place pass over out          */
  char kernels[184];          /* the kernels launched, in order, joined by
                                 " + ", NUL-terminated                         */
} gdn_prefill_plan;

/*
 * gdn_prefill_query_plan -- host-only: fills `plan` with what gdn_prefill (or
 * gdn_prefill_slots) would launch for this problem, num_seqs sequences and
 * total_tokens tokens, with outputs requested.  Enqueues nothing and touches
 * no device memory; the same function resolves GDN_ALGO_AUTO for gdn_prefill.
 * Returns the status gdn_prefill would return for an explicit
 * GDN_ALGO_CHUNKED request that the geometry does not serve.
 */
gdn_status gdn_prefill_query_plan(const gdn_problem* problem, int32_t num_seqs,
                                  int32_t total_tokens, gdn_prefill_plan* plan);

/*
 * gdn_prefill_static_workspace -- gdn_prefill for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops and
 * harnesses that forbid allocation.  Same arguments and result as
 * gdn_prefill, with problem->workspace NULL and workspace_bytes 0: where the
 * chunked form runs in two passes, its workspace is an array of
 * GDN_STATIC_WORKSPACE_BYTES that the library holds in each device's memory
 * from its first use there until the process ends.  The call allocates
 * nothing: no hipMalloc, no hipFree, no allocating library routine.
 *   - A problem whose two-pass workspace (gdn_prefill_workspace_size) exceeds
 *     GDN_STATIC_WORKSPACE_BYTES is refused with GDN_ERR_UNSUPPORTED and
 *     nothing is enqueued; forms without a workspace run as in gdn_prefill.
 *   - Every call on one device shares that device's array: calls that overlap
 *     in time on one device (on different streams, or from several threads
 *     without ordering) race on it and give undefined results.  Calls in
 *     stream order are safe; nothing in the array needs clearing between
 *     them, as each call writes all it reads.
 */
#define GDN_STATIC_WORKSPACE_BYTES (64ull << 20)
gdn_status gdn_prefill_static_workspace(const gdn_problem* problem, int32_t num_seqs,
                                        const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                        int32_t total_tokens, const void* q, const void* k,
                                        const void* v, const float* initial_state, void* out,
                                        float* final_state, hipStream_t stream);

/*
 * Slot-indexed state pool ([P3] nuvec-core, fast/imp.rs, `gated_delta_slots`:
 * recurrent states live in a pool and each sequence of a batch names its
 * state by an int32 slot; the state is gathered, run and scattered back).
 *
 *   state_pool  [num_slots, h_v, d_k, d_v] float32, read and updated in place
 *   slots       device int32 [n] (n = num_seqs or batch): sequence i uses
 *               state_pool[slots[i]].  A slot outside [0, num_slots) marks a
 *               padding sequence: it runs from a zero state and nothing is
 *               written back for it (its outputs are still written).  Slots
 *               inside the range must be distinct.
 *   slots_host  optional host copy of slots; when given, distinctness is
 *               checked (GDN_ERR_INVALID_ARGUMENT on a repeated slot).  The
 *               kernels bounds-check every slot they read.
 * Everything else is as in gdn_prefill / gdn_decode_step.
 */
gdn_status gdn_prefill_slots(const gdn_problem* problem, int32_t num_seqs,
                             const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                             int32_t total_tokens, const void* q, const void* k,
                             const void* v, float* state_pool, int32_t num_slots,
                             const int32_t* slots, const int32_t* slots_host,
                             void* out, hipStream_t stream);

gdn_status gdn_decode_step_slots(const gdn_problem* problem, int32_t batch,
                                 const void* q, const void* k, const void* v,
                                 float* state_pool, int32_t num_slots,
                                 const int32_t* slots, const int32_t* slots_host,
                                 void* out, hipStream_t stream);

/*
 * gdn_gate_prologue -- the gate prologue alone ([P1] `linear_attention_gate_op`,
 * [P4] fused gate branch), for callers that feed precomputed gates:
 *     g[t,h] = -exp(A_log[h]) * softplus(a[t,h] + dt_bias[h])
 *     beta[t,h] = sigmoid(b[t,h])
 * computed in float32 and narrowed once to io_dtype.
 *   a, b        [tokens, h_v] io_dtype (b may be NULL when beta is NULL)
 *   A_log, dt_bias [h_v] float32
 *   g, beta     [tokens, h_v] io_dtype outputs; either may be NULL.
 */
gdn_status gdn_gate_prologue(int32_t tokens, int32_t h_v, int32_t io_dtype,
                             const void* a, const void* b, const float* A_log,
                             const float* dt_bias, void* g, void* beta,
                             hipStream_t stream);

/* ------------------------------------------------------------------------
 * The block's neighbouring operations: the causal depthwise convolution in
 * front of the recurrence and the gated RMSNorm after it.
 * ---------------------------------------------------------------------- */

/* Largest convolution kernel (taps per channel). */
#define GDN_MAX_CONV_KERNEL 64

/* Causal depthwise conv1d with a carried state ([P1] `causal_conv_op`,
 * CausalConvWithState, channels-last; [P3] `causal_conv1d_slots` fallback
 * graph).  With carry = (kernel_size - 1) * dilation, sequence n's padded
 * input is its state (the last `carry` inputs seen so far, oldest first)
 * followed by its new inputs, and per channel c
 *     z_t = bias[c] + sum_j weight[c, j] * xp(t - carry + j * dilation)
 *     y_t = z_t, or z_t * sigmoid(z_t) with GDN_ACT_SILU
 * (a cross-correlation: the last tap meets the current input).  The new
 * state is the last `carry` positions of the padded input; a sequence with
 * no tokens keeps its state.  Accumulation is float32; y is narrowed once. */
typedef struct gdn_conv_problem {
  int32_t channels;     /* C >= 1                                          */
  int32_t kernel_size;  /* K, 1 .. GDN_MAX_CONV_KERNEL                      */
  int32_t dilation;     /* >= 1, (K - 1) * dilation <= 4096                */
  int32_t io_dtype;     /* gdn_dtype of x, y, weight, bias and the states  */
  int32_t activation;   /* GDN_ACT_NONE or GDN_ACT_SILU                    */
  const void* weight;   /* [C, K] io_dtype                                 */
  const void* bias;     /* [C] io_dtype, or NULL                           */
} gdn_conv_problem;

/*
 * gdn_causal_conv -- the convolution over packed variable-length sequences.
 *   cu_seqlens, cu_seqlens_host, total_tokens  as in gdn_prefill
 *   x, y            [total_tokens, C] io_dtype (y may not overlap x)
 *   initial_state   [num_seqs, carry, C] io_dtype, or NULL for zeros
 *   final_state     [num_seqs, carry, C] io_dtype, or NULL; it may be the
 *                   same pointer as initial_state (updated in place) but
 *                   must not overlap it otherwise.
 */
gdn_status gdn_causal_conv(const gdn_conv_problem* problem, int32_t num_seqs,
                           const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                           int32_t total_tokens, const void* x, const void* initial_state,
                           void* y, void* final_state, hipStream_t stream);

/*
 * gdn_causal_conv_step -- one token for each of `batch` sequences, the
 * state resident in device memory and shifted in place:
 *   x, y    [batch, C] io_dtype
 *   state   [batch, carry, C] io_dtype, read and overwritten
 * Same result as gdn_causal_conv with cu_seqlens = {0, 1, ..., batch} and
 * final_state == initial_state == state.
 */
gdn_status gdn_causal_conv_step(const gdn_conv_problem* problem, int32_t batch, const void* x,
                                void* state, void* y, hipStream_t stream);

/*
 * The convolution over a slot-indexed state pool ([P3] nuvec-core, fast/imp.rs,
 * `causal_conv1d_slots`: pool [slots, K - 1, C] and int32 slots [B]; each
 * sequence's state pool[slots[b]] is put in front of its new inputs, the
 * depthwise convolution (and silu) runs over them, and the last K - 1 inputs
 * are written back to the same pool row).
 *   state_pool  [num_slots, carry, C] io_dtype, read and updated in place
 *   slots       device int32 [n] (n = num_seqs or batch): sequence i's state
 *               is state_pool[slots[i]].  A slot outside [0, num_slots) is a
 *               padding sequence: it starts from a zero state and nothing is
 *               written back for it (its outputs are still written).  Slots
 *               inside the range must be distinct.
 *   slots_host  optional host copy; when given, distinctness is checked
 *               (GDN_ERR_INVALID_ARGUMENT on a repeated slot).  The kernels
 *               bounds-check every slot they read.
 * Everything else is as in gdn_causal_conv / gdn_causal_conv_step (carry =
 * (kernel_size - 1) * dilation; [P3] has dilation 1).
 */
gdn_status gdn_causal_conv_slots(const gdn_conv_problem* problem, int32_t num_seqs,
                                 const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                 int32_t total_tokens, const void* x, void* state_pool,
                                 int32_t num_slots, const int32_t* slots,
                                 const int32_t* slots_host, void* y, hipStream_t stream);

gdn_status gdn_causal_conv_step_slots(const gdn_conv_problem* problem, int32_t batch,
                                      const void* x, void* state_pool, int32_t num_slots,
                                      const int32_t* slots, const int32_t* slots_host, void* y,
                                      hipStream_t stream);

/*
 * gdn_decode_step_conv -- the conv step in front of the decode step, in one
 * launch ([P1] `causal_conv_op` feeding `linear_attention_op`, both with a
 * one-token time axis): per sequence b, the token row x[b] holds the conv
 * inputs of q, k and v, C = 2 h_qk d_k + h_v d_v channels in the order
 *     q [h_qk, d_k] | k [h_qk, d_k] | v [h_v, d_v],
 * and the step runs on the conv outputs as gdn_causal_conv_step would store
 * them (narrowed to io_dtype).  Same result as gdn_causal_conv_step(conv, x,
 * state = conv_state -> conv_state_out, y) followed by gdn_decode_step on the
 * three slices of y, without y in memory.
 *   conv            io_dtype equal to problem->io_dtype, channels = C,
 *                   dilation 1, kernel_size 1 .. 4 (else GDN_ERR_UNSUPPORTED)
 *   x               [batch, C] io_dtype
 *   conv_state      [batch, K - 1, C] io_dtype, read (NULL when K = 1)
 *   conv_state_out  [batch, K - 1, C] io_dtype, receives the carried inputs
 *                   one token later (NULL when K = 1).  It must not overlap
 *                   conv_state: the q and k channels are read by several
 *                   workgroups, so the shift cannot be done in place; callers
 *                   alternate two buffers.
 *   state, out      as in gdn_decode_step (state updated in place)
 * Served for d_k in {16, 32, 64, 128, 256}, d_v a multiple of the decode
 * kernel's columns per workgroup (128 when d_k <= 128 and d_v > 64, else 64),
 * and a per-head decay or none; other problems give GDN_ERR_UNSUPPORTED.  The
 * problem's optional output norm applies as in gdn_decode_step.  No buffer
 * may overlap another except the read-only inputs among themselves.
 */
gdn_status gdn_decode_step_conv(const gdn_problem* problem, const gdn_conv_problem* conv,
                                int32_t batch, const void* x, const void* conv_state,
                                void* conv_state_out, float* state, void* out,
                                hipStream_t stream);

/*
 * gdn_gated_rmsnorm -- gated RMSNorm ([P1] `gated_rms_norm_op`): each row of
 * `width` elements is split into width / group groups of `group` consecutive
 * elements, and per group, in float32,
 *     y = x / sqrt(mean(x^2) + eps) * scale * act(gate)
 * with act = silu (GDN_ACT_SILU) or sigmoid (GDN_ACT_SIGMOID).
 *   x, gate, y  [rows, width] io_dtype (y may be x)
 *   scale       [group] io_dtype
 * width must be a multiple of group; groups of up to 512 16-byte vectors
 * (4096 bf16/f16 or 2048 f32 elements; 512 elements when the group is not a
 * multiple of 16 bytes) are served, larger ones give GDN_ERR_UNSUPPORTED.
 */
gdn_status gdn_gated_rmsnorm(int64_t rows, int32_t width, int32_t group, int32_t io_dtype,
                             const void* x, const void* gate, const void* scale, float eps,
                             int32_t activation, void* y, hipStream_t stream);

/* Message for the last non-OK status returned on the calling thread; the
 * empty string after a call that returned GDN_OK.  The pages' execute paths
 * report each failed check with a message before launching anything ([P4]
 * `LinearAttentionKernel::execute`, its invalid-argument and not-implemented
 * returns); this ABI keeps the message per thread instead of in an exception.
 * The pointer stays valid until the next libgdn call on the same thread. */
const char* gdn_last_error(void);

/* Fixed name of a status code ("GDN_OK", ...), a static string. */
const char* gdn_status_string(gdn_status status);

/* GDN_ABI_VERSION of the built library, to be compared with the header a
 * caller was compiled against (the struct layouts above change with it). */
int32_t gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
