// gdn_launch.hpp -- parameter blocks and launchers of the libgdn kernels
// (internal to the library; the public C ABI is include/gdn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Gate inputs as the kernels see them (one of the two pairs is used).
struct GateArgs {
  int32_t raw;          // 0: g / beta given; 1: a / b / A_log / dt_bias given
  int32_t decays;       // the rule decays the state (g / a read)
  int32_t deltas;       // the rule applies the delta correction (beta / b read)
  int32_t per_key;      // g / a are [tokens, h_v, d_k]; A_log / dt_bias [h_v, d_k]
  int32_t beta_shared;  // beta / b are [tokens]
  const void* g;        // [tokens, h_v] io dtype
  const void* beta;     // [tokens, h_v] io dtype
  const void* a;        // [tokens, h_v] io dtype
  const void* b;        // [tokens, h_v] io dtype
  const float* A_log;   // [h_v]
  const float* dt_bias; // [h_v]
};

// Gated RMSNorm of the output rows (one group of d_v per (token, value head)),
// applied where the kernel that forms o owns whole rows.
struct NormEpilogue {
  const void* gate;       // [tokens, h_v, d_v] io dtype; null: no norm
  const void* scale;      // [d_v] io dtype
  float eps;
  float inv_n;            // 1 / d_v
  int32_t silu;           // 1: gate * sigmoid(gate); 0: sigmoid(gate)
};

// Serial scan over packed sequences.
struct ScanParams {
  const void* q;          // [T, h_qk, d_k]
  const void* k;          // [T, h_qk, d_k]
  const void* v;          // [T, h_v, d_v]
  GateArgs gates;
  const float* s0;        // [N, h_v, d_k, d_v] or null
  void* out;              // [T, h_v, d_v] or null
  float* sN;              // [N, h_v, d_k, d_v] or null
  const int32_t* cu;      // [N + 1]
  // State pool indirection: when slots != null, sequence n's state is
  // s0/sN[slots[n]] (both point at the pool); a slot outside [0, num_slots)
  // starts from zeros and is not written back.
  const int32_t* slots;   // [N] or null (state n belongs to sequence n)
  int32_t num_slots;
  int32_t num_seqs;
  int32_t total_tokens;
  int32_t h_qk, h_v, d_k, d_v;
  int32_t ratio;          // h_v / h_qk
  int32_t col_blocks;     // column blocks per (sequence, head)
  float scale;
  int32_t window;         // > 0: history of the last `window` states per sequence
  float* history;         // [N, window, h_v, d_k, d_v]
  NormEpilogue norm;      // the two-pass chunked form applies it when norm.gate != null
  // The column-block state pass's order of the sequences (position -> sequence,
  // a permutation of [0, num_seqs)) when num_ordered = num_seqs; else the
  // identity.  Set from the host's sequence lengths (up to 64 sequences).
  int32_t num_ordered;
  uint8_t seq_order[64];
};

// Causal depthwise conv in front of the decode step: the step's q, k and v
// are the conv outputs of one token row x = [q | k | v] of C = 2 h_qk d_k +
// h_v d_v channels (dilation 1, K <= 4 taps).  Every output is narrowed to
// the I/O dtype, as a separate conv step would store it, before the
// recurrence reads it.  The carried inputs are read from `state` and the
// shifted ones written to `state_out` (they may not overlap: several
// workgroups read one q/k channel's carried inputs).
struct ConvPrologue {
  const void* x;          // [B, C] io dtype; null: no conv (q, k, v given)
  const void* state;      // [B, K - 1, C] io dtype (K > 1)
  void* state_out;        // [B, K - 1, C] io dtype (K > 1)
  const void* weight;     // [C, K] io dtype
  const void* bias;       // [C] io dtype or null
  int32_t channels;       // C
  int32_t ksize;          // K, 1 .. 4
  int32_t silu;
};

// One decode token per sequence, state updated in place.
struct DecodeParams {
  const void* q;          // [B, h_qk, d_k]
  const void* k;          // [B, h_qk, d_k]
  const void* v;          // [B, h_v, d_v]
  GateArgs gates;
  float* state;           // [B, h_v, d_k, d_v], or the pool [num_slots, ...] when slots != null
  void* out;              // [B, h_v, d_v]
  const int32_t* slots;   // [B] or null; see ScanParams
  int32_t num_slots;
  int32_t batch;
  int32_t b_offset;       // first sequence of this launch (set by the launcher)
  int32_t h_qk, h_v, d_k, d_v;
  int32_t ratio;
  int32_t col_blocks;
  float scale;
  NormEpilogue norm;      // applied when norm.gate != null (then col_blocks == 1)
  ConvPrologue conv;      // applied when conv.x != null (then q, k, v are unused)
};

struct GatePrologueParams {
  const void* a;
  const void* b;
  const float* A_log;
  const float* dt_bias;
  void* g;
  void* beta;
  int64_t rows;
  int32_t h_v;
};

// Causal depthwise conv1d with a carried state, over packed sequences (or
// one token per sequence for the step form).
struct ConvParams {
  const void* x;          // [T, C]
  const void* weight;     // [C, K]
  const void* bias;       // [C] or null
  const void* s0;         // [N, carry, C] or null (zeros)
  void* y;                // [T, C]
  void* sN;               // [N, carry, C] or null; may equal s0
  const int32_t* cu;      // [N + 1]; null for the step form (sequence n = token n)
  int32_t num_seqs;
  int32_t total_tokens;
  int32_t channels;
  int32_t ksize;
  int32_t dilation;
  int32_t carry;          // (ksize - 1) * dilation
  int32_t silu;
  // State pool indirection: when slots != null, sequence n's state is row
  // slots[n] of s0/sN (both point at the pool [num_slots, carry, C]); a slot
  // outside [0, num_slots) starts from zeros and is not written back.
  const int32_t* slots;   // [N] or null
  int32_t num_slots;
};

// Gated RMSNorm over groups of `group` elements.
struct NormParams {
  const void* x;          // [rows, width]
  const void* gate;       // [rows, width]
  const void* scale;      // [group]
  void* y;                // [rows, width]
  int64_t groups;         // rows * width / group
  int32_t group;
  float eps;
  int32_t activation;     // 1 silu, 2 sigmoid
};

// io_dtype: the gdn_dtype of the I/O tensors (0 float32, 1 bfloat16,
// 2 float16).  Each launcher enqueues on `stream` and returns the launch
// status.
hipError_t launch_prefill_scan(ScanParams p, int io_dtype, hipStream_t stream);
hipError_t launch_decode_step(DecodeParams p, int io_dtype, hipStream_t stream);
hipError_t launch_gate_prologue(GatePrologueParams p, int io_dtype, hipStream_t stream);
hipError_t launch_causal_conv(ConvParams p, int io_dtype, hipStream_t stream);
hipError_t launch_causal_conv_step(ConvParams p, int io_dtype, hipStream_t stream);
// Whether the norm kernel serves this group size (at most 512 vectors of
// 16 bytes, or 512 elements when the group is not a multiple of 16 bytes).
bool gated_rmsnorm_supported(int io_dtype, int group);
hipError_t launch_gated_rmsnorm(NormParams p, int io_dtype, hipStream_t stream);

// Chunked (matrix-core) prefill: whether a geometry is built, the state
// columns one workgroup owns, and the launcher.
bool chunked_supported(int io_bf16, int d_k, int d_v, const GateArgs& gates, int window);
int chunked_columns_per_block(int d_k, int d_v);
hipError_t launch_prefill_chunked(ScanParams p, int io_bf16, hipStream_t stream);
// The chunked prefill in two passes (chunk-parallel preparation, then the
// sequential state pass) through a caller-provided workspace.
bool split_supported(int io_bf16, int d_k, int d_v, const GateArgs& gates, int window);
int split_columns_per_block(int d_v, int units);
// Whether the bf16 two-pass state pass applies a gated RMSNorm in its output
// store (128-column blocks own whole rows of up to 128 columns; taken where
// the column rule picks 128-column blocks anyway).
bool split_fuses_norm(int d_v, int units);
size_t split_workspace_bytes(int num_seqs, int total_tokens, int h_v, int d_k, int d_v, bool deltas);
hipError_t launch_prefill_split(ScanParams p, void* workspace, hipStream_t stream);
// The chunk table at the head of a two-pass workspace: cs [N + 1] int32 (the
// chunks before each sequence), then info [bound] int2 (first token, tokens of
// every chunk), each in a 256-byte aligned slot.
int chunk_table_bound(int num_seqs, int total_tokens);
size_t chunk_table_bytes(int num_seqs, int total_tokens);
hipError_t launch_chunk_table(const int32_t* cu, int num_seqs, int total_tokens, void* workspace, hipStream_t stream);
// The two-pass chunked prefill for float32 I/O (d_k 128 or 256): matrix-core
// products on operands split into two bfloat16 parts.
bool wide_supported(int io_dtype, int d_k, int d_v, const GateArgs& gates, int window);
size_t wide_workspace_bytes(int num_seqs, int total_tokens, int h_v, int d_k, int d_v);
hipError_t launch_prefill_wide(ScanParams p, void* workspace, hipStream_t stream);
// Whether GDN_ALGO_AUTO takes the float32 two-pass form at this d_k (when a workspace is given).
bool wide_auto(int d_k);

// Index of sequence n's state and whether it exists (slot-pool indirection).
__device__ __forceinline__ int state_slot(const int32_t* slots, int32_t num_slots, int n, bool* valid) {
  if (slots == nullptr) {
    *valid = true;
    return n;
  }
  const int s = slots[n];
  *valid = s >= 0 && s < num_slots;
  return *valid ? s : 0;
}

// Columns one scan wave owns for a given d_k (used to size the grid).
int scan_columns_per_wave(const ScanParams& p);
// Whether the serial scan of `p` runs scan_plain_kernel (else scan_kernel).
bool scan_takes_plain_kernel(const ScanParams& p);
// Whether the bf16 two-pass state pass runs the row-split chunk_rows_kernel
// (else chunk_state_kernel with split_columns_per_block columns).
bool split_takes_rows_kernel(int d_k, int d_v, int units, bool deltas);

// Compute units of the current device (queried once per device; 256 when
// there is no device to ask).  Thread-safe.
int device_compute_units();
// Raise a kernel's dynamic-LDS limit to `bytes` on the current device, once
// per (kernel, device).  Thread-safe.
hipError_t ensure_dynamic_lds(const void* kernel, int bytes);
// The device address (per device, resolved once) and size of the library's
// own two-pass workspace, a file-scope device array.
hipError_t static_workspace(void** ptr, size_t* bytes);
// Columns one decode workgroup owns.
int decode_columns_per_block(int d_k, int d_v, bool per_key);
// Whether the decode kernel applies a gated RMSNorm in its output store (its
// workgroup owns whole rows: d_v at most the columns per block).
bool decode_fuses_norm(int d_k, int d_v, bool per_key);
// Whether the decode kernel can take its inputs through the conv prologue:
// d_k one of 16, 32, 64, 128, 256, d_v a multiple of the columns per block,
// a per-head (or no) decay.
bool decode_takes_conv(int d_k, int d_v, bool per_key);

}  // namespace gdn
