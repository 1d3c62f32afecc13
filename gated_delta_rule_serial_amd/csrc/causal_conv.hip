// causal_conv.hip -- causal depthwise conv1d with a carried state (gfx950),
// the operation in front of the gated delta-rule recurrence in its block.
//
// Definition ([P1] onnxruntime-ep-mlx, src/ops/ssm.rs, `causal_conv_op`
// (CausalConvWithState); [P3] nuvec-core, fast/imp.rs, the
// `causal_conv1d_slots` fallback graph): the carried state (the last
// carry = (K - 1) * dilation inputs of the sequence so far) is put in front
// of the new inputs along time, and per channel c
//     z_t = bias_c + sum_j w[c, j] * xp(t - carry + j * dilation)
//     y_t = z_t (or z_t * sigmoid(z_t) with silu)
// where xp(p) is the state for p < 0 and the input for p >= 0; the new
// state is the last `carry` positions of the padded input.  Layouts are
// channels-last: x, y [T, C], states [N, carry, C], w [C, K].  With a state
// pool ([P3] `causal_conv1d_slots`: pool [slots, K - 1, C], int32 slots [B])
// sequence n's state is row slots[n] of the pool, gathered and scattered back
// in place; a slot outside the pool is a padding sequence (zero state,
// nothing written back).
//
// HBM-bound elementwise work (K multiply-adds per element).  Kernels:
//   conv_window_kernel  dilation 1, K <= 4, C a multiple of one 16-byte
//       vector: a thread owns one channel vector (16 bytes) of kSeg = 8
//       consecutive tokens of the packed axis and issues all its loads at
//       once (weights, bias, the K - 1 rows in front and the kSeg rows); a
//       wave reads 1 KiB contiguous per row and writes it with 16-byte
//       stores.  A segment that touches a sequence start reads the carried
//       state for positions before it.  Consecutive segments run on one L2
//       domain, so the rows in front of a segment tend to come from L2.  The silu uses
//       the hardware exp2 / reciprocal: with the precise forms the kernel
//       was bound by the vector ALUs, not by HBM.
//   conv_generic_kernel any K and dilation: one thread per (token, channel).
//   conv_state_kernel   the new state, one thread per (sequence, channel),
//       after the outputs (stream order), so the state may be updated in place.
//   conv_step_kernel    one token per sequence, state read and shifted in place.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 8;                // token rows loaded at once
constexpr int kSeg = kChunk;             // tokens per thread in the window kernel
constexpr int kXcds = 8;                 // L2 domains; workgroups go to them round-robin

// Sequence holding packed token t: the n with cu[n] <= t < cu[n + 1].
__device__ __forceinline__ int find_seq(const int32_t* cu, int num_seqs, int t) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Bounds of sequence n clamped into [0, T], so that a malformed cu_seqlens
// (which is not read back to the host) can never send an access out of x.
__device__ __forceinline__ int seq_begin(const int32_t* cu, int n, int T) { return min(max(cu[n], 0), T); }
__device__ __forceinline__ int seq_end(const int32_t* cu, int n, int T) {
  return min(max(cu[n + 1], seq_begin(cu, n, T)), T);
}

template <typename IO>
__device__ __forceinline__ float silu_if(float z, int silu) {
  return silu ? z * fast_sigmoid(z) : z;
}

// Row of the state array that holds sequence n's state (n itself, or its
// slot in a pool), or -1 when it has none (a padding slot).
__device__ __forceinline__ int state_row(const ConvParams& p, int n) {
  if (p.slots == nullptr) return n;
  const int s = p.slots[n];
  return (s >= 0 && s < p.num_slots) ? s : -1;
}

// Padded input of sequence n (first token t0, state row sr, -1 for none) at
// position p relative to the sequence start, channel c.
template <typename IO>
__device__ __forceinline__ float xp_at(const IO* __restrict__ x, const IO* __restrict__ s0, int C, int carry,
                                       int sr, int t0, int p, int c) {
  if (p >= 0) return widen(x[static_cast<size_t>(t0 + p) * C + c]);
  if (s0 == nullptr || sr < 0 || p < -carry) return 0.0f;
  return widen(s0[(static_cast<size_t>(sr) * carry + carry + p) * C + c]);
}

// Grid: kXcds * segs_per_xcd * channel_blocks workgroups.  Workgroup L runs
// on L2 domain L % kXcds; it takes channel block (L / kXcds) % channel_blocks
// and segment (L % kXcds) * segs_per_xcd + (L / kXcds) / channel_blocks, so a
// domain walks consecutive segments of the packed axis in order and the
// K - 1 rows in front of a segment are still in its L2.
template <typename IO, int K, bool SILU>
__global__ __launch_bounds__(kThreads) void conv_window_kernel(ConvParams p, int channel_blocks, int segs_per_xcd) {
  constexpr int V = 16 / static_cast<int>(sizeof(IO));
  constexpr int W = K - 1;     // rows in front of a token that its output reads
  constexpr int R = W + kSeg;  // rows held: tokens t_first - W .. t_first + kSeg - 1
  const int C = p.channels;
  const int L = static_cast<int>(blockIdx.x);
  const int slot = L / kXcds;
  const int seg = (L % kXcds) * segs_per_xcd + slot / channel_blocks;
  const int cv = (slot % channel_blocks) * kThreads + static_cast<int>(threadIdx.x);
  const int t_first = seg * kSeg;
  if (cv * V >= C || t_first >= p.total_tokens) return;
  const int c0 = cv * V;
  const int t_stop = min(t_first + kSeg, p.total_tokens);
  const IO* __restrict__ x = static_cast<const IO*>(p.x);
  const IO* __restrict__ s0 = static_cast<const IO*>(p.s0);
  const IO* __restrict__ wt = static_cast<const IO*>(p.weight) + static_cast<size_t>(c0) * K;
  IO* __restrict__ y = static_cast<IO*>(p.y);

  // Every load is issued first and unconditionally (a load under a condition
  // is waited for on its own): the weights [C, K] (the V channels' K taps are
  // V * K consecutive elements), the bias (the weights stand in when there is
  // none) and the R rows, clamped into [0, t_stop - 1].  A row before the
  // token's sequence or past the segment's end is loaded and not used.
  RawSlice<IO, V * K> rw;
  rw.load(wt);
  RawSlice<IO, V> rb;
  rb.load(p.bias != nullptr ? static_cast<const IO*>(p.bias) + c0 : wt);
  RawSlice<IO, V> raw[R];
#pragma unroll
  for (int r = 0; r < R; ++r)
    raw[r].load(x + static_cast<size_t>(min(max(t_first - W + r, 0), t_stop - 1)) * C + c0);
  __builtin_amdgcn_sched_barrier(0);

  int n = find_seq(p.cu, p.num_seqs, t_first);
  int ts = seq_begin(p.cu, n, p.total_tokens), te = seq_end(p.cu, n, p.total_tokens);
  float w[K][V], bias[V];
  {
    float wf[V * K];
    rw.widen_to(wf);
#pragma unroll
    for (int e = 0; e < V; ++e)
#pragma unroll
      for (int j = 0; j < K; ++j) w[j][e] = wf[e * K + j];
    rb.widen_to(bias);
#pragma unroll
    for (int e = 0; e < V; ++e) bias[e] = p.bias != nullptr ? bias[e] : 0.0f;
  }

  if (t_first + kSeg <= p.total_tokens && t_first - W >= ts && t_first + kSeg <= te) {
    // the segment and the rows in front of it lie in one sequence: output
    // i reads rows i .. i + W
    float rows[R][V];
#pragma unroll
    for (int r = 0; r < R; ++r) raw[r].widen_to(rows[r]);
#pragma unroll
    for (int i = 0; i < kSeg; ++i) {
      float out[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        float z = bias[e];
#pragma unroll
        for (int j = 0; j < K; ++j) z = fmaf(w[j][e], rows[i + j][e], z);
        out[e] = SILU ? z * fast_sigmoid(z) : z;
      }
      store_slice<IO, V>(y + static_cast<size_t>(t_first + i) * C + c0, out);
    }
    return;
  }

  // General case: a sequence starts in front of or inside the segment, or
  // the segment is the last, partial one.  Token t reads input t - m from
  // the held rows when it belongs to t's sequence, from the sequence's
  // carried state when it lies up to carry positions before it, else zero.
#pragma unroll
  for (int i = 0; i < kSeg; ++i) {
    const int t = t_first + i;
    if (t >= t_stop) break;
    if (t >= te) {  // t opens a later (non-empty) sequence
      while (n + 1 < p.num_seqs && seq_end(p.cu, n, p.total_tokens) <= t) ++n;
      ts = seq_begin(p.cu, n, p.total_tokens);
      te = seq_end(p.cu, n, p.total_tokens);
    }
    float z[V], in[V];
    raw[W + i].widen_to(in);
#pragma unroll
    for (int e = 0; e < V; ++e) z[e] = fmaf(w[W][e], in[e], bias[e]);
#pragma unroll
    for (int m = 1; m <= W; ++m) {
      const int pos = t - m - ts;  // position in the sequence; < 0 is the state
      if (pos >= 0) {
        raw[W + i - m].widen_to(in);
      } else if (s0 != nullptr && pos >= -p.carry && state_row(p, n) >= 0) {
        RawSlice<IO, V> r;
        r.load(s0 + (static_cast<size_t>(state_row(p, n)) * p.carry + p.carry + pos) * C + c0);
        r.widen_to(in);
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e) in[e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < V; ++e) z[e] = fmaf(w[W - m][e], in[e], z[e]);
    }
    float out[V];
#pragma unroll
    for (int e = 0; e < V; ++e) out[e] = SILU ? z[e] * fast_sigmoid(z[e]) : z[e];
    store_slice<IO, V>(y + static_cast<size_t>(t) * C + c0, out);
  }
}

template <typename IO>
__global__ __launch_bounds__(kThreads) void conv_generic_kernel(ConvParams p) {
  const int C = p.channels, K = p.ksize;
  const IO* __restrict__ x = static_cast<const IO*>(p.x);
  const IO* __restrict__ s0 = static_cast<const IO*>(p.s0);
  const IO* __restrict__ wt = static_cast<const IO*>(p.weight);
  const IO* __restrict__ bs = static_cast<const IO*>(p.bias);
  IO* __restrict__ y = static_cast<IO*>(p.y);
  const int64_t total = static_cast<int64_t>(p.total_tokens) * C;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * kThreads) {
    const int t = static_cast<int>(e / C);
    const int c = static_cast<int>(e % C);
    const int n = find_seq(p.cu, p.num_seqs, t);
    const int t0 = seq_begin(p.cu, n, p.total_tokens);
    float z = bs != nullptr ? widen(bs[c]) : 0.0f;
    for (int j = 0; j < K; ++j)
      z = fmaf(widen(wt[static_cast<size_t>(c) * K + j]),
               xp_at(x, s0, C, p.carry, state_row(p, n), t0, t - t0 - p.carry + j * p.dilation, c), z);
    narrow_store(y + e, silu_if<IO>(z, p.silu));
  }
}

// New state of sequence n: sN[n, i] = xp(L - carry + i).  In ascending i the
// source position L + i (state) or an input row never precedes an already
// written destination, so sN may be s0.
template <typename IO>
__global__ __launch_bounds__(kThreads) void conv_state_kernel(ConvParams p) {
  const int C = p.channels;
  const IO* __restrict__ x = static_cast<const IO*>(p.x);
  const IO* s0 = static_cast<const IO*>(p.s0);
  IO* sN = static_cast<IO*>(p.sN);
  const int64_t total = static_cast<int64_t>(p.num_seqs) * C;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * kThreads) {
    const int n = static_cast<int>(e / C);
    const int c = static_cast<int>(e % C);
    const int sr = state_row(p, n);
    if (sr < 0) continue;  // a padding slot keeps nothing
    const int t0 = seq_begin(p.cu, n, p.total_tokens);
    const int L = seq_end(p.cu, n, p.total_tokens) - t0;
    if (L == 0 && s0 == sN) continue;  // the state is unchanged
    for (int i = 0; i < p.carry; ++i) {
      const float v = xp_at(x, s0, C, p.carry, sr, t0, L - p.carry + i, c);
      narrow_store(sN + (static_cast<size_t>(sr) * p.carry + i) * C + c, v);
    }
  }
}

// One token per sequence: y from the state and x, then the state shifts by
// one position in place (ascending order reads s[i + 1] before writing it).
template <typename IO>
__global__ __launch_bounds__(kThreads) void conv_step_kernel(ConvParams p) {
  const int C = p.channels, K = p.ksize;
  const IO* __restrict__ x = static_cast<const IO*>(p.x);
  const IO* __restrict__ wt = static_cast<const IO*>(p.weight);
  const IO* __restrict__ bs = static_cast<const IO*>(p.bias);
  IO* __restrict__ y = static_cast<IO*>(p.y);
  IO* st = static_cast<IO*>(p.sN);
  const int64_t total = static_cast<int64_t>(p.num_seqs) * C;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * kThreads) {
    const int b = static_cast<int>(e / C);
    const int c = static_cast<int>(e % C);
    const int sr = state_row(p, b);  // -1: a padding slot, zero state, nothing kept
    IO* sb = sr >= 0 ? st + static_cast<size_t>(sr) * p.carry * C + c : nullptr;
    const IO xv = x[e];
    float z = bs != nullptr ? widen(bs[c]) : 0.0f;
    for (int j = 0; j < K; ++j) {
      const int pos = j * p.dilation - p.carry;  // <= 0
      const float xin = pos == 0 ? widen(xv) : (sb != nullptr ? widen(sb[static_cast<size_t>(p.carry + pos) * C]) : 0.0f);
      z = fmaf(widen(wt[static_cast<size_t>(c) * K + j]), xin, z);
    }
    narrow_store(y + e, silu_if<IO>(z, p.silu));
    if (sb == nullptr) continue;
    for (int i = 0; i + 1 < p.carry; ++i) sb[static_cast<size_t>(i) * C] = sb[static_cast<size_t>(i + 1) * C];
    if (p.carry > 0) sb[static_cast<size_t>(p.carry - 1) * C] = xv;
  }
}

unsigned grid_for(int64_t elems) {
  const int64_t want = (elems + kThreads - 1) / kThreads;
  return static_cast<unsigned>(want < 8192 ? (want > 0 ? want : 1) : 8192);
}

template <typename IO, bool SILU>
void launch_window(const ConvParams& p, int cb, int per_xcd, dim3 grid, hipStream_t stream) {
  switch (p.ksize) {
    case 1: hipLaunchKernelGGL((conv_window_kernel<IO, 1, SILU>), grid, dim3(kThreads), 0, stream, p, cb, per_xcd); break;
    case 2: hipLaunchKernelGGL((conv_window_kernel<IO, 2, SILU>), grid, dim3(kThreads), 0, stream, p, cb, per_xcd); break;
    case 3: hipLaunchKernelGGL((conv_window_kernel<IO, 3, SILU>), grid, dim3(kThreads), 0, stream, p, cb, per_xcd); break;
    default: hipLaunchKernelGGL((conv_window_kernel<IO, 4, SILU>), grid, dim3(kThreads), 0, stream, p, cb, per_xcd); break;
  }
}

template <typename IO>
hipError_t launch_conv_io(const ConvParams& p, hipStream_t stream) {
  constexpr int V = 16 / static_cast<int>(sizeof(IO));
  if (p.total_tokens > 0 && p.y != nullptr) {
    const bool window = p.dilation == 1 && p.ksize <= 4 && p.channels % V == 0;
    if (window) {
      const int cb = (p.channels / V + kThreads - 1) / kThreads;
      const int segs = (p.total_tokens + kSeg - 1) / kSeg;
      const int per_xcd = (segs + kXcds - 1) / kXcds;
      const dim3 grid(static_cast<unsigned>(kXcds * per_xcd * cb));
      if (p.silu) launch_window<IO, true>(p, cb, per_xcd, grid, stream);
      else launch_window<IO, false>(p, cb, per_xcd, grid, stream);
    } else {
      hipLaunchKernelGGL((conv_generic_kernel<IO>), dim3(grid_for(static_cast<int64_t>(p.total_tokens) * p.channels)),
                         dim3(kThreads), 0, stream, p);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.sN != nullptr && p.carry > 0 && p.num_seqs > 0) {
    hipLaunchKernelGGL((conv_state_kernel<IO>), dim3(grid_for(static_cast<int64_t>(p.num_seqs) * p.channels)),
                       dim3(kThreads), 0, stream, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <typename IO>
hipError_t launch_step_io(const ConvParams& p, hipStream_t stream) {
  if (p.num_seqs == 0) return hipSuccess;
  hipLaunchKernelGGL((conv_step_kernel<IO>), dim3(grid_for(static_cast<int64_t>(p.num_seqs) * p.channels)),
                     dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_causal_conv(ConvParams p, int io_dtype, hipStream_t stream) {
  if (io_dtype == 1) return launch_conv_io<bf16_t>(p, stream);
  if (io_dtype == 2) return launch_conv_io<f16_t>(p, stream);
  return launch_conv_io<float>(p, stream);
}

hipError_t launch_causal_conv_step(ConvParams p, int io_dtype, hipStream_t stream) {
  if (io_dtype == 1) return launch_step_io<bf16_t>(p, stream);
  if (io_dtype == 2) return launch_step_io<f16_t>(p, stream);
  return launch_step_io<float>(p, stream);
}

}  // namespace gdn
