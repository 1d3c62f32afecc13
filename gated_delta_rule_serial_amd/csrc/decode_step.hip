// decode_step.hip -- one gated delta-rule token per sequence, state in HBM
// updated in place (gfx950).
//
// Per (sequence b, value head h), with the decay D = diag(alpha) (alpha_i =
// exp(g) for a per-head decay, exp(g_i) per key dimension, 1 without decay),
// the state S (d_k x d_v float32) is read once and written once:
//     a = S^T (alpha k),  c = S^T (alpha q),  kq = k . q   (one pass over S)
//     delta = beta (v - a)       (retrieval on the decayed state; v for the
//                                 rules without the delta correction)
//     o     = scale (c + delta kq)                (= scale S'^T q)
//     S'    = D S + k delta^T                     (written back)
// This is the order of [P4] onnx-runtime-ep-cuda, src/kernels/
// linear_attention.rs, `linear_attention_core` steps 1-4 (readout of the
// updated state) with the readout expanded algebraically so that it needs no
// second pass over S: S'^T q = alpha S^T q + delta (k . q).
//
// Mapping: a 256-thread workgroup owns BC state columns of one (b, h), BC =
// 128 (d_k <= 128) or 64; the grid is (column block, h, b), so no index needs
// an integer division.  Thread (rg, tc), tc in [0, BC/4), holds rows
// rg*RPT .. rg*RPT + RPT - 1 of columns 4 tc .. 4 tc + 3 in VGPRs, RPT =
// d_k BC / 1024; a wave's load instruction covers 256 / BC rows of BC
// contiguous floats.  The column sums are first reduced across the row groups
// of each wave with lane exchanges, then across the four waves through LDS;
// the first BC threads write o and broadcast delta through LDS; every thread
// then writes its tile.  The state traffic (read + write once) is the
// kernel's HBM cost; it uses non-temporal 16-byte accesses, since no state
// byte is reused.
//
// With the conv prologue (CONV), q, k and v are not read: they are the
// outputs of the causal depthwise conv (and silu) over one token row x = [q |
// k | v] and the carried inputs of each channel, z = bias + sum_j w_j xp_j
// with the last tap on x ([P1] `causal_conv_op` with a one-token time axis).
// Each is rounded to the I/O dtype, as the conv would store it, and then
// widened: the result is that of the conv step followed by the decode step.
// The workgroup computes the 2 d_k q and k channels of its head once (one per
// thread) and shares them through LDS; the first BC threads compute their own
// v column.  The shifted carried inputs go to a second buffer, written for a
// q/k channel by the head group's first workgroup and for a v channel by the
// workgroup that owns its column.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kColsPerThread = 4;

// One conv channel of one token: its input, up to three carried inputs, its
// taps and bias.  The loads are unconditional (indices clamped into the
// buffers, x standing in for absent ones), so that they issue as one batch
// with no branch and one wait covers them.
template <typename IO>
struct ConvChannel {
  static constexpr int kMaxTaps = 4;
  IO x, s[kMaxTaps - 1], w[kMaxTaps], bias;

  __device__ __forceinline__ void load(const ConvPrologue& cv, int b, int ch) {
    const int C = cv.channels, K = cv.ksize, carry = K - 1;
    const IO* xp = static_cast<const IO*>(cv.x) + static_cast<size_t>(b) * C + ch;
    const IO* st = carry > 0 ? static_cast<const IO*>(cv.state) + static_cast<size_t>(b) * carry * C + ch : xp;
    const IO* wt = static_cast<const IO*>(cv.weight) + static_cast<size_t>(ch) * K;
    const IO* bp = cv.bias != nullptr ? static_cast<const IO*>(cv.bias) + ch : xp;
    x = *xp;
#pragma unroll
    for (int j = 0; j < kMaxTaps - 1; ++j) s[j] = st[static_cast<size_t>(min(j, max(carry - 1, 0))) * C];
#pragma unroll
    for (int j = 0; j < kMaxTaps; ++j) w[j] = wt[min(j, K - 1)];
    bias = *bp;
  }

  // z = bias + sum_j w_j xp_j in tap order (the last tap meets x), then silu,
  // rounded to IO and widened back
  __device__ __forceinline__ float out(const ConvPrologue& cv) const {
    const int K = cv.ksize;
    float z = cv.bias != nullptr ? widen(bias) : 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxTaps; ++j)
      if (j < K) z = fmaf(widen(w[j]), j == K - 1 ? widen(x) : widen(s[j < kMaxTaps - 1 ? j : 0]), z);
    if (cv.silu) z = z * fast_sigmoid(z);
    IO r;
    narrow_store(&r, z);
    return widen(r);
  }

  // the carried inputs one token later: rows 1 .. K - 2, then x
  __device__ __forceinline__ void keep(const ConvPrologue& cv, int b, int ch) const {
    const int C = cv.channels, carry = cv.ksize - 1;
    IO* st = static_cast<IO*>(cv.state_out) + static_cast<size_t>(b) * carry * C + ch;
#pragma unroll
    for (int j = 0; j + 1 < kMaxTaps - 1; ++j)
      if (j + 1 < carry) st[static_cast<size_t>(j) * C] = s[j + 1];
    if (carry > 0) st[static_cast<size_t>(carry - 1) * C] = x;
  }
};

// BC: state columns per workgroup (64 or 128).  FULL: d_k == DK and d_v a
// multiple of BC, so every thread's tile lies inside the state and the
// accesses need no masks.  NORM: the workgroup owns the whole output row
// (d_v <= BC) and writes the gated RMSNorm of o instead of o: each wave sums
// o^2 over its 64 columns with DPP, the partials meet in LDS at the barrier
// that publishes delta, and the first BC threads store y.  CONV: the inputs
// come through the conv prologue (FULL shapes with a per-head decay only).
template <typename IO, int DK, int BC, bool PERKEY, bool FULL, bool NORM, bool CONV>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeParams p) {
  constexpr int kColThreads = BC / kColsPerThread;
  constexpr int kRowGroups = kThreads / kColThreads;
  constexpr int kBlockCols = BC;
  constexpr int RPT = DK / kRowGroups;
  static_assert(RPT >= 1 && RPT * kRowGroups == DK, "row groups must tile d_k");
  static_assert(!CONV || (FULL && !PERKEY), "the conv prologue serves whole tiles with a per-head decay");
  constexpr int kConvQK = CONV ? (2 * DK + kThreads - 1) / kThreads : 0;  // q/k channels per thread
  __shared__ float red_a[kWaves][kBlockCols];
  __shared__ float sh_qk[CONV ? 2 * DK : 1];
  __shared__ float red_c[kWaves][kBlockCols];
  __shared__ float red_kq[kWaves];
  __shared__ float sh_delta[kBlockCols];
  __shared__ float red_ss[kBlockCols / 64];

  const int tid = static_cast<int>(threadIdx.x);
  const int tc = tid % kColThreads;
  const int rg = tid / kColThreads;
  const int cb = static_cast<int>(blockIdx.x);
  const int h = static_cast<int>(blockIdx.y);
  const int b = p.b_offset + static_cast<int>(blockIdx.z);
  const int hq = h / p.ratio;
  const int d_k = FULL ? DK : p.d_k, d_v = p.d_v;
  const int j0 = cb * kBlockCols + tc * kColsPerThread;  // first column of this thread
  const int row0 = rg * RPT;
  const bool vec_cols = FULL || ((d_v % 4 == 0) && (j0 + kColsPerThread <= d_v));

  bool has_state;
  const int sidx = state_slot(p.slots, p.num_slots, b, &has_state);
  float* __restrict__ Sg = p.state + (static_cast<size_t>(sidx) * p.h_v + h) * static_cast<size_t>(d_k) * d_v;

  // ---- conv prologue inputs (CONV), then its gate inputs, issued ahead of the
  //      state tile in one batch with no branch: a load under a branch is
  //      waited for where the branch joins, so every index is clamped into its
  //      buffer (x stands in for an absent one) and unused values are dropped
  ConvChannel<IO> cqk[kConvQK > 0 ? kConvQK : 1], cv_v;
  IO beta_c{}, g_c{};
  if constexpr (CONV) {
#pragma unroll
    for (int u = 0; u < kConvQK; ++u) {
      const int c = min(tid + u * kThreads, 2 * DK - 1);  // past 2 d_k: loaded, not used
      cqk[u].load(p.conv, b, (c < DK ? hq : p.h_qk + hq - 1) * DK + c);
    }
    cv_v.load(p.conv, b, 2 * p.h_qk * DK + h * d_v + cb * kBlockCols + tid % kBlockCols);
    const IO* x0 = static_cast<const IO*>(p.conv.x);
    const size_t gi = static_cast<size_t>(b) * p.h_v + h;
    const bool dl = p.gates.deltas != 0, dc = p.gates.decays != 0;
    beta_c = (dl ? static_cast<const IO*>(p.gates.raw ? p.gates.b : p.gates.beta) : x0)
        [dl ? (p.gates.beta_shared ? static_cast<size_t>(b) : gi) : 0];
    g_c = (dc ? static_cast<const IO*>(p.gates.raw ? p.gates.a : p.gates.g) : x0)[dc ? gi : 0];
  }

  // ---- state tile (the plain kernel issues it first: it is the long-latency
  //      traffic); a padding slot starts from zeros
  float S[RPT][kColsPerThread];
  if (!has_state) {
#pragma unroll
    for (int m = 0; m < RPT; ++m)
#pragma unroll
      for (int cc = 0; cc < kColsPerThread; ++cc) S[m][cc] = 0.0f;
  } else {
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      const int i = row0 + m;
      if (FULL || (i < d_k && vec_cols)) {
        const float4 x = load_stream4(Sg + static_cast<size_t>(i) * d_v + j0);
        S[m][0] = x.x;
        S[m][1] = x.y;
        S[m][2] = x.z;
        S[m][3] = x.w;
      } else {
#pragma unroll
        for (int cc = 0; cc < kColsPerThread; ++cc)
          S[m][cc] = (i < d_k && j0 + cc < d_v) ? Sg[static_cast<size_t>(i) * d_v + j0 + cc] : 0.0f;
      }
    }
  }

  // ---- conv outputs (while the tile is in flight): q and k of the head to
  //      LDS, this thread's v column to a register; then the carried inputs,
  //      one token later, to conv.state_out
  float v_conv = 0.0f;
  if constexpr (CONV) {
    float zqk[kConvQK > 0 ? kConvQK : 1];
#pragma unroll
    for (int u = 0; u < kConvQK; ++u) zqk[u] = cqk[u].out(p.conv);
    v_conv = cv_v.out(p.conv);
#pragma unroll
    for (int u = 0; u < kConvQK; ++u)
      if (tid + u * kThreads < 2 * DK) sh_qk[tid + u * kThreads] = zqk[u];
    if (cb == 0 && h == hq * p.ratio) {  // the head group's first workgroup keeps q and k
#pragma unroll
      for (int u = 0; u < kConvQK; ++u) {
        const int c = tid + u * kThreads;
        if (c < 2 * DK) cqk[u].keep(p.conv, b, (c < DK ? hq : p.h_qk + hq - 1) * DK + c);
      }
    }
    if (tid < kBlockCols) cv_v.keep(p.conv, b, 2 * p.h_qk * DK + h * d_v + cb * kBlockCols + tid);
  }

  // ---- k, q rows of this thread (from LDS with the conv prologue, below)
  RawSlice<IO, RPT> rk, rq;
  if constexpr (!CONV) {
    const IO* kq_base_k = static_cast<const IO*>(p.k) + (static_cast<size_t>(b) * p.h_qk + hq) * d_k + row0;
    const IO* kq_base_q = static_cast<const IO*>(p.q) + (static_cast<size_t>(b) * p.h_qk + hq) * d_k + row0;
    if (FULL || d_k == DK) {
      rk.load(kq_base_k);
      rq.load(kq_base_q);
    } else {
      rk.load_masked(kq_base_k, d_k - row0);
      rq.load_masked(kq_base_q, d_k - row0);
    }
  }

  // ---- the norm's gate and scale of this thread's output column (the first
  //      BC threads), issued early: they are read after the last barrier
  float n_gate = 0.0f, n_scale = 0.0f;
  if constexpr (NORM) {
    if (tid < kBlockCols && (FULL || tid < d_v)) {
      n_gate = widen(static_cast<const IO*>(p.norm.gate)[(static_cast<size_t>(b) * p.h_v + h) * d_v + tid]);
      n_scale = widen(static_cast<const IO*>(p.norm.scale)[tid]);
    }
  }

  // ---- gates: beta per (b, h) (or per b); the decay per (b, h) or, per key
  //      dimension, per row of this thread (alpha_r).
  const size_t gidx = static_cast<size_t>(b) * p.h_v + h;
  const bool decays = p.gates.decays != 0, deltas = p.gates.deltas != 0;
  float beta = 0.0f;
  if constexpr (CONV) {
    if (deltas) beta = p.gates.raw ? gate_sigmoid(widen(beta_c)) : widen(beta_c);
  } else if (deltas) {
    const size_t bi = p.gates.beta_shared ? static_cast<size_t>(b) : gidx;
    if (p.gates.raw) beta = gate_sigmoid(widen(static_cast<const IO*>(p.gates.b)[bi]));
    else beta = widen(static_cast<const IO*>(p.gates.beta)[bi]);
  }
  // per-head decay: one alpha, applied to the column sums; per key dimension:
  // alpha_r for this thread's rows, folded into k and q
  float alpha = 1.0f;
  float alpha_r[PERKEY ? RPT : 1];
  if constexpr (PERKEY) {
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      const int i = row0 + m;
      float lg = 0.0f;
      if (decays && i < d_k) {
        const size_t gi = gidx * d_k + i;
        const size_t pi = static_cast<size_t>(h) * d_k + i;
        if (p.gates.raw)
          lg = gate_log_decay(widen(static_cast<const IO*>(p.gates.a)[gi]), p.gates.A_log[pi], p.gates.dt_bias[pi]);
        else
          lg = widen(static_cast<const IO*>(p.gates.g)[gi]);
      }
      alpha_r[m] = expf(lg);
    }
  } else if (decays) {
    float lg;
    if constexpr (CONV)
      lg = p.gates.raw ? gate_log_decay(widen(g_c), p.gates.A_log[h], p.gates.dt_bias[h]) : widen(g_c);
    else if (p.gates.raw)
      lg = gate_log_decay(widen(static_cast<const IO*>(p.gates.a)[gidx]), p.gates.A_log[h], p.gates.dt_bias[h]);
    else
      lg = widen(static_cast<const IO*>(p.gates.g)[gidx]);
    alpha = expf(lg);
  }

  float kf[RPT], qf[RPT];
  if constexpr (CONV) {
    __syncthreads();  // q and k of the head are in LDS
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      qf[m] = sh_qk[row0 + m];
      kf[m] = sh_qk[DK + row0 + m];
    }
  } else {
    rk.widen_to(kf);
    rq.widen_to(qf);
  }
  // the decayed state's retrieval and readout sums: (diag(alpha) S)^T x = S^T (alpha x)
  float ka[PERKEY ? RPT : 1], qa[PERKEY ? RPT : 1];
  if constexpr (PERKEY) {
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      ka[m] = alpha_r[m] * kf[m];
      qa[m] = alpha_r[m] * qf[m];
    }
  }

  // ---- partial column sums over this thread's rows
  float pa[kColsPerThread], pc[kColsPerThread];
  float pkq = 0.0f;
#pragma unroll
  for (int cc = 0; cc < kColsPerThread; ++cc) {
    pa[cc] = 0.0f;
    pc[cc] = 0.0f;
  }
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
#pragma unroll
    for (int cc = 0; cc < kColsPerThread; ++cc) {
      pa[cc] = fmaf(S[m][cc], PERKEY ? ka[PERKEY ? m : 0] : kf[m], pa[cc]);
      pc[cc] = fmaf(S[m][cc], PERKEY ? qa[PERKEY ? m : 0] : qf[m], pc[cc]);
    }
    pkq = fmaf(kf[m], qf[m], pkq);
  }
  // the row groups inside one wave (lanes tc, tc + kColThreads, ...) are
  // summed with lane exchanges; LDS then holds one partial per wave
#pragma unroll
  for (int off = kColThreads; off < 64; off *= 2) {
#pragma unroll
    for (int cc = 0; cc < kColsPerThread; ++cc) {
      pa[cc] = off == 16 ? xor16_sum(pa[cc]) : xor32_sum(pa[cc]);
      pc[cc] = off == 16 ? xor16_sum(pc[cc]) : xor32_sum(pc[cc]);
    }
    pkq = off == 16 ? xor16_sum(pkq) : xor32_sum(pkq);
  }
  const int wave = tid / 64;
  if (tid % 64 < kColThreads) {
#pragma unroll
    for (int cc = 0; cc < kColsPerThread; ++cc) {
      red_a[wave][tc * kColsPerThread + cc] = PERKEY ? pa[cc] : alpha * pa[cc];
      red_c[wave][tc * kColsPerThread + cc] = PERKEY ? pc[cc] : alpha * pc[cc];
    }
    if (tc == 0) red_kq[wave] = pkq;
  }
  __syncthreads();

  // ---- the first BC threads finish the column sums, write o (or keep it for
  //      the norm), publish delta
  float o_keep = 0.0f;
  if (tid < kBlockCols) {
    float a = 0.0f, cs = 0.0f, kq = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      a += red_a[w][tid];
      cs += red_c[w][tid];
      kq += red_kq[w];
    }
    const int j = cb * kBlockCols + tid;
    float vv = 0.0f;
    if constexpr (CONV) vv = v_conv;
    else if (FULL || j < d_v) vv = widen(static_cast<const IO*>(p.v)[(static_cast<size_t>(b) * p.h_v + h) * d_v + j]);
    const float delta = deltas ? beta * (vv - a) : vv;
    sh_delta[tid] = delta;
    if constexpr (NORM) {
      // whole waves take this branch (BC is a multiple of 64): the DPP sum sees every lane
      o_keep = (FULL || j < d_v) ? p.scale * fmaf(delta, kq, cs) : 0.0f;
      const float sq = group_sum<64>(o_keep * o_keep);
      if ((tid & 63) == 0) red_ss[tid >> 6] = sq;
    } else if (FULL || j < d_v) {
      const float o = p.scale * fmaf(delta, kq, cs);
      narrow_store(static_cast<IO*>(p.out) + (static_cast<size_t>(b) * p.h_v + h) * d_v + j, o);
    }
  }
  __syncthreads();
  if constexpr (NORM) {
    if (tid < kBlockCols && (FULL || tid < d_v)) {
      float ss = 0.0f;
#pragma unroll
      for (int w = 0; w < kBlockCols / 64; ++w) ss += red_ss[w];
      const float inv = __builtin_amdgcn_rsqf(fmaf(ss, p.norm.inv_n, p.norm.eps));
      narrow_store(static_cast<IO*>(p.out) + (static_cast<size_t>(b) * p.h_v + h) * d_v + tid,
                   gated_norm(o_keep, inv, n_scale, n_gate, p.norm.silu));
    }
  }

  // ---- S' = alpha S + k delta^T, written back in place
  float dl[kColsPerThread];
#pragma unroll
  for (int cc = 0; cc < kColsPerThread; ++cc) dl[cc] = sh_delta[tc * kColsPerThread + cc];
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = row0 + m;
    // with the conv prologue k is read from LDS again: the registers it held
    // are not kept across the barriers
    const float km = CONV ? sh_qk[DK + row0 + m] : kf[m];
    float o4[kColsPerThread];
#pragma unroll
    for (int cc = 0; cc < kColsPerThread; ++cc)
      o4[cc] = fmaf(S[m][cc], PERKEY ? alpha_r[PERKEY ? m : 0] : alpha, km * dl[cc]);
    if (!has_state) {
      // padding slot: the updated state is discarded
    } else if (FULL || (i < d_k && vec_cols)) {
      store_stream4(Sg + static_cast<size_t>(i) * d_v + j0, make_float4(o4[0], o4[1], o4[2], o4[3]));
    } else if (i < d_k) {
#pragma unroll
      for (int cc = 0; cc < kColsPerThread; ++cc)
        if (j0 + cc < d_v) Sg[static_cast<size_t>(i) * d_v + j0 + cc] = o4[cc];
    }
  }
}

template <typename IO, int DK, int BC, bool PERKEY, bool FULL, bool NORM, bool CONV = false>
hipError_t launch_grid(DecodeParams p, hipStream_t stream) {
  // grid: (column block, value head, sequence); the sequence axis is split
  // into launches of at most 65535
  constexpr int kMaxZ = 65535;
  for (int off = 0; off < p.batch; off += kMaxZ) {
    p.b_offset = off;
    const unsigned nz = static_cast<unsigned>(p.batch - off < kMaxZ ? p.batch - off : kMaxZ);
    hipLaunchKernelGGL((decode_kernel<IO, DK, BC, PERKEY, FULL, NORM, CONV>),
                       dim3(static_cast<unsigned>(p.col_blocks), static_cast<unsigned>(p.h_v), nz),
                       dim3(kThreads), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename IO, int DK, int BC, bool NORM>
hipError_t launch_norm(const DecodeParams& p, hipStream_t stream) {
  const bool full = p.d_k == DK && p.d_v % BC == 0;
  if (p.conv.x != nullptr) {
    // the API admits the conv prologue for whole tiles with a per-head decay only
    if (!full || (p.gates.per_key && p.gates.decays)) return hipErrorInvalidValue;
    return launch_grid<IO, DK, BC, false, true, NORM, true>(p, stream);
  }
  if constexpr (BC == 64) {
    if (p.gates.per_key && p.gates.decays)
      return full ? launch_grid<IO, DK, BC, true, true, NORM>(p, stream)
                  : launch_grid<IO, DK, BC, true, false, NORM>(p, stream);
  }
  return full ? launch_grid<IO, DK, BC, false, true, NORM>(p, stream)
              : launch_grid<IO, DK, BC, false, false, NORM>(p, stream);
}

template <typename IO, int DK, int BC>
hipError_t launch_bc(const DecodeParams& p, hipStream_t stream) {
  // the fused norm needs one column block per row (the API checks it)
  return p.norm.gate != nullptr && p.col_blocks == 1 ? launch_norm<IO, DK, BC, true>(p, stream)
                                                     : launch_norm<IO, DK, BC, false>(p, stream);
}

template <typename IO, int DK>
hipError_t launch_dk(const DecodeParams& p, hipStream_t stream) {
  if (p.batch == 0 || p.h_v == 0 || p.col_blocks == 0) return hipSuccess;
  if constexpr (DK <= 128) {
    if (decode_columns_per_block(p.d_k, p.d_v, p.gates.per_key && p.gates.decays) == 128)
      return launch_bc<IO, DK, 128>(p, stream);
  }
  return launch_bc<IO, DK, 64>(p, stream);
}

template <typename IO>
hipError_t launch_io(const DecodeParams& p, hipStream_t stream) {
  if (p.d_k <= 16) return launch_dk<IO, 16>(p, stream);
  if (p.d_k <= 32) return launch_dk<IO, 32>(p, stream);
  if (p.d_k <= 64) return launch_dk<IO, 64>(p, stream);
  if (p.d_k <= 128) return launch_dk<IO, 128>(p, stream);
  return launch_dk<IO, 256>(p, stream);
}

}  // namespace

// A workgroup takes a whole 128-column row block when d_k <= 128 (its 16 x 4
// register tile per thread still fits), d_v is wider than 64 and the decay is
// per head (a per-key decay keeps a second per-row array live); otherwise 64.
int decode_columns_per_block(int d_k, int d_v, bool per_key) {
  return (d_k <= 128 && d_v > 64 && !per_key) ? 128 : 64;
}

bool decode_fuses_norm(int d_k, int d_v, bool per_key) { return d_v <= decode_columns_per_block(d_k, d_v, per_key); }

bool decode_takes_conv(int d_k, int d_v, bool per_key) {
  const bool dk_bucket = d_k == 16 || d_k == 32 || d_k == 64 || d_k == 128 || d_k == 256;
  return dk_bucket && !per_key && d_v % decode_columns_per_block(d_k, d_v, per_key) == 0;
}

hipError_t launch_decode_step(DecodeParams p, int io_dtype, hipStream_t stream) {
  if (io_dtype == 1) return launch_io<bf16_t>(p, stream);
  if (io_dtype == 2) return launch_io<f16_t>(p, stream);
  return launch_io<float>(p, stream);
}

}  // namespace gdn
