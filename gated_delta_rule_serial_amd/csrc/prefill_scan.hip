// prefill_scan.hip -- serial-scan prefill of the gated delta rule on gfx950.
//
// What is computed (per sequence n, value head h, token t; state S is d_k x d_v
// float32):  S <- exp(g_t) S;  r = S^T k_t;  S <- S + k_t (beta_t (v_t - r))^T;
// o_t = scale S^T q_t on the updated S.  Pages: [P4] onnx-runtime-ep-cuda,
// src/kernels/linear_attention.rs, `linear_attention_core` steps 1-4 and the
// module doc "Parallelization" (each state column evolves on its own);
// [P1] onnxruntime-ep-mlx, src/ops/ssm.rs, the wide scan (float32 working
// state, only I/O stores rounded).
//
// Mapping on a CDNA4 wavefront (64 lanes):
//   * one wave owns CPW = 64 / R state columns of one (sequence, value head);
//   * the R consecutive lanes of a column each hold RPL = DK / R rows of it
//     in VGPRs for the whole scan (no scratch, no LDS);
//   * the two d_k dot products per token (retrieval before the update,
//     readout after it) are partial sums over a lane's rows followed by a
//     DPP row-op reduction over the R lanes (plus the gfx950 lane swaps
//     across 16-lane rows and wave halves for R = 32 and 64);
//   * q_t, k_t, v_t are loaded as packed words PF tokens ahead of use
//     through a register ring, so global latency overlaps the serial chain;
//   * the gates of 64 tokens are computed once, lane-parallel (lane l takes
//     token t0 + l), and read per token with v_readlane; a per-key-dim decay
//     instead travels with q/k through the ring (the lane's RPL rows);
//   * the update rule ([P4] `UpdateRule`) switches the decay and the delta
//     correction off uniformly per launch; the optional state history stores
//     the lane's rows after each of the last W tokens.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

namespace {

constexpr int kWave = 64;
// Tokens of q/k/v in flight ahead of use.  Four suffice when several waves
// share a SIMD; the widest head (d_k = 256, a whole wave per column) runs
// few waves per SIMD, and there the serial chain of one token is far shorter
// than a load's latency, so it keeps eight in flight.
template <int DK>
constexpr int prefetch_depth() { return DK >= 256 ? 8 : 4; }

// Lanes per column for each padded key size (rows per lane = DK / R).
template <int DK>
struct ScanShape;
template <> struct ScanShape<16> { static constexpr int R = 4; };
template <> struct ScanShape<32> { static constexpr int R = 8; };
template <> struct ScanShape<64> { static constexpr int R = 8; };
template <> struct ScanShape<128> { static constexpr int R = 16; };
template <> struct ScanShape<256> { static constexpr int R = 64; };  // one column per wave

// GENERAL = false compiles the plain gated delta rule with no state history
// (the rule flags and the window are constants); GENERAL = true reads them
// at run time and serves every other variant.
// FULL: d_k == DK, so every lane's rows exist and the q/k loads need no masks.
template <typename IO, int DK, bool RAW, bool PERKEY, bool GENERAL, bool FULL>
__global__ __launch_bounds__(kWave) void scan_kernel(ScanParams p) {
  constexpr int R = ScanShape<DK>::R;
  constexpr int CPW = kWave / R;
  constexpr int RPL = DK / R;
  constexpr int kPrefetch = prefetch_depth<DK>();
  // Tokens per loop iteration.  Ring registers that cross the loop's back
  // edge with loads in flight make the compiler wait for those loads at the
  // loop head; d_k = 256 (few waves per SIMD to hide that) unrolls a whole
  // 64-token gate block, so the wait comes once per 64 tokens.  With masked
  // rows (d_k below 256) and half-precision words that unroll left the ring
  // partly in scratch (112 bytes of private segment), so those variants
  // keep the ring-sized group.
  constexpr int kGroup = (DK >= 256 && !GENERAL && (FULL || sizeof(IO) == 4)) ? kWave : kPrefetch;

  const int lane = static_cast<int>(threadIdx.x);
  const int c = lane / R;        // column within the wave
  const int r = lane % R;        // row slice within the column
  int unit = static_cast<int>(blockIdx.x);
  const int cb = unit % p.col_blocks;
  unit /= p.col_blocks;
  const int h = unit % p.h_v;
  const int n = unit / p.h_v;
  const int hq = h / p.ratio;
  const int j = cb * CPW + c;
  const bool col_ok = j < p.d_v;
  const int row0 = r * RPL;
  const bool full_rows = FULL || (p.d_k == DK);
  const int row_limit = p.d_k - row0;  // rows of this lane's slice that exist
  const bool decays = GENERAL ? p.gates.decays != 0 : true;
  const bool deltas = GENERAL ? p.gates.deltas != 0 : true;

  const int t_begin = p.cu[n];
  const int t_end = p.cu[n + 1];

  // ---- initial state (column j, rows row0 .. row0 + RPL - 1)
  bool has_state;
  const int sidx = state_slot(p.slots, p.num_slots, n, &has_state);
  float S[RPL];
  const size_t state_elems = static_cast<size_t>(p.d_k) * p.d_v;
  const size_t sbase = (static_cast<size_t>(sidx) * p.h_v + h) * state_elems;
#pragma unroll
  for (int m = 0; m < RPL; ++m) {
    const int i = row0 + m;
    S[m] = (p.s0 != nullptr && has_state && col_ok && i < p.d_k) ? p.s0[sbase + static_cast<size_t>(i) * p.d_v + j]
                                                                  : 0.0f;
  }

  // ---- state history: slot w of sequence n holds the state after token
  //      t_end - W + w; slots before the first token are zero
  const int W = GENERAL ? p.window : 0;
  auto history_slot = [&](int w) {
    return p.history + ((static_cast<size_t>(n) * W + w) * p.h_v + h) * state_elems;
  };
  if (W > 0 && col_ok) {
    for (int w = 0; w < W - (t_end - t_begin); ++w) {
#pragma unroll
      for (int m = 0; m < RPL; ++m)
        if (row0 + m < p.d_k) history_slot(w)[static_cast<size_t>(row0 + m) * p.d_v + j] = 0.0f;
    }
  }

  const IO* __restrict__ qg = static_cast<const IO*>(p.q);
  const IO* __restrict__ kg = static_cast<const IO*>(p.k);
  const IO* __restrict__ vg = static_cast<const IO*>(p.v);
  IO* __restrict__ og = static_cast<IO*>(p.out);
  const size_t qk_stride = static_cast<size_t>(p.h_qk) * p.d_k;
  const size_t qk_off = static_cast<size_t>(hq) * p.d_k + row0;
  const size_t v_stride = static_cast<size_t>(p.h_v) * p.d_v;
  const size_t v_off = static_cast<size_t>(h) * p.d_v + (col_ok ? j : 0);

  // ---- gates.  Per-head gates: lane l holds (alpha, beta) of token blk + l.
  //      Per-key-dim decay: the decay of this lane's rows travels with q/k.
  const IO* __restrict__ ga = static_cast<const IO*>(RAW ? p.gates.a : p.gates.g);
  const IO* __restrict__ gb = static_cast<const IO*>(RAW ? p.gates.b : p.gates.beta);
  float A_log = 0.0f, dt_bias = 0.0f;           // per-head raw decay parameters
  float A_log_r[RPL], dt_bias_r[RPL];           // per-key-dim raw decay parameters
#pragma unroll
  for (int m = 0; m < RPL; ++m) A_log_r[m] = dt_bias_r[m] = 0.0f;
  if constexpr (RAW) {
    if (t_begin < t_end && decays) {  // the parameters may be absent when nothing reads them
      if constexpr (PERKEY) {
#pragma unroll
        for (int m = 0; m < RPL; ++m)
          if (row0 + m < p.d_k) {
            A_log_r[m] = p.gates.A_log[static_cast<size_t>(h) * p.d_k + row0 + m];
            dt_bias_r[m] = p.gates.dt_bias[static_cast<size_t>(h) * p.d_k + row0 + m];
          }
      } else {
        A_log = p.gates.A_log[h];
        dt_bias = p.gates.dt_bias[h];
      }
    }
  }
  RawScalar<IO> next_ga, next_gb;  // raw per-head gate inputs of the next 64-token block
  auto fetch_gate_block = [&](int blk) {
    const int t = blk + lane;
    next_ga.w = 0u;
    next_gb.w = 0u;
    if (t < t_end) {
      if (decays && !PERKEY) next_ga.load(ga + static_cast<size_t>(t) * p.h_v + h);
      if (deltas) next_gb.load(gb + (p.gates.beta_shared ? static_cast<size_t>(t) : static_cast<size_t>(t) * p.h_v + h));
    }
  };
  float blk_alpha = 1.0f, blk_beta = 0.0f;
  fetch_gate_block(t_begin);

  // ---- q/k/v (and per-key-dim decay) ring
  RawSlice<IO, RPL> ring_k[kPrefetch], ring_q[kPrefetch];
  RawSlice<IO, PERKEY ? RPL : 1> ring_g[kPrefetch];
  RawScalar<IO> ring_v[kPrefetch];
  auto fetch_token = [&](int slot, int t) {
    const size_t qk = static_cast<size_t>(t) * qk_stride + qk_off;
    if (full_rows) {
      ring_k[slot].load(kg + qk);
      ring_q[slot].load(qg + qk);
    } else {
      ring_k[slot].load_masked(kg + qk, row_limit);
      ring_q[slot].load_masked(qg + qk, row_limit);
    }
    if constexpr (PERKEY) {
      if (decays) {
        const IO* gp = ga + (static_cast<size_t>(t) * p.h_v + h) * p.d_k + row0;
        if (full_rows) ring_g[slot].load(gp);
        else ring_g[slot].load_masked(gp, row_limit);
      }
    }
    ring_v[slot].load(vg + static_cast<size_t>(t) * v_stride + v_off);
  };
  // every slot holds a real token (clamped to the last one), so padded tokens
  // at the end compute on finite values
  if (t_begin < t_end) {
#pragma unroll
    for (int s = 0; s < kPrefetch; ++s) fetch_token(s, min(t_begin + s, t_end - 1));
  }

  const float scale = p.scale;
  const int hist_from = (t_end - t_begin) - W;  // first token (relative) whose state is kept
  // The last group runs whole: tokens past the end take alpha = 1 and a zero
  // update (the state stays as it is) and store nothing, so the unrolled
  // group has one exit.
  for (int tb = t_begin; tb < t_end; tb += kGroup) {
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      const int s = u % kPrefetch;  // ring slot
      const int t = tb + u;
      const bool live = t < t_end;
      const int rel = (t - t_begin) & (kWave - 1);
      if (rel == 0) {
        // gates of tokens t .. t + 63, one per lane, then prefetch the next block
        if (decays && !PERKEY) {
          if constexpr (RAW) blk_alpha = expf(gate_log_decay(next_ga.value(), A_log, dt_bias));
          else blk_alpha = expf(next_ga.value());
        }
        if (deltas) {
          if constexpr (RAW) blk_beta = gate_sigmoid(next_gb.value());
          else blk_beta = next_gb.value();
        }
        fetch_gate_block(t + kWave);
      }
      const float beta = live ? readlane(blk_beta, rel) : 0.0f;

      float kf[RPL], qf[RPL];
      ring_k[s].widen_to(kf);
      ring_q[s].widen_to(qf);
      const float vv = ring_v[s].value();
      float gr[PERKEY ? RPL : 1];
      if constexpr (PERKEY) ring_g[s].widen_to(gr);
      // unconditional (clamped to the last token): a conditional load would
      // make the slot a choice between old and new values, which the compiler
      // resolves with a copy that waits for the load
      fetch_token(s, min(t + kPrefetch, t_end - 1));

      float po0 = 0.0f, po1 = 0.0f;
      if constexpr (PERKEY) {
        // decay row by row, then retrieval, delta update and readout
        if (decays && live) {
#pragma unroll
          for (int m = 0; m < RPL; ++m) {
            const float lg = RAW ? gate_log_decay(gr[m], A_log_r[m], dt_bias_r[m]) : gr[m];
            S[m] *= expf(lg);
          }
        }
        float delta = live ? vv : 0.0f;  // a padded token leaves the state as it is
        if (deltas) {
          float pr0 = 0.0f, pr1 = 0.0f;
#pragma unroll
          for (int m = 0; m < RPL; m += 2) {
            pr0 = fmaf(S[m], kf[m], pr0);
            if (m + 1 < RPL) pr1 = fmaf(S[m + 1], kf[m + 1], pr1);
          }
          delta = beta * (vv - group_sum<R>(pr0 + pr1));
        }
#pragma unroll
        for (int m = 0; m < RPL; m += 2) {
          S[m] = fmaf(kf[m], delta, S[m]);
          po0 = fmaf(S[m], qf[m], po0);
          if (m + 1 < RPL) {
            S[m + 1] = fmaf(kf[m + 1], delta, S[m + 1]);
            po1 = fmaf(S[m + 1], qf[m + 1], po1);
          }
        }
      } else {
        const float alpha = (decays && live) ? readlane(blk_alpha, rel) : 1.0f;
        // retrieval against the decayed state: r = alpha * (S^T k)
        float delta = live ? vv : 0.0f;  // a padded token leaves the state as it is
        if (deltas) {
          float pr0 = 0.0f, pr1 = 0.0f;
#pragma unroll
          for (int m = 0; m < RPL; m += 2) {
            pr0 = fmaf(S[m], kf[m], pr0);
            if (m + 1 < RPL) pr1 = fmaf(S[m + 1], kf[m + 1], pr1);
          }
          const float rsum = group_sum<R>(pr0 + pr1);
          delta = beta * (vv - alpha * rsum);
        }
        // decay + rank-1 update, and the readout partial of the updated state
#pragma unroll
        for (int m = 0; m < RPL; m += 2) {
          S[m] = fmaf(S[m], alpha, kf[m] * delta);
          po0 = fmaf(S[m], qf[m], po0);
          if (m + 1 < RPL) {
            S[m + 1] = fmaf(S[m + 1], alpha, kf[m + 1] * delta);
            po1 = fmaf(S[m + 1], qf[m + 1], po1);
          }
        }
      }
      const float o = group_sum<R>(po0 + po1) * scale;
      if (og != nullptr && r == 0 && col_ok && live)
        narrow_store(og + static_cast<size_t>(t) * v_stride + v_off, o);
      const int w = (t - t_begin) - hist_from;
      if (W > 0 && w >= 0 && col_ok && live) {
#pragma unroll
        for (int m = 0; m < RPL; ++m)
          if (row0 + m < p.d_k) history_slot(w)[static_cast<size_t>(row0 + m) * p.d_v + j] = S[m];
      }
    }
  }

  // ---- final state
  if (p.sN != nullptr && has_state && col_ok) {
#pragma unroll
    for (int m = 0; m < RPL; ++m) {
      const int i = row0 + m;
      if (i < p.d_k) p.sN[sbase + static_cast<size_t>(i) * p.d_v + j] = S[m];
    }
  }
}

// The plain gated delta rule with every row present (d_k = 128 or 256): CPW
// state columns per wave, R = 64 / CPW lanes per column, RPL = DK / R rows per
// lane.  Against scan_kernel:
//   * the readout reduction of token t and the retrieval reduction of token
//     t + 1 (both read the state after token t) run interleaved, so the
//     dependent steps of one fill the other's hazard slots;
//   * q/k/v addresses are wave-uniform bases advanced token by token plus a
//     fixed lane offset, with no per-token 64-bit products;
//   * whole 64-token blocks run without bounds checks; the last block or two
//     run a guarded copy, P tokens at a time;
//   * a block's 64 outputs of a column leave in one store, lane u holding
//     token u's;
//   * the column blocks of a (sequence, head) are placed on one XCD.
// d_k = 256 takes two columns per wave (32 lanes, 8 rows each) and 16 tokens
// in flight: with one wave per SIMD, load latency would otherwise set the
// pace.  d_k = 128 keeps scan_kernel's four columns per wave (16 lanes, 8
// rows each, no lane swaps) and 8 tokens in flight.
template <int DK>
struct PlainShape {
  static constexpr int CPW = DK >= 256 ? 2 : 4;  // columns per wave
  static constexpr int P = DK >= 256 ? 16 : 8;   // tokens of q/k/v in flight (ring slots)
  static constexpr int R = kWave / CPW;          // lanes per column
  static constexpr int RPL = DK / R;             // rows per lane
};

template <typename IO, bool RAW, int DK>
__global__ __launch_bounds__(kWave) void scan_plain_kernel(ScanParams p) {
  static_assert(DK == 128 || DK == 256, "the plain scan covers d_k = 128 and 256");
  constexpr int CPW = PlainShape<DK>::CPW;
  constexpr int R = PlainShape<DK>::R;
  constexpr int RPL = PlainShape<DK>::RPL;
  constexpr int P = PlainShape<DK>::P;
  const int lane = static_cast<int>(threadIdx.x);
  const int c = lane / R;  // column within the wave
  // blocks go round-robin over the 8 XCDs: the column blocks of one (sequence,
  // head) unit are placed 8 apart, on one XCD, so its q/k rows come from that
  // XCD's L2 for all of them
  const int xcd = static_cast<int>(blockIdx.x) % 8, rr = static_cast<int>(blockIdx.x) / 8;
  const int unit = (rr / p.col_blocks) * 8 + xcd;
  const int cb = rr % p.col_blocks;
  if (unit >= p.num_seqs * p.h_v) return;  // the grid is padded to whole rounds of 8 units
  const int h = unit % p.h_v;
  const int n = unit / p.h_v;
  const int hq = h / p.ratio;
  const int j = cb * CPW + c;
  const bool col_ok = j < p.d_v;
  const int row0 = (lane % R) * RPL;
  const int t_begin = p.cu[n];
  const int t_end = p.cu[n + 1];

  bool has_state;
  const int sidx = state_slot(p.slots, p.num_slots, n, &has_state);
  const size_t sbase = (static_cast<size_t>(sidx) * p.h_v + h) * static_cast<size_t>(DK) * p.d_v;
  float S[RPL];
#pragma unroll
  for (int m = 0; m < RPL; ++m)
    S[m] = (p.s0 != nullptr && has_state && col_ok) ? p.s0[sbase + static_cast<size_t>(row0 + m) * p.d_v + j] : 0.0f;

  if (t_end > t_begin) {
    const IO* __restrict__ qg = static_cast<const IO*>(p.q);
    const IO* __restrict__ kg = static_cast<const IO*>(p.k);
    const IO* __restrict__ vg = static_cast<const IO*>(p.v);
    IO* __restrict__ og = static_cast<IO*>(p.out);
    const size_t qk_stride = static_cast<size_t>(p.h_qk) * DK;
    const size_t v_stride = static_cast<size_t>(p.h_v) * p.d_v;
    const IO* kbase = kg + static_cast<size_t>(hq) * DK;
    const IO* qbase = qg + static_cast<size_t>(hq) * DK;
    const IO* vbase = vg + static_cast<size_t>(h) * p.d_v + cb * CPW;  // + the lane's column
    const int vcol = col_ok ? c : 0;
    const float scale = p.scale;

    // gates: lane l of a block holds token blk + l (loaded clamped one block ahead)
    const IO* __restrict__ ga = static_cast<const IO*>(RAW ? p.gates.a : p.gates.g);
    const IO* __restrict__ gb = static_cast<const IO*>(RAW ? p.gates.b : p.gates.beta);
    const float A_log = RAW ? p.gates.A_log[h] : 0.0f;
    const float dt_bias = RAW ? p.gates.dt_bias[h] : 0.0f;
    RawScalar<IO> next_ga, next_gb;
    auto fetch_gate_block = [&](int blk) __attribute__((always_inline)) {
      const int t = min(blk + lane, t_end - 1);
      next_ga.load(ga + static_cast<size_t>(t) * p.h_v + h);
      next_gb.load(gb + (p.gates.beta_shared ? static_cast<size_t>(t) : static_cast<size_t>(t) * p.h_v + h));
    };
    float blk_alpha = 1.0f, blk_beta = 0.0f;
    auto open_block = [&](int blk) __attribute__((always_inline)) {
      if constexpr (RAW) {
        blk_alpha = expf(gate_log_decay(next_ga.value(), A_log, dt_bias));
        blk_beta = gate_sigmoid(next_gb.value());
      } else {
        blk_alpha = expf(next_ga.value());
        blk_beta = next_gb.value();
      }
      fetch_gate_block(blk + kWave);
    };

    // q/k/v ring: slot (t - t_begin) % P holds token t
    RawSlice<IO, RPL> ring_k[P], ring_q[P];
    RawScalar<IO> ring_v[P];
    auto load_token = [&](int s, int t) __attribute__((always_inline)) {
      ring_k[s].load(kbase + static_cast<size_t>(t) * qk_stride + row0);
      ring_q[s].load(qbase + static_cast<size_t>(t) * qk_stride + row0);
      ring_v[s].load(vbase + static_cast<size_t>(t) * v_stride + vcol);
    };
    fetch_gate_block(t_begin);
#pragma unroll
    for (int s = 0; s < P; ++s) load_token(s, min(t_begin + s, t_end - 1));

    // two-chain partial dot product of the lane's rows
    auto dot = [&](const float* x) __attribute__((always_inline)) {
      float a = S[0] * x[0], b = S[1] * x[1];
#pragma unroll
      for (int m = 2; m < RPL; m += 2) {
        a = fmaf(S[m], x[m], a);
        b = fmaf(S[m + 1], x[m + 1], b);
      }
      return a + b;
    };
    // retrieval of the first token
    float rcur;
    {
      float kf[RPL];
      ring_k[0].widen_to(kf);
      rcur = group_sum<R>(dot(kf));
    }
    float o_acc[CPW];  // column c, lane u: output of token blk + u
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc) o_acc[cc] = 0.0f;

    // one token: update with rcur, then the readout of t and the retrieval of t + 1
    auto token = [&](int s, int rel, bool live) __attribute__((always_inline)) {
      const float beta = live ? readlane(blk_beta, rel) : 0.0f;
      const float alpha = live ? readlane(blk_alpha, rel) : 1.0f;
      float kf[RPL], qf[RPL], kn[RPL];
      ring_k[s].widen_to(kf);
      ring_q[s].widen_to(qf);
      const float vv = ring_v[s].value();
      const float delta = live ? beta * (vv - alpha * rcur) : 0.0f;
#pragma unroll
      for (int m = 0; m < RPL; ++m) S[m] = fmaf(S[m], alpha, kf[m] * delta);
      ring_k[(s + 1) % P].widen_to(kn);
      float po = dot(qf), pn = dot(kn);
      group_sum2<R>(po, pn);
      // the column sums into lane rel of the output registers (read first:
      // a lane read inside the select would make it a branch)
#pragma unroll
      for (int cc = 0; cc < CPW; ++cc) {
        const float val = readlane(po, cc * R) * scale;
        o_acc[cc] = (lane == rel) ? val : o_acc[cc];
      }
      rcur = pn;
    };
    auto store_block = [&](int blk) __attribute__((always_inline)) {
      if (og != nullptr && blk + lane < t_end) {
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc)
          if (cb * CPW + cc < p.d_v)
            narrow_store(og + static_cast<size_t>(blk + lane) * v_stride + static_cast<size_t>(h) * p.d_v + cb * CPW + cc,
                         o_acc[cc]);
      }
    };

    int blk = t_begin;
    // ---- whole blocks: every token and every prefetch (t + P) lies inside the sequence
    {
      // wave-uniform token bases; the lane's rows and column are fixed offsets from them
      const IO* pk = kbase + static_cast<size_t>(t_begin + P) * qk_stride;
      const IO* pq = qbase + static_cast<size_t>(t_begin + P) * qk_stride;
      const IO* pv = vbase + static_cast<size_t>(t_begin + P) * v_stride;
      for (; blk + kWave + P <= t_end; blk += kWave) {
        open_block(blk);
        // eight tokens per iteration (one turn of the ring): a short loop body
        // stays in the instruction cache
        for (int g8 = 0; g8 < kWave; g8 += P) {
#pragma unroll
          for (int u = 0; u < P; ++u) {
            token(u, g8 + u, true);
            // the slot just consumed takes token t + P
            ring_k[u].load(pk + row0);
            ring_q[u].load(pq + row0);
            ring_v[u].load(pv + vcol);
            pk += qk_stride;
            pq += qk_stride;
            pv += v_stride;
          }
        }
        store_block(blk);
      }
    }
    // ---- the rest, eight tokens at a time: padded tokens leave the state
    //      as it is, prefetches are clamped to the last token
    for (; blk < t_end; blk += kWave) {
      open_block(blk);
      for (int g8 = 0; g8 < kWave && blk + g8 < t_end; g8 += P) {
#pragma unroll
        for (int u = 0; u < P; ++u) {
          const int t = blk + g8 + u;
          token(u, g8 + u, t < t_end);
          load_token(u, min(t + P, t_end - 1));
        }
      }
      store_block(blk);
    }
  }

  if (p.sN != nullptr && has_state && col_ok) {
#pragma unroll
    for (int m = 0; m < RPL; ++m) p.sN[sbase + static_cast<size_t>(row0 + m) * p.d_v + j] = S[m];
  }
}

// Whether a launch takes scan_plain_kernel (the plain rule, d_k = 128 or 256).
// At d_k = 128 only small grids take it (at most two waves per SIMD): larger
// ones hide latency with scan_kernel's higher occupancy instead (measured on
// the 8-sequence, 33k-token workload).
bool plain_scan(const ScanParams& p) {
  const bool per_key = p.gates.per_key && p.gates.decays;
  const bool plain = p.gates.decays && p.gates.deltas && p.window == 0;
  if (!plain || per_key) return false;
  if (p.d_k == 256) return true;
  if (p.d_k != 128) return false;
  const int64_t waves = static_cast<int64_t>(p.num_seqs) * p.h_v * ((p.d_v + PlainShape<128>::CPW - 1) / PlainShape<128>::CPW);
  return waves <= 2 * 4 * static_cast<int64_t>(device_compute_units());
}

template <typename IO, int DK, bool RAW>
hipError_t launch_gates(const ScanParams& p, unsigned blocks, hipStream_t stream) {
  const bool per_key = p.gates.per_key && p.gates.decays;
  const bool plain = p.gates.decays && p.gates.deltas && p.window == 0;
  if constexpr (DK == 256 || DK == 128) {
    if (plain_scan(p)) {
      hipLaunchKernelGGL((scan_plain_kernel<IO, RAW, DK>), dim3(blocks), dim3(kWave), 0, stream, p);
      return hipGetLastError();
    }
  }
  if (per_key)
    hipLaunchKernelGGL((scan_kernel<IO, DK, RAW, true, true, false>), dim3(blocks), dim3(kWave), 0, stream, p);
  else if (plain && p.d_k == DK)
    hipLaunchKernelGGL((scan_kernel<IO, DK, RAW, false, false, true>), dim3(blocks), dim3(kWave), 0, stream, p);
  else if (plain)
    hipLaunchKernelGGL((scan_kernel<IO, DK, RAW, false, false, false>), dim3(blocks), dim3(kWave), 0, stream, p);
  else
    hipLaunchKernelGGL((scan_kernel<IO, DK, RAW, false, true, false>), dim3(blocks), dim3(kWave), 0, stream, p);
  return hipGetLastError();
}

template <typename IO, int DK>
hipError_t launch_dk(const ScanParams& p, hipStream_t stream) {
  const int units = p.num_seqs * p.h_v;
  if (units == 0) return hipSuccess;
  const unsigned blocks = ((DK == 256 || DK == 128) && plain_scan(p))
                              ? static_cast<unsigned>((units + 7) / 8) * 8u * p.col_blocks
                              : static_cast<unsigned>(units) * p.col_blocks;
  if (blocks == 0) return hipSuccess;
  return p.gates.raw ? launch_gates<IO, DK, true>(p, blocks, stream) : launch_gates<IO, DK, false>(p, blocks, stream);
}

template <typename IO>
hipError_t launch_io(const ScanParams& p, hipStream_t stream) {
  if (p.d_k <= 16) return launch_dk<IO, 16>(p, stream);
  if (p.d_k <= 32) return launch_dk<IO, 32>(p, stream);
  if (p.d_k <= 64) return launch_dk<IO, 64>(p, stream);
  if (p.d_k <= 128) return launch_dk<IO, 128>(p, stream);
  return launch_dk<IO, 256>(p, stream);
}

}  // namespace

bool scan_takes_plain_kernel(const ScanParams& p) { return plain_scan(p); }

int scan_columns_per_wave(const ScanParams& p) {
  const int d_k = p.d_k;
  if (plain_scan(p)) return d_k == 256 ? PlainShape<256>::CPW : PlainShape<128>::CPW;
  if (d_k <= 16) return kWave / ScanShape<16>::R;
  if (d_k <= 32) return kWave / ScanShape<32>::R;
  if (d_k <= 64) return kWave / ScanShape<64>::R;
  if (d_k <= 128) return kWave / ScanShape<128>::R;
  return kWave / ScanShape<256>::R;
}

hipError_t launch_prefill_scan(ScanParams p, int io_dtype, hipStream_t stream) {
  if (io_dtype == 1) return launch_io<bf16_t>(p, stream);
  if (io_dtype == 2) return launch_io<f16_t>(p, stream);
  return launch_io<float>(p, stream);
}

}  // namespace gdn
