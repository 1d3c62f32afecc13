// prefill_chunked.hip -- chunked prefill of the gated delta rule on gfx950
// MFMA (bf16 operands, f32 accumulation).
//
// The pages run the recurrence token by token and decline a chunked ("WY")
// form because nothing in a node's shape guarantees normalised keys or a
// bounded decay ([P1] onnxruntime-ep-mlx, src/ops/ssm.rs, module doc and the
// scan kernel's comment).  This path is the chunked form of the same
// recurrence, derived from it, for callers whose decay is a true decay
// (g <= 0) -- which the raw-gate prologue always produces.
//
// Derivation.  With alpha_t = exp(g_t) the update of [P4] onnx-runtime-ep-cuda,
// src/kernels/linear_attention.rs, `linear_attention_core` steps 1-4 reads
//     S_t = alpha_t S_{t-1} + k_t d_t^T,   d_t = beta_t (v_t - alpha_t S_{t-1}^T k_t),
//     o_t = scale S_t^T q_t.
// Inside a chunk of C tokens starting from S_0, let G_t = g_1 + ... + g_t and
// gam_t = exp(G_t).  Unrolling,
//     S_t = gam_t S_0 + sum_{s<=t} exp(G_t - G_s) k_s d_s^T,
// so d_t = beta_t v_t - beta_t gam_t S_0^T k_t - sum_{s<t} beta_t exp(G_t - G_s) (k_t.k_s) d_s,
// i.e. (I + A) D = diag(beta) V - diag(beta gam) K S_0 with the strictly lower
// A_ts = beta_t exp(G_t - G_s) k_t.k_s.  With T = (I + A)^-1:
//     D   = U - W S_0,        U = T diag(beta) V,   W = T diag(beta gam) K
// (the gated and linear rules have no delta correction: A = 0, U = V, W = 0)
//     O   = scale (diag(gam) Q S_0 + M D),   M_ts = exp(G_t - G_s) q_t.k_s  (s <= t)
//     S_C = gam_C S_0 + K^T diag(exp(G_C - G_s)) D.
// Every exponent is a sum of log-decays over a forward range, so with g <= 0
// every factor lies in [0, 1].  g is clamped below at -1e4 (exp of it is 0 in
// float) so that a g of -infinity (a reset) never forms inf - inf.
//
// Mapping.  One workgroup (8 waves, two per SIMD) owns NC columns of the state of one
// (sequence, value head) and walks the sequence chunk by chunk; the state
// slice S (DK x NC, f32) stays in MFMA accumulator registers across chunks.
// Per chunk, all operands are staged in LDS with k contiguous so that every
// MFMA operand fragment is one 16-byte LDS read:
//   1. store K, Q (rows), K^T, V^T (columns of this block) and the gates of
//      the chunk, which were loaded into registers during the previous chunk,
//      then start loading the next chunk; prefix-sum G (log2 units) in double;
//   2. P = K K^T and R = Q K^T (MFMA), tile by tile, with one exp2 per
//      (t, s) shared by both -> A (f32) and M (bf16);
//   3. T = (I + A)^-1: 16x16 diagonal blocks by forward substitution in f32,
//      off-diagonal blocks by block substitution with f32 MFMA;
//   4. W = T diag(beta gam) K and U = T diag(beta) V (MFMA);
//   5. X = W S and Y = Q S (MFMA); D = U - X;
//   6. O = scale (gam Y + M D) -> out;  S <- gam_C S + K^T (exp(G_C - G) D).
// Operands are rounded to bf16 for the MFMA (products accumulate in f32); the
// state itself is carried in f32.
#include "chunk_mfma.hpp"
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

namespace {


constexpr int kC = 64;          // chunk length (tokens)
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kSC = kC + 8;     // bf16 row stride of C-long rows
constexpr int kSA = kC + 8;     // f32 row stride of A (its buffer later holds T' and T'' in bf16)
constexpr int kST = kC + 4;     // f32 row stride of T
constexpr float kMinLogDecay = -1.0e4f;
constexpr double kLog2e = 1.4426950408889634;


template <int DK, int NC>
struct Lds {
  static constexpr int SK = DK + 8;  // bf16 row stride of DK-long rows
  // byte offsets
  static constexpr int kKs = 0;                              // K rows   [C][SK] bf16 (later W)
  static constexpr int kQs = kKs + kC * SK * 2;              // Q rows   [C][SK] bf16
  static constexpr int kKT = kQs + kC * SK * 2;              // K^T      [DK][SC] bf16
  static constexpr int kVt = kKT + DK * kSC * 2;             // V^T      [NC][SC] bf16 (beta applied later via T)
  static constexpr int kAf = kVt + NC * kSC * 2;             // A        [C][SA] f32 (later T' and T'' bf16)
  static constexpr int kTf = kAf + kC * kSA * 4;             // T        [C][ST] f32
  static constexpr int kMs = kTf + kC * kST * 4;             // M        [C][SC] bf16
  static constexpr int kSt = kMs + kC * kSC * 2;             // S^T      [NC][SK] bf16
  static constexpr int kDt = kSt + NC * SK * 2;              // D^T      [NC][SC] bf16
  static constexpr int kDtt = kDt + NC * kSC * 2;            // (exp(G_C - G) D)^T [NC][SC] bf16
  static constexpr int kXs = kDtt + NC * kSC * 2;            // solve scratch [4 waves][16][20] f32
  static constexpr int kGd = kXs + 4 * 16 * 20 * 4;          // G        [C] f64
  static constexpr int kGam = kGd + kC * 8;                  // gam      [C] f32
  static constexpr int kBet = kGam + kC * 4;                 // beta     [C] f32
  static constexpr int kBytes = kBet + kC * 4;
  static_assert(2 * kC * kSC * 2 <= kC * kSA * 4, "T' and T'' must fit in the A buffer");
  static_assert(kBytes <= 160 * 1024, "LDS budget of one gfx950 workgroup");
};

template <typename IO, int DK, int NC, bool RAW>
__global__ __launch_bounds__(kThreads) void chunk_kernel(ScanParams p) {
  using L = Lds<DK, NC>;
  constexpr int SK = L::SK;
  constexpr int CT = NC / 16;                  // column tiles of the block
  constexpr int CTW = CT / 2;                  // column tiles per wave in the (token, column) products
  constexpr int KTW = DK / 32;                 // key tiles per wave in W = T' K
  constexpr int STW = (DK / 16) * CT / kWaves; // state tiles per wave
  static_assert(CT % 2 == 0 && STW >= 1, "block shape");
  extern __shared__ __align__(16) unsigned char smem[];
  bf16_t* Ks = reinterpret_cast<bf16_t*>(smem + L::kKs);
  bf16_t* Ws = Ks;  // W overwrites K once P, R and K^T are formed
  bf16_t* Qs = reinterpret_cast<bf16_t*>(smem + L::kQs);
  bf16_t* KT = reinterpret_cast<bf16_t*>(smem + L::kKT);
  bf16_t* Vt = reinterpret_cast<bf16_t*>(smem + L::kVt);
  float* Af = reinterpret_cast<float*>(smem + L::kAf);
  bf16_t* Tp = reinterpret_cast<bf16_t*>(smem + L::kAf);                  // T diag(beta gam)
  bf16_t* Tpp = reinterpret_cast<bf16_t*>(smem + L::kAf + kC * kSC * 2);  // T diag(beta)
  float* Tf = reinterpret_cast<float*>(smem + L::kTf);
  bf16_t* Ms = reinterpret_cast<bf16_t*>(smem + L::kMs);
  bf16_t* St = reinterpret_cast<bf16_t*>(smem + L::kSt);
  bf16_t* Dt = reinterpret_cast<bf16_t*>(smem + L::kDt);
  bf16_t* Dtt = reinterpret_cast<bf16_t*>(smem + L::kDtt);
  float* Xs = reinterpret_cast<float*>(smem + L::kXs);
  double* Gd = reinterpret_cast<double*>(smem + L::kGd);
  float* Gam = reinterpret_cast<float*>(smem + L::kGam);
  float* Bet = reinterpret_cast<float*>(smem + L::kBet);

  const int tid = static_cast<int>(threadIdx.x);
  const int w = tid >> 6;
  const int lane = tid & 63;
  // this wave's row block (16 tokens) and column half in the (token, column) products
  const int rb = w & 3;
  const int chalf = w >> 2;
  int unit = static_cast<int>(blockIdx.x);
  const int cb = unit % p.col_blocks;
  unit /= p.col_blocks;
  const int h = unit % p.h_v;
  const int n = unit / p.h_v;
  const int hq = h / p.ratio;
  const int J0 = cb * NC;
  const int t_begin = p.cu[n];
  const int t_end = p.cu[n + 1];
  const int d_v = p.d_v;
  bool has_state;
  const int sidx = state_slot(p.slots, p.num_slots, n, &has_state);
  const size_t sbase = (static_cast<size_t>(sidx) * p.h_v + h) * static_cast<size_t>(DK) * d_v;

  // ---- state slice in accumulators: wave w owns state tiles w*STW .. w*STW+STW-1
  //      (tile index = row tile * CT + column tile)
  f32x4 S[STW];
#pragma unroll
  for (int e = 0; e < STW; ++e) {
    const int ri = (w * STW + e) / CT, cj = (w * STW + e) % CT;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * ri + acc_row(lane, i);
      const int col = J0 + 16 * cj + acc_col(lane);
      S[e][i] = (p.s0 != nullptr && has_state && col < d_v) ? p.s0[sbase + static_cast<size_t>(row) * d_v + col]
                                                             : 0.0f;
    }
  }
  auto publish_state = [&]() {  // S^T (bf16) for the next chunk's X = W S and Y = Q S
#pragma unroll
    for (int e = 0; e < STW; ++e) {
      const int ri = (w * STW + e) / CT, cj = (w * STW + e) % CT;
      const int row = 16 * ri + acc_row(lane, 0);
      const int col = 16 * cj + acc_col(lane);
      uint2 pk;
      pk.x = static_cast<uint32_t>(to_bf16(S[e][0])) | (static_cast<uint32_t>(to_bf16(S[e][1])) << 16);
      pk.y = static_cast<uint32_t>(to_bf16(S[e][2])) | (static_cast<uint32_t>(to_bf16(S[e][3])) << 16);
      *reinterpret_cast<uint2*>(St + col * SK + row) = pk;
    }
  };
  publish_state();

  const IO* qg = static_cast<const IO*>(p.q);
  const IO* kg = static_cast<const IO*>(p.k);
  // Rules without the delta correction (gated, linear) write v as it is:
  // A = 0, so T = I, with weight 1 in T'' = T diag(beta), T' = 0, and D = V.
  const bool delta_rule = p.gates.deltas != 0;
  const IO* vg = static_cast<const IO*>(p.v);
  IO* og = static_cast<IO*>(p.out);
  const size_t qk_stride = static_cast<size_t>(p.h_qk) * DK;
  const size_t v_stride = static_cast<size_t>(p.h_v) * d_v;
  float A_log = 0.0f, dt_bias = 0.0f;
  if constexpr (RAW) {
    if (t_begin < t_end && p.gates.decays) {
      A_log = p.gates.A_log[h];
      dt_bias = p.gates.dt_bias[h];
    }
  }

  // the upper tiles of M are never written per chunk: zero them once (M is an
  // MFMA operand over its full k range)
  for (int e = tid; e < 6 * 256; e += kThreads) {
    const int tile = e >> 8;
    const int tb = tile < 3 ? 0 : (tile < 5 ? 1 : 2);
    const int cs = tile < 3 ? tile + 1 : (tile < 5 ? tile - 1 : 3);
    const int t = 16 * tb + ((e & 255) >> 4), s = 16 * cs + (e & 15);
    Ms[t * kSC + s] = 0;
  }

  // ---- register staging of one chunk's inputs (loaded one chunk ahead)
  constexpr int VPR = DK / 8;                              // 8-element vectors per K/Q row
  constexpr int KQ_IT = kC * VPR / kThreads;               // vectors per thread
  constexpr int VPV = NC / 8;                              // 8-element vectors per V row
  // V rows are staged in token pairs: (pair, 8 columns) items, two rows each
  constexpr int V_PAIRS = (kC / 2) * VPV;
  constexpr int V_IT = (V_PAIRS + kThreads - 1) / kThreads;
  static_assert(KQ_IT >= 1, "block shape");
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  u32x4 rk[KQ_IT], rq[KQ_IT], rv[2 * V_IT];
  // gate inputs of token (chunk start + lane) as raw 16-bit patterns, widened
  // where they are used
  uint32_t rg = 0u, rb_ = 0u;
  // Unconditional (clamped) loads: a load under a condition becomes a choice
  // between old and new values that the compiler settles with a copy waiting
  // for the load right after it is issued.  Rows past the chunk and columns
  // past d_v are zeroed when staged.
  auto fetch = [&](int c0) {
    const int Ln = (t_end - c0) < kC ? (t_end - c0) : kC;
#pragma unroll
    for (int it = 0; it < KQ_IT; ++it) {
      const int v = tid + it * kThreads;
      const int t = min(v / VPR, Ln - 1);
      const int c8 = (v % VPR) * 8;
      const size_t off = static_cast<size_t>(c0 + t) * qk_stride + static_cast<size_t>(hq) * DK + c8;
      rk[it] = *reinterpret_cast<const u32x4*>(kg + off);
      rq[it] = *reinterpret_cast<const u32x4*>(qg + off);
    }
#pragma unroll
    for (int it = 0; it < V_IT; ++it) {
      const int v = min(tid + it * kThreads, V_PAIRS - 1);
      const int t = 2 * (v % (kC / 2));
      const int col = min(J0 + (v / (kC / 2)) * 8, d_v - 8);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        rv[2 * it + hh] = *reinterpret_cast<const u32x4*>(vg + static_cast<size_t>(c0 + min(t + hh, Ln - 1)) * v_stride +
                                                         static_cast<size_t>(h) * d_v + col);
    }
    {
      const int tl = c0 + min(lane, Ln - 1);
      const size_t gi = static_cast<size_t>(tl) * p.h_v + h;
      const size_t bi = p.gates.beta_shared ? static_cast<size_t>(tl) : gi;
      // a gate the rule does not use reads K's first element instead (its
      // pointer may be null), so the loads stay unconditional
      const IO* bsrc = delta_rule ? static_cast<const IO*>(RAW ? p.gates.b : p.gates.beta) : kg;
      const size_t bix = delta_rule ? bi : 0;
      const IO* gsrc = p.gates.decays ? static_cast<const IO*>(RAW ? p.gates.a : p.gates.g) : bsrc;
      rg = reinterpret_cast<const uint16_t*>(gsrc)[p.gates.decays ? gi : bix];
      rb_ = reinterpret_cast<const uint16_t*>(bsrc)[bix];
    }
  };
  if (t_begin < t_end) fetch(t_begin);

  for (int t0 = t_begin; t0 < t_end; t0 += kC) {
    const int L = (t_end - t0) < kC ? (t_end - t0) : kC;

    // ================= 1. stage the chunk in LDS, start loading the next one
#pragma unroll
    for (int it = 0; it < KQ_IT; ++it) {
      const int v = tid + it * kThreads;
      const int t = v / VPR;
      const int c8 = (v % VPR) * 8;
      const u32x4 zero = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(Ks + t * SK + c8) = t < L ? rk[it] : zero;
      *reinterpret_cast<u32x4*>(Qs + t * SK + c8) = t < L ? rq[it] : zero;
    }
    // V^T from token pairs: one 4-byte word (tokens t, t + 1) per column; the
    // 32 pairs of a wave fill 32 consecutive words and its two 8-column groups
    // sit 32 banks apart, so the writes are free of bank conflicts
#pragma unroll
    for (int it = 0; it < V_IT; ++it) {
      const int v = tid + it * kThreads;
      if (v < V_PAIRS) {
        const int t = 2 * (v % (kC / 2)), c8 = (v / (kC / 2)) * 8;
        const bool col_ok = J0 + c8 < d_v;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t a = (col_ok && t < L) ? ((e & 1) ? (rv[2 * it][e >> 1] >> 16) : (rv[2 * it][e >> 1] & 0xffffu)) : 0u;
          const uint32_t b = (col_ok && t + 1 < L) ? ((e & 1) ? (rv[2 * it + 1][e >> 1] >> 16) : (rv[2 * it + 1][e >> 1] & 0xffffu)) : 0u;
          *reinterpret_cast<uint32_t*>(Vt + (c8 + e) * kSC + t) = a | (b << 16);
        }
      }
    }
    // gates and the in-chunk prefix sum of the log-decay, in log2 units (wave 0, lane = token)
    if (w == 0) {
      float g = 0.0f, b = 0.0f;
      if (lane < L) {
        if constexpr (RAW) {
          g = p.gates.decays ? gate_log_decay(widen_bits16<IO>(rg), A_log, dt_bias) : 0.0f;
          b = delta_rule ? gate_sigmoid(widen_bits16<IO>(rb_)) : 1.0f;
        } else {
          g = p.gates.decays ? widen_bits16<IO>(rg) : 0.0f;
          b = delta_rule ? widen_bits16<IO>(rb_) : 1.0f;
        }
        g = fmaxf(g, kMinLogDecay);
      }
      const double G = wave_prefix_sum(static_cast<double>(g) * kLog2e, lane);
      Gd[lane] = G;
      Gam[lane] = fast_exp2(static_cast<float>(G));
      Bet[lane] = b;
    }
    if (t0 + kC < t_end) fetch(t0 + kC);  // in flight while this chunk computes
    __syncthreads();

    // ================= 2. P = K K^T, R = Q K^T -> A (f32) and M (bf16); K^T
    // K^T from the staged rows (needed from step 4 on): item (i, 8 tokens) reads
    // a column segment of K (consecutive i across lanes: no bank conflicts) and
    // writes it as one 16-byte row segment of K^T
#pragma unroll
    for (int it = 0; it < DK * (kC / 8) / kThreads; ++it) {
      const int item = tid + it * kThreads;
      const int i = item % DK;
      const int t8 = (item / DK) * 8;
      uint32_t wv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        wv[e] = static_cast<uint32_t>(Ks[(t8 + 2 * e) * SK + i]) |
                (static_cast<uint32_t>(Ks[(t8 + 2 * e + 1) * SK + i]) << 16);
      *reinterpret_cast<uint4*>(KT + i * kSC + t8) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    }
    // the 10 lower tiles (tb >= cs), dealt round-robin to the waves; P and R of a
    // tile share the decay factor exp(G_t - G_s)
    for (int tj = w; tj < 10; tj += kWaves) {
      int tb = 0;
      while ((tb + 1) * (tb + 2) / 2 <= tj) ++tb;
      const int cs = tj - tb * (tb + 1) / 2;
      f32x4 pacc = {0.0f, 0.0f, 0.0f, 0.0f}, racc = {0.0f, 0.0f, 0.0f, 0.0f};
      pacc = mma<DK>(pacc, Ks + 16 * tb * SK, SK, Ks + 16 * cs * SK, SK, lane);
      racc = mma<DK>(racc, Qs + 16 * tb * SK, SK, Ks + 16 * cs * SK, SK, lane);
      const int s_ = 16 * cs + acc_col(lane);
      const double Gs = Gd[s_];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * tb + acc_row(lane, i);
        const float dec = (s_ <= t) ? fast_exp2(static_cast<float>(Gd[t] - Gs)) : 0.0f;
        Af[t * kSA + s_] = (s_ < t && delta_rule) ? Bet[t] * dec * pacc[i] : 0.0f;
        Ms[t * kSC + s_] = to_bf16(dec * racc[i]);
      }
    }
    __syncthreads();

    // ================= 3. T = (I + A)^-1
    // 3a. diagonal block w (waves 0-3) by forward substitution (lane c < 16 owns column c)
    if (w < 4) {
      const int c = lane & 15;
      const float* Ab = Af + (16 * w) * kSA + 16 * w;
      float d[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x0 = (r == c) ? 1.0f : 0.0f, x1 = 0.0f;
#pragma unroll
        for (int s2 = 0; s2 < r; s2 += 2) {
          x0 = fmaf(-Ab[r * kSA + s2], d[s2], x0);
          if (s2 + 1 < r) x1 = fmaf(-Ab[r * kSA + s2 + 1], d[s2 + 1], x1);
        }
        d[r] = x0 + x1;
      }
      if (lane < 16) {
#pragma unroll
        for (int r = 0; r < 16; ++r) Tf[(16 * w + r) * kST + 16 * w + c] = d[r];
      }
    }
    __syncthreads();
    // 3b. off-diagonal blocks, by distance from the diagonal:
    //     T_ij = -D_i sum_{k=j}^{i-1} A_ik T_kj
    for (int dist = 1; dist < 4; ++dist) {
      const int i = w + dist, j = w;
      if (i < 4) {
        f32x4 x = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int k = j; k < i; ++k)
          x = mma_f32(x, Af + (16 * i) * kSA + 16 * k, kSA, Tf + (16 * k) * kST + 16 * j, kST, lane);
        float* xs = Xs + w * 16 * 20;
#pragma unroll
        for (int e = 0; e < 4; ++e) xs[acc_row(lane, e) * 20 + acc_col(lane)] = x[e];
        // the scratch tile is private to this wave: a wave-level barrier suffices
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        f32x4 y = {0.0f, 0.0f, 0.0f, 0.0f};
        y = mma_f32(y, Tf + (16 * i) * kST + 16 * i, kST, xs, 20, lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) Tf[(16 * i + acc_row(lane, e)) * kST + 16 * j + acc_col(lane)] = -y[e];
      }
      __syncthreads();
    }
    // 3c. T' = T diag(beta gam) and T'' = T diag(beta) in bf16, zero above the diagonal
    for (int e = tid; e < kC * kC; e += kThreads) {
      const int t = e >> 6, s2 = e & 63;
      const float tv = (s2 <= t) ? Tf[t * kST + s2] : 0.0f;
      const float bs = Bet[s2];
      Tp[t * kSC + s2] = to_bf16(delta_rule ? tv * bs * Gam[s2] : 0.0f);
      Tpp[t * kSC + s2] = to_bf16(tv * bs);
    }
    __syncthreads();

    // ================= 4. W = T' K (-> LDS), U = T'' V (registers)
    const int kmax = (rb < 2) ? 32 : 64;  // rows of block rb vanish for s >= 16 (rb + 1)
#pragma unroll
    for (int e = 0; e < KTW; ++e) {
      const int ci = chalf * KTW + e;
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      acc = mma_range(acc, Tp + (16 * rb) * kSC, kSC, KT + (16 * ci) * kSC, kSC, 0, kmax, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) Ws[(16 * rb + acc_row(lane, i)) * SK + 16 * ci + acc_col(lane)] = to_bf16(acc[i]);
    }
    f32x4 U[CTW];
#pragma unroll
    for (int e = 0; e < CTW; ++e) {
      const int cj = chalf * CTW + e;
      U[e] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      U[e] = mma_range(U[e], Tpp + (16 * rb) * kSC, kSC, Vt + (16 * cj) * kSC, kSC, 0, kmax, lane);
    }
    __syncthreads();

    // ================= 5. D = U - W S, Y = gam Q S
    f32x4 Y[CTW];
    const double GC = Gd[kC - 1];
#pragma unroll
    for (int e = 0; e < CTW; ++e) {
      const int cj = chalf * CTW + e;
      f32x4 x = {0.0f, 0.0f, 0.0f, 0.0f}, y = {0.0f, 0.0f, 0.0f, 0.0f};
      x = mma<DK>(x, Ws + (16 * rb) * SK, SK, St + (16 * cj) * SK, SK, lane);
      y = mma<DK>(y, Qs + (16 * rb) * SK, SK, St + (16 * cj) * SK, SK, lane);
      const int t = 16 * rb + acc_row(lane, 0);
      const int col = 16 * cj + acc_col(lane);
      float dl[4], dd[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dl[i] = U[e][i] - x[i];
        dd[i] = dl[i] * fast_exp2(static_cast<float>(GC - Gd[t + i]));
        Y[e][i] = Gam[t + i] * y[i];
      }
      uint2 pk;
      pk.x = static_cast<uint32_t>(to_bf16(dl[0])) | (static_cast<uint32_t>(to_bf16(dl[1])) << 16);
      pk.y = static_cast<uint32_t>(to_bf16(dl[2])) | (static_cast<uint32_t>(to_bf16(dl[3])) << 16);
      *reinterpret_cast<uint2*>(Dt + col * kSC + t) = pk;
      pk.x = static_cast<uint32_t>(to_bf16(dd[0])) | (static_cast<uint32_t>(to_bf16(dd[1])) << 16);
      pk.y = static_cast<uint32_t>(to_bf16(dd[2])) | (static_cast<uint32_t>(to_bf16(dd[3])) << 16);
      *reinterpret_cast<uint2*>(Dtt + col * kSC + t) = pk;
    }
    __syncthreads();

    // ================= 6. O = scale (Y + M D);  S <- gam_C S + K^T Dtt
#pragma unroll
    for (int e = 0; e < CTW; ++e) {
      const int cj = chalf * CTW + e;
      f32x4 o = Y[e];
      o = mma_range(o, Ms + (16 * rb) * kSC, kSC, Dt + (16 * cj) * kSC, kSC, 0, kmax, lane);
      if (og != nullptr) {
        const int col = J0 + 16 * cj + acc_col(lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * rb + acc_row(lane, i);
          if (t < L && col < d_v)
            narrow_store(og + static_cast<size_t>(t0 + t) * v_stride + static_cast<size_t>(h) * d_v + col,
                         p.scale * o[i]);
        }
      }
    }
    const float gamC = Gam[kC - 1];
#pragma unroll
    for (int e = 0; e < STW; ++e) {
      const int ri = (w * STW + e) / CT, cj = (w * STW + e) % CT;
      f32x4 acc = S[e] * gamC;
      acc = mma<kC>(acc, KT + (16 * ri) * kSC, kSC, Dtt + (16 * cj) * kSC, kSC, lane);
      S[e] = acc;
    }
    publish_state();
    __syncthreads();
  }

  // ---- final state
  if (p.sN != nullptr && has_state) {
#pragma unroll
    for (int e = 0; e < STW; ++e) {
      const int ri = (w * STW + e) / CT, cj = (w * STW + e) % CT;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * ri + acc_row(lane, i);
        const int col = J0 + 16 * cj + acc_col(lane);
        if (col < d_v) p.sN[sbase + static_cast<size_t>(row) * d_v + col] = S[e][i];
      }
    }
  }
}

template <typename IO, int DK, int NC, bool RAW>
hipError_t launch_variant(const ScanParams& p, hipStream_t stream) {
  auto kern = chunk_kernel<IO, DK, NC, RAW>;
  constexpr int bytes = Lds<DK, NC>::kBytes;
  const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), bytes);
  if (e != hipSuccess) return e;
  const unsigned blocks = static_cast<unsigned>(p.num_seqs) * p.h_v * p.col_blocks;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(kThreads), bytes, stream, p);
  return hipGetLastError();
}

template <typename IO, int DK, int NC>
hipError_t launch_nc(const ScanParams& p, hipStream_t stream) {
  return p.gates.raw ? launch_variant<IO, DK, NC, true>(p, stream) : launch_variant<IO, DK, NC, false>(p, stream);
}

}  // namespace

bool chunked_supported(int io_bf16, int d_k, int d_v, const GateArgs& gates, int window) {
  return io_bf16 && (d_k == 64 || d_k == 128) && d_v % 8 == 0 && !gates.per_key && window == 0;
}

int chunked_columns_per_block(int d_k, int d_v) {
  (void)d_k;
  return d_v >= 64 ? 64 : 32;
}

hipError_t launch_prefill_chunked(ScanParams p, int io_bf16, hipStream_t stream) {
  if (!chunked_supported(io_bf16, p.d_k, p.d_v, p.gates, p.window)) return hipErrorInvalidValue;
  const int nc = chunked_columns_per_block(p.d_k, p.d_v);
  if (p.d_k == 128) return nc == 64 ? launch_nc<bf16_t, 128, 64>(p, stream) : launch_nc<bf16_t, 128, 32>(p, stream);
  return nc == 64 ? launch_nc<bf16_t, 64, 64>(p, stream) : launch_nc<bf16_t, 64, 32>(p, stream);
}

}  // namespace gdn
