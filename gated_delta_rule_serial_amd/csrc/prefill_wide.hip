// prefill_wide.hip -- the two-pass chunked prefill for float32 I/O (gfx950
// MFMA, d_k 128 or 256).
//
// The chunked form is the one the bfloat16 two-pass prefill uses, derived
// from [P4] onnx-runtime-ep-cuda, src/kernels/linear_attention.rs,
// `linear_attention_core` steps 1-4.  Per chunk of C = 64 tokens (G_t the
// in-chunk prefix of the log-decay, gam_t = exp(G_t), T = (I + A)^-1 with the
// strictly lower A_ts = beta_t exp(G_t - G_s) k_t.k_s):
//     W  = T diag(beta gam) K          U = T diag(beta) V
//     M_ts = scale exp(G_t - G_s) q_t.k_s (s <= t)
//     Kt = diag(exp(G_last - G)) K
// depend on the chunk alone, while
//     D = U - W S,   O = scale diag(gam) Q S + M D,   S <- gam_last S + Kt^T D
// carry the state from chunk to chunk.  The gated and linear rules have no
// delta correction: A = 0, W = 0 and U = V, so D = V.
//
// Float32 I/O asks for float32-class products, which the bfloat16 matrix
// cores give when each operand x is split into hi = bf16(x) and
// lo = bf16(x - hi) and a product is formed from the three terms
// hi.hi + hi.lo + lo.hi (the dropped lo.lo is below 2^-16 of the product).
// Accumulation is float32 throughout, and the state is carried in float32
// MFMA accumulators.
//
// Pass 1 (wide_prep_kernel): one workgroup per (chunk, value head) computes
// W, scale diag(gam) Q, Kt^T and M as split operand fragments, U in float32
// and gam_last into a caller-provided workspace.  Pass 2 (wide_state_kernel): one
// workgroup of d_k / 32 waves per (sequence, value head, block of 16 state
// columns); wave w owns rows [32 w, 32 w + 32) of the state block and the
// partial products W S and Q S over its rows meet in LDS once per chunk.
#include "chunk_mfma.hpp"
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

namespace {

constexpr int kC = 64;            // chunk length (tokens)
constexpr int kThreads = 256;     // four waves (pass 1)
constexpr int kSF = kC + 4;       // f32 row stride of the 64 x 64 matrices in LDS
constexpr int kSH = kC + 8;       // bf16 row stride of the split T diag(beta) and T diag(beta gam)
constexpr float kMinLogDecay = -1.0e4f;
#ifndef WIDE_TOUCH_AHEAD
#define WIDE_TOUCH_AHEAD 3
#endif
constexpr int kTouchAhead = WIDE_TOUCH_AHEAD;  // chunks between a record's touch and its use
constexpr double kLog2e = 1.4426950408889634;

__host__ __device__ constexpr size_t align256w(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// One (chunk, value head) record.  Fragments are 1 KiB: the 64 lanes x 16
// bytes one wave loads as an operand of v_mfma_f32_16x16x32_bf16, hi part then
// lo part.  The contraction index inside each 32-wide block is permuted so
// that lane group g holds k = 4 g .. 4 g + 3 and 16 + 4 g .. 16 + 4 g + 3, the
// order in which two stacked accumulator tiles hold the other operand (state
// rows for W, the tokens of D for Kt^T and M).
//   w   [DK / 32 key blocks][4 token tiles][hi, lo]      rows: tokens, k: keys
//   qf  [DK / 32 key blocks][4 token tiles][hi, lo]      scale diag(gam) Q, as w
//   kt  [DK / 16 key tiles][2 token blocks][hi, lo]      rows: keys, k: tokens
//   ms  [6 lower blocks][hi, lo]                          rows: tokens, k: tokens
//   u   [d_v / 16 column tiles][4 token tiles][64 lanes][4] f32, accumulator order
//   gam gam_last (f32, in a 256-byte slot)
struct WideRec {
  size_t w, qf, kt, ms, u, gam, bytes;
  __host__ __device__ WideRec(int dk, int dv) {
    w = 0;
    qf = w + static_cast<size_t>(dk / 32) * 8 * 1024;
    kt = qf + static_cast<size_t>(dk / 32) * 8 * 1024;
    ms = kt + static_cast<size_t>(dk / 16) * 4 * 1024;
    u = ms + 12 * 1024;
    gam = u + static_cast<size_t>(dv / 16) * 4 * 1024;
    bytes = align256w(gam + 256);
  }
};

// M block (token tile tt, token block kb), kb <= tt / 2
__device__ __forceinline__ int m_block(int tt, int kb) { return tt < 2 ? tt : 2 + 2 * (tt - 2) + kb; }

__device__ __forceinline__ int wseq_lo(const int32_t* cu, int n, int T) { return min(max(cu[n], 0), T); }
__device__ __forceinline__ int wseq_hi(const int32_t* cu, int n, int T) {
  return min(max(cu[n + 1], wseq_lo(cu, n, T)), T);
}

struct Split8 {
  bf16x8 hi, lo;
};

// x = hi + lo + r with hi = bf16(x), lo = bf16(x - hi), |r| <= 2^-17 |x|
// (both roundings to nearest even).
__device__ __forceinline__ Split8 split8(const float (&x)[8]) {
  Split8 s;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 h = static_cast<__bf16>(x[e]);
    s.hi[e] = h;
    s.lo[e] = static_cast<__bf16>(x[e] - static_cast<float>(h));
  }
  return s;
}

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

// acc += A B from split operands: the two small cross terms first.
__device__ __forceinline__ f32x4 mma3(f32x4 acc, const Split8& a, const Split8& b) {
  acc = mfma_bf16(a.lo, b.hi, acc);
  acc = mfma_bf16(a.hi, b.lo, acc);
  return mfma_bf16(a.hi, b.hi, acc);
}

// k (inside a 32-wide block) of slot e of lane group g
__device__ __forceinline__ int slot_k(int g, int e) { return 4 * g + (e & 3) + 16 * (e >> 2); }

typedef unsigned u32x4w __attribute__((ext_vector_type(4)));

// Record stores are nontemporal: the records (about 1 GiB at 32 K tokens and
// d = 256) stream through, and the q and k rows that the preparation reads
// again keep their place in L2.
__device__ __forceinline__ void store_frag(unsigned char* dst, const bf16x8& f, int lane) {
  __builtin_nontemporal_store(f, reinterpret_cast<bf16x8*>(dst + 16 * lane));
}
__device__ __forceinline__ bf16x8 load_frag(const unsigned char* src, int lane) {
  return *reinterpret_cast<const bf16x8*>(src + 16 * lane);
}

__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
// slots 0-3 from p[0..3], slots 4-7 from p[16..19]
__device__ __forceinline__ void load8_perm(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 16);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// ---------------------------------------------------------------- pass 1
struct WidePrepLds {
  static constexpr int kAf = 0;                          // A      [C][SF] f32
  static constexpr int kTf = kAf + kC * kSF * 4;         // T      [C][SF] f32
  static constexpr int kMf = kTf + kC * kSF * 4;         // M      [C][SF] f32
  static constexpr int kTb = kMf + kC * kSF * 4;         // T diag(beta)      [hi, lo][C][SH] bf16
  static constexpr int kXs = kTb + 2 * kC * kSH * 2;     // solve scratch [4][16][20] f32
  static constexpr int kGd = kXs + 4 * 16 * 20 * 4;      // G   [C] f64 (log2 units)
  static constexpr int kGam = kGd + kC * 8;              // gam [C] f32
  static constexpr int kEps = kGam + kC * 4;             // exp(G_last - G) [C] f32
  static constexpr int kBet = kEps + kC * 4;             // beta [C] f32
  static constexpr int kBytes = kBet + kC * 4;
  static_assert(2 * kBytes <= 160 * 1024, "two workgroups per gfx950 compute unit");
};

template <int DK, bool RAW>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void wide_prep_kernel(ScanParams p, unsigned char* ws, size_t rec_bytes,
                                                             const int32_t* cs, const int2* __restrict__ info) {
  using L_ = WidePrepLds;
  extern __shared__ __align__(16) unsigned char smem[];
  float* Af = reinterpret_cast<float*>(smem + L_::kAf);
  float* Tf = reinterpret_cast<float*>(smem + L_::kTf);
  float* Mf = reinterpret_cast<float*>(smem + L_::kMf);
  __bf16* Tb = reinterpret_cast<__bf16*>(smem + L_::kTb);
  float* Xs = reinterpret_cast<float*>(smem + L_::kXs);
  double* Gd = reinterpret_cast<double*>(smem + L_::kGd);
  float* Gam = reinterpret_cast<float*>(smem + L_::kGam);
  float* Eps = reinterpret_cast<float*>(smem + L_::kEps);
  float* Bet = reinterpret_cast<float*>(smem + L_::kBet);

  const int items = cs[p.num_seqs] * p.h_v;
  const int item = static_cast<int>(blockIdx.x);
  if (item >= items) return;
  const int c = item / p.h_v, h = item % p.h_v;
  const int2 ci = info[c];
  const int t0 = ci.x, Lc = ci.y;
  const int hq = h / p.ratio;
  const int d_v = p.d_v;
  const int tid = static_cast<int>(threadIdx.x);
  const int w = tid >> 6, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const float* kg = static_cast<const float*>(p.k);
  const float* qg = static_cast<const float*>(p.q);
  const float* vg = static_cast<const float*>(p.v);
  const size_t qk_stride = static_cast<size_t>(p.h_qk) * DK;
  const size_t v_stride = static_cast<size_t>(p.h_v) * d_v;
  const WideRec rec(DK, d_v);
  unsigned char* base = ws + static_cast<size_t>(item) * rec_bytes;
  // row of token t of this chunk (clamped into the chunk: rows past its end
  // are finite and meet zero factors, beta = 0 for them)
  auto krow = [&](int t) __attribute__((always_inline)) {
    return kg + static_cast<size_t>(t0 + min(t, Lc - 1)) * qk_stride + static_cast<size_t>(hq) * DK;
  };
  auto qrow = [&](int t) __attribute__((always_inline)) {
    return qg + static_cast<size_t>(t0 + min(t, Lc - 1)) * qk_stride + static_cast<size_t>(hq) * DK;
  };

  // Rules without the delta correction (gated, linear) write v as it is: A = 0,
  // so T = I, with weight 1 in U = T diag(beta) V and 0 in W, and D = V.
  const bool delta_rule = p.gates.deltas != 0;
  // ================= 1. gates, the prefix sum of the log-decay, decay factors
  if (w == 0) {
    float gv = 0.0f, b = 0.0f;
    if (lane < Lc) {
      const size_t gi = static_cast<size_t>(t0 + lane) * p.h_v + h;
      const size_t bi = p.gates.beta_shared ? static_cast<size_t>(t0 + lane) : gi;
      if constexpr (RAW) {
        gv = p.gates.decays ? gate_log_decay(static_cast<const float*>(p.gates.a)[gi], p.gates.A_log[h], p.gates.dt_bias[h]) : 0.0f;
        b = delta_rule ? gate_sigmoid(static_cast<const float*>(p.gates.b)[bi]) : 1.0f;
      } else {
        gv = p.gates.decays ? static_cast<const float*>(p.gates.g)[gi] : 0.0f;
        b = delta_rule ? static_cast<const float*>(p.gates.beta)[bi] : 1.0f;
      }
      gv = fmaxf(gv, kMinLogDecay);
    }
    const double G = wave_prefix_sum(static_cast<double>(gv) * kLog2e, lane);
    const double Glast = readlane(G, 63);
    Gd[lane] = G;
    const float gam = fast_exp2(static_cast<float>(G));
    Gam[lane] = gam;
    Eps[lane] = fast_exp2(static_cast<float>(Glast - G));
    Bet[lane] = b;
    if (lane == 63) *reinterpret_cast<float*>(base + rec.gam) = gam;
  }
  __syncthreads();

  // ================= 2. P = K K^T, R = Q K^T (row tile w, lower tiles) -> A, M
  {
    const int tt = w;
    f32x4 pacc[4], racc[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      pacc[st] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      racc[st] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    const float* ka_row = krow(16 * tt + r16) + 8 * g;
    const float* qa_row = qrow(16 * tt + r16) + 8 * g;
    // the rows of key block kb + 1 are loaded while block kb is multiplied
    float xa[2][8], xq[2][8], xb[2][4][8];
    auto fetch = [&](int kb, int buf) __attribute__((always_inline)) {
      load8(ka_row + 32 * kb, xa[buf]);
      load8(qa_row + 32 * kb, xq[buf]);
#pragma unroll
      for (int st = 0; st < 4; ++st)
        if (st <= tt) load8(krow(16 * st + r16) + 8 * g + 32 * kb, xb[buf][st]);
    };
    fetch(0, 0);
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) {
      const int buf = kb & 1;
      if (kb + 1 < DK / 32) fetch(kb + 1, buf ^ 1);
      const Split8 KA = split8(xa[buf]);
      const Split8 QA = split8(xq[buf]);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        if (st <= tt) {
          const Split8 KB = split8(xb[buf][st]);
          pacc[st] = mma3(pacc[st], KA, KB);
          racc[st] = mma3(racc[st], QA, KB);
        }
      }
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int s = 16 * st + acc_col(lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * tt + acc_row(lane, i);
        float a = 0.0f, m = 0.0f;
        if (st <= tt && s <= t) {
          const float dec = fast_exp2(static_cast<float>(Gd[t] - Gd[s]));
          m = p.scale * dec * racc[st][i];
          if (s < t && delta_rule) a = Bet[t] * dec * pacc[st][i];
        }
        Af[t * kSF + s] = a;
        Mf[t * kSF + s] = m;
      }
    }
  }
  __syncthreads();

  // ================= 3. M fragments; T = (I + A)^-1 (diagonal blocks by
  // substitution, the rest by block substitution on the f32 MFMA)
  {
    const int g4 = 4 * g;
    for (int blk = w; blk < 6; blk += 4) {
      const int tt = blk < 2 ? blk : 2 + (blk - 2) / 2;
      const int kb = blk < 2 ? 0 : (blk - 2) % 2;
      float x[8];
      load8_perm(Mf + (16 * tt + r16) * kSF + 32 * kb + g4, x);
      const Split8 s = split8(x);
      store_frag(base + rec.ms + (2 * blk) * 1024, s.hi, lane);
      store_frag(base + rec.ms + (2 * blk + 1) * 1024, s.lo, lane);
    }
  }
  {
    const int cc = lane & 15;
    const float* Ab = Af + (16 * w) * kSF + 16 * w;
    float d[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x0 = (r == cc) ? 1.0f : 0.0f, x1 = 0.0f;
#pragma unroll
      for (int s2 = 0; s2 < r; s2 += 2) {
        x0 = fmaf(-Ab[r * kSF + s2], d[s2], x0);
        if (s2 + 1 < r) x1 = fmaf(-Ab[r * kSF + s2 + 1], d[s2 + 1], x1);
      }
      d[r] = x0 + x1;
    }
    if (lane < 16) {
#pragma unroll
      for (int r = 0; r < 16; ++r) Tf[(16 * w + r) * kSF + 16 * w + cc] = d[r];
    }
  }
  __syncthreads();
  for (int dist = 1; dist < 4; ++dist) {
    const int i = w + dist, j = w;
    if (i < 4) {
      f32x4 x = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int k = j; k < i; ++k)
        x = mma_f32(x, Af + (16 * i) * kSF + 16 * k, kSF, Tf + (16 * k) * kSF + 16 * j, kSF, lane);
      float* xs = Xs + w * 16 * 20;
#pragma unroll
      for (int e = 0; e < 4; ++e) xs[acc_row(lane, e) * 20 + acc_col(lane)] = x[e];
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
      f32x4 y = {0.0f, 0.0f, 0.0f, 0.0f};
      y = mma_f32(y, Tf + (16 * i) * kSF + 16 * i, kSF, xs, 20, lane);
#pragma unroll
      for (int e = 0; e < 4; ++e) Tf[(16 * i + acc_row(lane, e)) * kSF + 16 * j + acc_col(lane)] = -y[e];
    }
    __syncthreads();
  }
  // T diag(beta), split
  for (int e = tid; e < kC * kC; e += kThreads) {
    const int t = e >> 6, s = e & 63;
    const float tv = (s <= t) ? Tf[t * kSF + s] : 0.0f;
    const float xb = tv * Bet[s];
    const __bf16 hb = static_cast<__bf16>(xb);
    Tb[t * kSH + s] = hb;
    Tb[kC * kSH + t * kSH + s] = static_cast<__bf16>(xb - static_cast<float>(hb));
  }
  __syncthreads();

  // ================= 4. Kt^T, W and scale diag(gam) Q fragments.  W^T =
  // (diag(gam) K)^T (T diag(beta))^T is formed in accumulator tiles, which are
  // W's operand fragments in the permuted key order.
  {
    // B operand: lane supplies Tb[token 16 tt + r16][token' 32 kb + slot_k(g, e)], token' <= token
    Split8 TB[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        if (kb == 1 && tt < 2) continue;
        const int off = (16 * tt + r16) * kSH + 32 * kb + 4 * g;
#pragma unroll
        for (int hl = 0; hl < 2; ++hl) {
          const __bf16* src = Tb + hl * kC * kSH + off;
          const uint2 lo4 = *reinterpret_cast<const uint2*>(src);
          const uint2 hi4 = *reinterpret_cast<const uint2*>(src + 16);
          const u32x4w v = {lo4.x, lo4.y, hi4.x, hi4.y};
          (hl == 0 ? TB[kb][tt].hi : TB[kb][tt].lo) = __builtin_bit_cast(bf16x8, v);
        }
      }
    constexpr int PAIRS = DK / 128;  // key blocks of 32 (two key tiles each) per wave
    float gq[4];                     // scale gam of this lane's Q rows
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) gq[tt] = p.scale * Gam[16 * tt + r16];
    const float wgt = delta_rule ? 1.0f : 0.0f;  // W = 0 without the delta correction
    // every load of the wave's key blocks first: K^T slots (two key tiles x
    // two token blocks each), Q rows (four token tiles each)
    float xk[PAIRS][2][2][8], xqv[PAIRS][4][8];
#pragma unroll
    for (int pr = 0; pr < PAIRS; ++pr) {
      const int kbk = w * PAIRS + pr;
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 8; ++e) xk[pr][half][kb][e] = krow(32 * kb + slot_k(g, e))[32 * kbk + 16 * half + r16];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) load8_perm(qrow(16 * tt + r16) + 32 * kbk + 4 * g, xqv[pr][tt]);
    }
#pragma unroll
    for (int pr = 0; pr < PAIRS; ++pr) {
      const int kbk = w * PAIRS + pr;  // key block of 32
      auto& x = xk[pr];
      auto& qv = xqv[pr];

#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[tt][e] *= gq[tt];
        const Split8 qs = split8(qv[tt]);
        store_frag(base + rec.qf + ((kbk * 4 + tt) * 2) * 1024, qs.hi, lane);
        store_frag(base + rec.qf + ((kbk * 4 + tt) * 2 + 1) * 1024, qs.lo, lane);
      }
      f32x4 acc[2][4];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int r = 2 * kbk + half;  // key tile
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[half][tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          float xe[8], xg[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int tok = 32 * kb + slot_k(g, e);
            xe[e] = x[half][kb][e] * Eps[tok];
            xg[e] = x[half][kb][e] * Gam[tok] * wgt;
          }
          const Split8 KE = split8(xe);
          store_frag(base + rec.kt + ((r * 2 + kb) * 2) * 1024, KE.hi, lane);
          store_frag(base + rec.kt + ((r * 2 + kb) * 2 + 1) * 1024, KE.lo, lane);
          const Split8 KW = split8(xg);
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            if (kb == 1 && tt < 2) continue;
            acc[half][tt] = mma3(acc[half][tt], KW, TB[kb][tt]);
          }
        }
      }
      // acc[half][tt] element i of lane l: W[token 16 tt + r16][key 16 (2 kbk + half) + 4 g + i]
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        float xw[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xw[i] = acc[0][tt][i];
          xw[4 + i] = acc[1][tt][i];
        }
        const Split8 sw = split8(xw);
        store_frag(base + rec.w + ((kbk * 4 + tt) * 2) * 1024, sw.hi, lane);
        store_frag(base + rec.w + ((kbk * 4 + tt) * 2 + 1) * 1024, sw.lo, lane);
      }
    }
  }

  // ================= 5. U = T diag(beta) V, in accumulator order
  {
    Split8 TA[4][2];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb == 1 && tt < 2) continue;
        const int off = (16 * tt + r16) * kSH + 32 * kb + 8 * g;
        TA[tt][kb].hi = *reinterpret_cast<const bf16x8*>(Tb + off);
        TA[tt][kb].lo = *reinterpret_cast<const bf16x8*>(Tb + kC * kSH + off);
      }
    // the V columns of all this wave's column tiles are loaded first
    // (d_v <= 256: at most four tiles per wave; past d_v the loads are clamped
    // and unused)
    const int nct = d_v / 16;
    float xv[4][2][8];
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const int col = min(16 * (w + 4 * c4) + r16, d_v - 1);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int tok = min(32 * kb + 8 * g + e, Lc - 1);
          xv[c4][kb][e] = vg[static_cast<size_t>(t0 + tok) * v_stride + static_cast<size_t>(h) * d_v + col];
        }
    }
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const int ct = w + 4 * c4;
      if (ct >= nct) break;
      Split8 VB[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) VB[kb] = split8(xv[c4][kb]);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        acc = mma3(acc, TA[tt][0], VB[0]);
        if (tt >= 2) acc = mma3(acc, TA[tt][1], VB[1]);
        __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(base + rec.u + ((static_cast<size_t>(ct) * 4 + tt) * 64 + lane) * 16));
      }
    }
  }
}

// ---------------------------------------------------------------- pass 2
// One workgroup per (sequence, value head, 16-column tile) with one wave per
// 32 state rows (d_k / 32 waves: two per SIMD at d_k = 256, so that each
// compute unit keeps twice the fragment loads of four waves in flight).  Wave
// w holds rows [32 w, 32 w + 32) of the tile as two accumulator tiles.  Per
// chunk, with two barriers:
//  1. every wave forms its partial W S over its rows -> LDS; after the first
//     barrier, its partial Q S -> LDS (both double-buffered by chunk parity);
//  2. waves 0-3 sum the partials of token tile w: D = U - W S -> LDS;
//  3. after the second barrier every wave reads D and updates its rows,
//     S <- gam_C S + Kt^T D, and waves 0-3 write the output of token tile w,
//     O = (sum of the Q S partials) + M D.
template <int DK>
struct WideStateLds {
  static constexpr int NW = DK / 32;
  static constexpr int kX = 0;                              // X partials [2][NW][4 tt][64] f32x4
  static constexpr int kY = kX + 2 * NW * 4 * 64 * 16;      // Y partials [2][NW][4 tt][64] f32x4
  static constexpr int kD = kY + 2 * NW * 4 * 64 * 16;      // D          [4 tt][64] f32x4
  static constexpr int kBytes = kD + 4 * 64 * 16;
  static_assert(kBytes <= 160 * 1024, "LDS budget of one gfx950 workgroup");
};

template <int DK>
__global__ __launch_bounds__(64 * (DK / 32)) void wide_state_kernel(ScanParams p, const unsigned char* ws,
                                                                    size_t rec_bytes, const int32_t* cs, int units8) {
  using L_ = WideStateLds<DK>;
  constexpr int NW = L_::NW;
  constexpr int kThr = 64 * NW;
  extern __shared__ __align__(16) unsigned char smem[];
  f32x4* Xp = reinterpret_cast<f32x4*>(smem + L_::kX);
  f32x4* Yp = reinterpret_cast<f32x4*>(smem + L_::kY);
  f32x4* Dt = reinterpret_cast<f32x4*>(smem + L_::kD);

  const int unit = static_cast<int>(blockIdx.x) % units8;
  const int ct = static_cast<int>(blockIdx.x) / units8;
  const int units = p.num_seqs * p.h_v;
  if (unit >= units) return;
  const int n = unit / p.h_v, h = unit % p.h_v;
  const int d_v = p.d_v;
  const int T = p.total_tokens;
  const int tid = static_cast<int>(threadIdx.x);
  // w is wave-uniform, and the compiler is told so: a branch on it must skip
  // its MFMAs, which run whatever the execution mask
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, r16 = lane & 15;
  const int wt = w & 3;  // token tile of the second phase (waves 0-3)
  const int col = 16 * ct + r16;
  const int key0 = 32 * w;
  const WideRec rec(DK, d_v);
  float* og = static_cast<float*>(p.out);
  const size_t v_stride = static_cast<size_t>(p.h_v) * d_v;

  bool has_state = true;
  const int sidx = state_slot(p.slots, p.num_slots, n, &has_state);
  const size_t sbase = (static_cast<size_t>(sidx) * p.h_v + h) * DK * d_v;

  f32x4 S[2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      S[r][i] = (p.s0 != nullptr && has_state)
                    ? p.s0[sbase + static_cast<size_t>(key0 + 16 * r + acc_row(lane, i)) * d_v + col]
                    : 0.0f;

  const int lo = wseq_lo(p.cu, n, T), hi = wseq_hi(p.cu, n, T);
  const int nchunks = (hi - lo + kC - 1) / kC;
  const int c0 = cs[n];
  struct SetA {
    Split8 W[4];
    Split8 Q[4];
  };
  auto rec_of = [&](int j) __attribute__((always_inline)) {
    return ws + (static_cast<size_t>(c0 + min(j, nchunks - 1)) * p.h_v + h) * rec_bytes;
  };
  // The W fragments of the next chunk are loaded as soon as this chunk's W S
  // products have read theirs, the Q fragments after the Q S products: one
  // register set, refilled in two halves.  The operands used after the second
  // barrier (set B: Kt^T, M, U, the decay factor) are issued at the top of
  // their own chunk.  Loads of a chunk past the last are clamped to the last.
  auto load_w = [&](int j, SetA& a) __attribute__((always_inline)) {
    const unsigned char* rb = rec_of(j);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const size_t f = ((w * 4 + tt) * 2) * 1024;  // key block w of 32, token tile tt
      a.W[tt].hi = load_frag(rb + rec.w + f, lane);
      a.W[tt].lo = load_frag(rb + rec.w + f + 1024, lane);
    }
  };
  auto load_q = [&](int j, SetA& a) __attribute__((always_inline)) {
    const unsigned char* rb = rec_of(j);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const size_t f = ((w * 4 + tt) * 2) * 1024;
      a.Q[tt].hi = load_frag(rb + rec.qf + f, lane);
      a.Q[tt].lo = load_frag(rb + rec.qf + f + 1024, lane);
    }
  };
  // The column tiles of a unit share each chunk's record through one L2.
  // Each tile touches its share of the record kTouchAhead chunks ahead (one
  // 4-byte load per 128-byte line), so the record comes in from HBM while earlier
  // chunks compute and the fragment loads meet L2 hits.  The touch is issued
  // after the chunk's other loads and its value is consumed a chunk later,
  // so no wait ever falls on it early (loads complete in issue order).
  // Only when a tile's share fits one load per thread.
  const int nct = d_v / 16;
  const int lines = static_cast<int>(rec_bytes / 128);
  const int per_tile = (lines + nct - 1) / nct;
  const bool touching = per_tile <= kThr;
  int touched = 0, tv = 0;
  auto touch = [&](int j) __attribute__((always_inline)) {
    touched += tv;
    const int line = min(ct * per_tile + tid, lines - 1);
    tv = *reinterpret_cast<const int*>(ws + (static_cast<size_t>(c0 + min(j, nchunks - 1)) * p.h_v + h) * rec_bytes +
                                       static_cast<size_t>(line) * 128);
  };

  SetA a;
  auto chunk = [&](int j) __attribute__((always_inline)) {
    const int t0 = lo + kC * j;
    const int Lc = min(kC, hi - t0);
    const unsigned char* rb = rec_of(j);
    const int buf = j & 1;
    f32x4* Xb = Xp + buf * NW * 4 * 64;
    f32x4* Yb = Yp + buf * NW * 4 * 64;

    // ---- set B of this chunk: Kt^T over this wave's 32 rows; M blocks and
    //      the U tile of token tile wt (used by waves 0-3)
    Split8 KtA[2][2];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const unsigned char* f = rb + rec.kt + (((w * 2 + r) * 2 + kb) * 2) * 1024;
        KtA[r][kb].hi = load_frag(f, lane);
        KtA[r][kb].lo = load_frag(f + 1024, lane);
      }
    Split8 MA[2];
    f32x4 Uw = {0.0f, 0.0f, 0.0f, 0.0f};
    if (w < 4) {
      const unsigned char* f = rb + rec.ms + (2 * m_block(wt, 0)) * 1024;
      MA[0].hi = load_frag(f, lane);
      MA[0].lo = load_frag(f + 1024, lane);
      if (wt >= 2) {
        f = rb + rec.ms + (2 * m_block(wt, 1)) * 1024;
        MA[1].hi = load_frag(f, lane);
        MA[1].lo = load_frag(f + 1024, lane);
      } else {
        MA[1] = MA[0];
      }
      Uw = *reinterpret_cast<const f32x4*>(rb + rec.u + ((static_cast<size_t>(ct) * 4 + wt) * 64 + lane) * 16);
    }
    const float gam_last = *reinterpret_cast<const float*>(rb + rec.gam);

    // ---- 1. partial W S and Q S over this wave's rows (U of token tile w
    //      folded into wave w's W S partial of that tile: the partials sum to -D)
    Split8 SB;
    {
      float x[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = S[0][i];
        x[4 + i] = S[1][i];
      }
      SB = split8(x);
    }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      f32x4 xa = {0.0f, 0.0f, 0.0f, 0.0f};
      xa = mma3(xa, a.W[tt], SB);
      Xb[(w * 4 + tt) * 64 + lane] = tt == w ? xa - Uw : xa;
    }
    load_w(j + 1, a);
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      f32x4 ya = {0.0f, 0.0f, 0.0f, 0.0f};
      ya = mma3(ya, a.Q[tt], SB);
      Yb[(w * 4 + tt) * 64 + lane] = ya;
    }
    load_q(j + 1, a);
    if (touching) touch(j + kTouchAhead);

    // ---- 2. waves 0-3: D of token tile w
    if (w < 4) {
      f32x4 x = Xb[w * 64 + lane];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) x += Xb[(ww * 4 + w) * 64 + lane];
      Dt[w * 64 + lane] = -x;
    }
    __syncthreads();

    // ---- 3. D fragments; the output of tile w (waves 0-3); the state update
    Split8 DB[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const f32x4 d0 = Dt[(2 * kb) * 64 + lane], d1 = Dt[(2 * kb + 1) * 64 + lane];
      float x[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = d0[i];
        x[4 + i] = d1[i];
      }
      DB[kb] = split8(x);
    }
    if (w < 4 && og != nullptr) {
      f32x4 y = Yb[w * 64 + lane];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) y += Yb[(ww * 4 + w) * 64 + lane];
      f32x4 o = mma3(y, MA[0], DB[0]);
      if (w >= 2) o = mma3(o, MA[1], DB[1]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * w + acc_row(lane, i);
        if (t < Lc) og[static_cast<size_t>(t0 + t) * v_stride + static_cast<size_t>(h) * d_v + col] = o[i];
      }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      f32x4 sacc = S[r] * gam_last;
      sacc = mma3(sacc, KtA[r][0], DB[0]);
      sacc = mma3(sacc, KtA[r][1], DB[1]);
      S[r] = sacc;
    }
  };

  if (nchunks > 0) {
    load_w(0, a);
    load_q(0, a);
    for (int j = 0; j < nchunks; ++j) chunk(j);
  }

  // keeps the touches alive (never true: the host rejects negative token counts)
  if (p.total_tokens < 0 && touched + tv == 1) og[0] = 0.0f;
  if (p.sN != nullptr && has_state) {
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        p.sN[sbase + static_cast<size_t>(key0 + 16 * r + acc_row(lane, i)) * d_v + col] = S[r][i];
  }
}

template <typename K>
hipError_t set_lds_once(K kern, int bytes) {
  return ensure_dynamic_lds(reinterpret_cast<const void*>(kern), bytes);
}

template <int DK>
hipError_t launch_dk(const ScanParams& p, unsigned char* recs, size_t rec_bytes, const int32_t* cs, const int2* info,
                     int bound, hipStream_t stream) {
  if (bound > 0 && p.h_v > 0) {
    constexpr int bytes = WidePrepLds::kBytes;
    const unsigned grid = static_cast<unsigned>(bound) * static_cast<unsigned>(p.h_v);
    if (p.gates.raw) {
      auto kern = wide_prep_kernel<DK, true>;
      hipError_t e = set_lds_once(kern, bytes);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), bytes, stream, p, recs, rec_bytes, cs, info);
    } else {
      auto kern = wide_prep_kernel<DK, false>;
      hipError_t e = set_lds_once(kern, bytes);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), bytes, stream, p, recs, rec_bytes, cs, info);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int units = p.num_seqs * p.h_v;
  if (units == 0) return hipSuccess;
  // the column tiles of a unit sit units8 blocks apart: on one XCD (blocks
  // are dealt to the eight XCDs in turn), sharing its L2
  const int units8 = (units + 7) / 8 * 8;
  const unsigned blocks = static_cast<unsigned>(units8) * static_cast<unsigned>(p.d_v / 16);
  {
    constexpr int bytes = WideStateLds<DK>::kBytes;
    auto kern = wide_state_kernel<DK>;
    const hipError_t e = set_lds_once(kern, bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * (DK / 32)), bytes, stream, p, recs, rec_bytes, cs, units8);
  }
  return hipGetLastError();
}

}  // namespace

bool wide_supported(int io_dtype, int d_k, int d_v, const GateArgs& gates, int window) {
  return io_dtype == 0 && (d_k == 128 || d_k == 256) && d_v >= 16 && d_v <= 256 && d_v % 16 == 0 &&
         !gates.per_key && window == 0;
}

// Measured against the serial scan (8 or 32 heads, 1 or 8 sequences of 128 to
// 4096 tokens), the float32 chunked form is as fast at 128 tokens and faster
// from 256 on, at d_k 128 and 256 alike.
bool wide_auto(int d_k) { return d_k == 128 || d_k == 256; }

size_t wide_workspace_bytes(int num_seqs, int total_tokens, int h_v, int d_k, int d_v) {
  if (num_seqs <= 0) return 0;
  const WideRec rec(d_k, d_v);
  return chunk_table_bytes(num_seqs, total_tokens) +
         static_cast<size_t>(chunk_table_bound(num_seqs, total_tokens)) * h_v * rec.bytes;
}

hipError_t launch_prefill_wide(ScanParams p, void* workspace, hipStream_t stream) {
  if (p.num_seqs <= 0) return hipSuccess;
  if (!wide_supported(0, p.d_k, p.d_v, p.gates, p.window)) return hipErrorInvalidValue;
  const WideRec rec(p.d_k, p.d_v);
  const int T = p.total_tokens;
  hipError_t e = launch_chunk_table(p.cu, p.num_seqs, T, workspace, stream);
  if (e != hipSuccess) return e;
  const int32_t* cs = static_cast<const int32_t*>(workspace);
  const int2* info = reinterpret_cast<const int2*>(static_cast<unsigned char*>(workspace) +
                                                   align256w(static_cast<size_t>(p.num_seqs + 1) * 4));
  unsigned char* recs = static_cast<unsigned char*>(workspace) + chunk_table_bytes(p.num_seqs, T);
  const int bound = chunk_table_bound(p.num_seqs, T);
  return p.d_k == 256 ? launch_dk<256>(p, recs, rec.bytes, cs, info, bound, stream)
                      : launch_dk<128>(p, recs, rec.bytes, cs, info, bound, stream);
}

}  // namespace gdn
