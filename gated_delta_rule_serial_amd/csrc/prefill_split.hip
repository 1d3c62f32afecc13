// prefill_split.hip -- the chunked prefill in two passes (gfx950 MFMA, bf16
// operands, f32 accumulation): a chunk-parallel pass that prepares every
// chunk's factors, and a sequential pass that only carries the state.
//
// The chunked form is the one derived in prefill_chunked.hip from [P4]
// onnx-runtime-ep-cuda, src/kernels/linear_attention.rs, `linear_attention_core`
// steps 1-4.  Per chunk of C = 64 tokens (G_t the in-chunk prefix of the
// log-decay, gam_t = exp(G_t), T = (I + A)^-1 with the strictly lower
// A_ts = beta_t exp(G_t - G_s) k_t.k_s):
//     W  = T diag(beta gam) K          U = T diag(beta) V
//     M_ts = exp(G_t - G_s) q_t.k_s (s <= t)
//     Kt = diag(exp(G_last - G)) K     (the state-update factor)
// depend on the chunk alone, while
//     D   = U - W S
//     O   = scale (diag(gam) Q S + M D)
//     S  <- gam_last S + Kt^T D
// carry the state S from chunk to chunk.
//
// Pass 1 (chunk_prep_kernel): one workgroup per (chunk, value head) computes
// W, Kt^T, M, U and gam into a caller-provided workspace; all chunks of all
// sequences run at once.  Pass 2 (chunk_state_kernel): one workgroup per
// (sequence, value head, column block) walks its sequence's chunks, doing only
// the four products above with the state in MFMA accumulators.  The serial
// chain per chunk shrinks from the whole chunked step to those four products,
// and pass 1 fills the whole chip however few sequences and heads there are.
// A chunk table (chunk_table_kernel) maps the packed sequences to chunks.
#include "chunk_mfma.hpp"
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

namespace {

constexpr int kC = 64;        // chunk length (tokens)
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kSC = kC + 8;   // bf16 row stride of C-long rows
constexpr int kSA = kC + 8;   // f32 row stride of A (its buffer later holds T' and T'' in bf16)
constexpr int kST = kC + 4;   // f32 row stride of T
constexpr float kMinLogDecay = -1.0e4f;
constexpr double kLog2e = 1.4426950408889634;

__host__ __device__ constexpr size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// One (chunk, value head) record of the workspace.
struct Rec {
  size_t w, kt, m, u, g, bytes;
  __host__ __device__ Rec(int dk, int dvp) {
    w = 0;                                                  // W      [C][dk] bf16
    kt = w + static_cast<size_t>(kC) * dk * 2;              // Kt^T   [dk][C] bf16
    m = kt + static_cast<size_t>(dk) * kC * 2;              // M      [C][C] bf16
    u = m + static_cast<size_t>(kC) * kC * 2;               // U      [4][dvp / 16][64 lanes][4] f32
    g = u + static_cast<size_t>(kC) * dvp * 4;              // gam    [C] f32, then gam_last
    bytes = align256(g + (kC + 4) * 4);
  }
};

__host__ __device__ inline int pad16(int x) { return (x + 15) & ~15; }

__device__ __forceinline__ int seq_lo(const int32_t* cu, int n, int T) { return min(max(cu[n], 0), T); }
__device__ __forceinline__ int seq_hi(const int32_t* cu, int n, int T) {
  return min(max(cu[n + 1], seq_lo(cu, n, T)), T);
}

// cs[n] = chunks of the sequences before n; cs[N] = all chunks; info[c] =
// (first token, tokens) of chunk c.
__global__ __launch_bounds__(1024) void chunk_table_kernel(const int32_t* cu, int num_seqs, int T, int32_t* cs,
                                                           int2* info) {
  __shared__ int part[1024];
  const int tid = static_cast<int>(threadIdx.x);
  const int per = (num_seqs + 1023) / 1024;
  const int a = min(tid * per, num_seqs), b = min(a + per, num_seqs);
  auto chunks = [&](int n) { return (seq_hi(cu, n, T) - seq_lo(cu, n, T) + kC - 1) / kC; };
  int sum = 0;
  for (int n = a; n < b; ++n) sum += chunks(n);
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - sum;
  for (int n = a; n < b; ++n) {
    cs[n] = run;
    const int lo = seq_lo(cu, n, T), hi = seq_hi(cu, n, T);
    for (int t = lo; t < hi; t += kC) info[run++] = make_int2(t, min(kC, hi - t));
  }
  if (tid == 1023) cs[num_seqs] = part[1023];
}

// ---------------------------------------------------------------- pass 1
template <int DK, int DVT>
struct PrepLds {
  static constexpr int SK = DK + 8;
  static constexpr int DVP = 16 * DVT;
  static constexpr int kKs = 0;                          // K rows  [C][SK] bf16 (later W)
  static constexpr int kQs = kKs + kC * SK * 2;          // Q rows  [C][SK] bf16
  static constexpr int kKT = kQs + kC * SK * 2;          // K^T     [DK][SC] bf16
  static constexpr int kVt = kKT + DK * kSC * 2;         // V^T     [DVP][SC] bf16
  static constexpr int kAf = kVt + DVP * kSC * 2;        // A       [C][SA] f32 (later T', T'')
  static constexpr int kTf = kAf + kC * kSA * 4;         // T       [C][ST] f32
  static constexpr int kMs = kTf + kC * kST * 4;         // M       [C][SC] bf16
  static constexpr int kXs = kMs + kC * kSC * 2;         // solve scratch [4][16][20] f32
  static constexpr int kGd = kXs + 4 * 16 * 20 * 4;      // G       [C] f64
  static constexpr int kGam = kGd + kC * 8;              // gam     [C] f32
  static constexpr int kBet = kGam + kC * 4;             // beta    [C] f32
  static constexpr int kBytes = kBet + kC * 4;
  static_assert(2 * kC * kSC * 2 <= kC * kSA * 4, "T' and T'' must fit in the A buffer");
  static_assert(kBytes <= 160 * 1024, "LDS budget of one gfx950 workgroup");
};

// Persistent: one workgroup per CU (the LDS holds one) walks the (chunk,
// value head) items blockIdx.x, + gridDim.x, ...; the next item's K, Q, V rows
// and gates are loaded into registers while the current one computes.
template <typename IO, int DK, int DVT, bool RAW>
__global__ __launch_bounds__(kThreads) void chunk_prep_kernel(ScanParams p, unsigned char* ws, size_t rec_bytes,
                                                              const int32_t* cs, const int2* info, int items) {
  using L_ = PrepLds<DK, DVT>;
  constexpr int SK = L_::SK;
  constexpr int DVP = L_::DVP;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16_t* Ks = reinterpret_cast<bf16_t*>(smem + L_::kKs);
  bf16_t* Ws = Ks;
  bf16_t* Qs = reinterpret_cast<bf16_t*>(smem + L_::kQs);
  bf16_t* KT = reinterpret_cast<bf16_t*>(smem + L_::kKT);
  bf16_t* Vt = reinterpret_cast<bf16_t*>(smem + L_::kVt);
  float* Af = reinterpret_cast<float*>(smem + L_::kAf);
  bf16_t* Tp = reinterpret_cast<bf16_t*>(smem + L_::kAf);
  bf16_t* Tpp = reinterpret_cast<bf16_t*>(smem + L_::kAf + kC * kSC * 2);
  float* Tf = reinterpret_cast<float*>(smem + L_::kTf);
  bf16_t* Ms = reinterpret_cast<bf16_t*>(smem + L_::kMs);
  float* Xs = reinterpret_cast<float*>(smem + L_::kXs);
  double* Gd = reinterpret_cast<double*>(smem + L_::kGd);
  float* Gam = reinterpret_cast<float*>(smem + L_::kGam);
  float* Bet = reinterpret_cast<float*>(smem + L_::kBet);

  const int T = p.total_tokens;
  const int total = cs[p.num_seqs] * p.h_v;  // live items; the grid covers a bound
  const int n_items = items < total ? items : total;
  const int d_v = p.d_v;
  const int tid = static_cast<int>(threadIdx.x);
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int rb = w & 3;
  const int chalf = w >> 2;
  const Rec rec(DK, DVP);
  const IO* qg = static_cast<const IO*>(p.q);
  const IO* kg = static_cast<const IO*>(p.k);
  const IO* vg = static_cast<const IO*>(p.v);
  const size_t qk_stride = static_cast<size_t>(p.h_qk) * DK;
  const size_t v_stride = static_cast<size_t>(p.h_v) * d_v;

  // item i is chunk c = i / h_v (first token, tokens from the chunk table), head h = i % h_v
  struct Where {
    int c, h, t0, Lc;
  };
  auto locate = [&](int item, int2 ci) __attribute__((always_inline)) {
    Where at;
    at.c = item / p.h_v;
    at.h = item % p.h_v;
    at.t0 = ci.x;
    at.Lc = ci.y;
    return at;
  };
  auto info_of = [&](int item) __attribute__((always_inline)) {
    return item < n_items ? info[item / p.h_v] : make_int2(0, 0);
  };

  // ---- register staging of one item (vector-typed, so that it stays in registers)
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  constexpr int VPR = DK / 8;
  constexpr int KQ_IT = kC * VPR / kThreads;
  constexpr int VPV = DVP / 8;
  constexpr int V_IT = kC * VPV / kThreads;
  static_assert(KQ_IT >= 1 && V_IT >= 1, "block shape");
  u32x4 rk[KQ_IT], rq[KQ_IT], rv[V_IT];
  float rg = 0.0f, rbt = 0.0f;  // wave 0: gate inputs of token (chunk start + lane)
  auto fetch = [&](const Where& at) __attribute__((always_inline)) {
    const int hq = at.h / p.ratio;
#pragma unroll
    for (int it = 0; it < KQ_IT; ++it) {
      const int v = tid + it * kThreads;
      const int t = v / VPR, c8 = (v % VPR) * 8;
      rk[it] = u32x4{0u, 0u, 0u, 0u};
      rq[it] = u32x4{0u, 0u, 0u, 0u};
      if (t < at.Lc) {
        const size_t off = static_cast<size_t>(at.t0 + t) * qk_stride + static_cast<size_t>(hq) * DK + c8;
        rk[it] = *reinterpret_cast<const u32x4*>(kg + off);
        rq[it] = *reinterpret_cast<const u32x4*>(qg + off);
      }
    }
#pragma unroll
    for (int it = 0; it < V_IT; ++it) {
      const int v = tid + it * kThreads;
      const int t = v / VPV, c8 = (v % VPV) * 8;
      rv[it] = u32x4{0u, 0u, 0u, 0u};
      if (t < at.Lc && c8 < d_v)
        rv[it] = *reinterpret_cast<const u32x4*>(vg + static_cast<size_t>(at.t0 + t) * v_stride +
                                                 static_cast<size_t>(at.h) * d_v + c8);
    }
    if (w == 0) {
      rg = 0.0f;
      rbt = 0.0f;
      if (lane < at.Lc) {
        const size_t gi = static_cast<size_t>(at.t0 + lane) * p.h_v + at.h;
        const size_t bi = p.gates.beta_shared ? static_cast<size_t>(at.t0 + lane) : gi;
        if constexpr (RAW) {
          if (p.gates.decays) rg = widen(static_cast<const IO*>(p.gates.a)[gi]);
          rbt = widen(static_cast<const IO*>(p.gates.b)[bi]);
        } else {
          if (p.gates.decays) rg = widen(static_cast<const IO*>(p.gates.g)[gi]);
          rbt = widen(static_cast<const IO*>(p.gates.beta)[bi]);
        }
      }
    }
  };

  // the upper tiles of M stay zero for every item
  for (int e = tid; e < 6 * 256; e += kThreads) {
    const int tile = e >> 8;
    const int tb = tile < 3 ? 0 : (tile < 5 ? 1 : 2);
    const int cs_ = tile < 3 ? tile + 1 : (tile < 5 ? tile - 1 : 3);
    const int t = 16 * tb + ((e & 255) >> 4), s = 16 * cs_ + (e & 15);
    Ms[t * kSC + s] = 0;
  }

  int item = static_cast<int>(blockIdx.x);
  if (item >= n_items) return;
  Where at = locate(item, info[item / p.h_v]);
  fetch(at);
  int2 next_info = info_of(item + static_cast<int>(gridDim.x));  // one item ahead of the fetch
  for (; item < n_items; item += static_cast<int>(gridDim.x)) {
    const int h = at.h;
    const int Lc = at.Lc;
    unsigned char* base = ws + (static_cast<size_t>(at.c) * p.h_v + h) * rec_bytes;

    // ================= 1. stage K, Q rows and V^T; gates and the prefix sum of the log-decay
#pragma unroll
    for (int it = 0; it < KQ_IT; ++it) {
      const int v = tid + it * kThreads;
      const int t = v / VPR, c8 = (v % VPR) * 8;
      *reinterpret_cast<u32x4*>(Ks + t * SK + c8) = rk[it];
      *reinterpret_cast<u32x4*>(Qs + t * SK + c8) = rq[it];
    }
#pragma unroll
    for (int it = 0; it < V_IT; ++it) {
      const int v = tid + it * kThreads;
      const int t = v / VPV, c8 = (v % VPV) * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        Vt[(c8 + e) * kSC + t] =
            static_cast<bf16_t>((e & 1) ? (rv[it][e >> 1] >> 16) : (rv[it][e >> 1] & 0xffffu));
    }
    if (w == 0) {
      float g = 0.0f, b = 0.0f;
      if (lane < Lc) {
        if constexpr (RAW) {
          g = p.gates.decays ? gate_log_decay(rg, p.gates.A_log[h], p.gates.dt_bias[h]) : 0.0f;
          b = gate_sigmoid(rbt);
        } else {
          g = rg;
          b = rbt;
        }
        g = fmaxf(g, kMinLogDecay);
      }
      double G = static_cast<double>(g) * kLog2e;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const double y = __shfl_up(G, off, 64);
        if (lane >= off) G += y;
      }
      Gd[lane] = G;
      Gam[lane] = fast_exp2(static_cast<float>(G));
      Bet[lane] = b;
    }
    // the next item's inputs, in flight while this one computes
    const int next = item + static_cast<int>(gridDim.x);
    if (next < n_items) {
      at = locate(next, next_info);
      fetch(at);
      next_info = info_of(next + static_cast<int>(gridDim.x));
    }
    __syncthreads();

  // ================= 2. K^T; P = K K^T, R = Q K^T -> A (f32) and M (bf16)
  for (int ix = tid; ix < DK * (kC / 8); ix += kThreads) {
    const int i = ix % DK;
    const int t8 = (ix / DK) * 8;
    uint32_t wv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      wv[e] = static_cast<uint32_t>(Ks[(t8 + 2 * e) * SK + i]) | (static_cast<uint32_t>(Ks[(t8 + 2 * e + 1) * SK + i]) << 16);
    *reinterpret_cast<uint4*>(KT + i * kSC + t8) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  }
  for (int tj = w; tj < 10; tj += kWaves) {
    int tb = 0;
    while ((tb + 1) * (tb + 2) / 2 <= tj) ++tb;
    const int cs_ = tj - tb * (tb + 1) / 2;
    f32x4 pacc = {0.0f, 0.0f, 0.0f, 0.0f}, racc = {0.0f, 0.0f, 0.0f, 0.0f};
    pacc = mma<DK>(pacc, Ks + 16 * tb * SK, SK, Ks + 16 * cs_ * SK, SK, lane);
    racc = mma<DK>(racc, Qs + 16 * tb * SK, SK, Ks + 16 * cs_ * SK, SK, lane);
    const int s_ = 16 * cs_ + acc_col(lane);
    const double Gs = Gd[s_];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * tb + acc_row(lane, i);
      const float dec = (s_ <= t) ? fast_exp2(static_cast<float>(Gd[t] - Gs)) : 0.0f;
      Af[t * kSA + s_] = (s_ < t) ? Bet[t] * dec * pacc[i] : 0.0f;
      Ms[t * kSC + s_] = to_bf16(dec * racc[i]);
    }
  }
  __syncthreads();

  // ================= 3. T = (I + A)^-1 (diagonal blocks by substitution, the rest by block substitution)
  if (w < 4) {
    const int cc = lane & 15;
    const float* Ab = Af + (16 * w) * kSA + 16 * w;
    float d[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x0 = (r == cc) ? 1.0f : 0.0f, x1 = 0.0f;
#pragma unroll
      for (int s2 = 0; s2 < r; s2 += 2) {
        x0 = fmaf(-Ab[r * kSA + s2], d[s2], x0);
        if (s2 + 1 < r) x1 = fmaf(-Ab[r * kSA + s2 + 1], d[s2 + 1], x1);
      }
      d[r] = x0 + x1;
    }
    if (lane < 16) {
#pragma unroll
      for (int r = 0; r < 16; ++r) Tf[(16 * w + r) * kST + 16 * w + cc] = d[r];
    }
  }
  __syncthreads();
  for (int dist = 1; dist < 4; ++dist) {
    const int i = w + dist, j = w;
    if (i < 4) {
      f32x4 x = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int k = j; k < i; ++k)
        x = mma_f32(x, Af + (16 * i) * kSA + 16 * k, kSA, Tf + (16 * k) * kST + 16 * j, kST, lane);
      float* xs = Xs + w * 16 * 20;
#pragma unroll
      for (int e = 0; e < 4; ++e) xs[acc_row(lane, e) * 20 + acc_col(lane)] = x[e];
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
      f32x4 y = {0.0f, 0.0f, 0.0f, 0.0f};
      y = mma_f32(y, Tf + (16 * i) * kST + 16 * i, kST, xs, 20, lane);
#pragma unroll
      for (int e = 0; e < 4; ++e) Tf[(16 * i + acc_row(lane, e)) * kST + 16 * j + acc_col(lane)] = -y[e];
    }
    __syncthreads();
  }
  for (int e = tid; e < kC * kC; e += kThreads) {
    const int t = e >> 6, s2 = e & 63;
    const float tv = (s2 <= t) ? Tf[t * kST + s2] : 0.0f;
    const float bs = Bet[s2];
    Tp[t * kSC + s2] = to_bf16(tv * bs * Gam[s2]);
    Tpp[t * kSC + s2] = to_bf16(tv * bs);
  }
  __syncthreads();

  // ================= 4. W = T' K (-> LDS, over K), U = T'' V (-> workspace, tile order)
  const int kmax = (rb < 2) ? 32 : 64;  // T' and T'' vanish above the diagonal
  constexpr int KTW = DK / 32;
#pragma unroll
  for (int e = 0; e < KTW; ++e) {
    const int ci = chalf * KTW + e;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    acc = mma_range(acc, Tp + (16 * rb) * kSC, kSC, KT + (16 * ci) * kSC, kSC, 0, kmax, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) Ws[(16 * rb + acc_row(lane, i)) * SK + 16 * ci + acc_col(lane)] = to_bf16(acc[i]);
  }
  {
    float* ug = reinterpret_cast<float*>(base + rec.u);
    constexpr int UTW = DVT / 2;
#pragma unroll
    for (int e = 0; e < UTW; ++e) {
      const int cj = chalf * UTW + e;
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      acc = mma_range(acc, Tpp + (16 * rb) * kSC, kSC, Vt + (16 * cj) * kSC, kSC, 0, kmax, lane);
      *reinterpret_cast<f32x4*>(ug + ((static_cast<size_t>(rb) * DVT + cj) * 64 + lane) * 4) = acc;
    }
  }
  __syncthreads();

  // ================= 5. W, Kt^T = (exp(G_last - G_t) K)^T, M and gam to the workspace
  bf16_t* wg = reinterpret_cast<bf16_t*>(base + rec.w);
  for (int v = tid; v < kC * VPR; v += kThreads) {
    const int t = v / VPR, c8 = (v % VPR) * 8;
    *reinterpret_cast<uint4*>(wg + t * DK + c8) = *reinterpret_cast<const uint4*>(Ws + t * SK + c8);
  }
  bf16_t* ktg = reinterpret_cast<bf16_t*>(base + rec.kt);
  const double Glast = Gd[kC - 1];  // gates past the chunk's end are 0: G stays at its last value
  for (int ix = tid; ix < DK * (kC / 8); ix += kThreads) {
    const int i = ix / (kC / 8);
    const int t8 = (ix % (kC / 8)) * 8;
    uint32_t wv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a0 = widen(KT[i * kSC + t8 + 2 * e]) * fast_exp2(static_cast<float>(Glast - Gd[t8 + 2 * e]));
      const float a1 = widen(KT[i * kSC + t8 + 2 * e + 1]) * fast_exp2(static_cast<float>(Glast - Gd[t8 + 2 * e + 1]));
      wv[e] = static_cast<uint32_t>(to_bf16(a0)) | (static_cast<uint32_t>(to_bf16(a1)) << 16);
    }
    *reinterpret_cast<uint4*>(ktg + i * kC + t8) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  }
  bf16_t* mg = reinterpret_cast<bf16_t*>(base + rec.m);
  for (int v = tid; v < kC * (kC / 8); v += kThreads) {
    const int t = v / (kC / 8), s8 = (v % (kC / 8)) * 8;
    *reinterpret_cast<uint4*>(mg + t * kC + s8) = *reinterpret_cast<const uint4*>(Ms + t * kSC + s8);
  }
  if (w == 0) {
    float* gg = reinterpret_cast<float*>(base + rec.g);
    gg[lane] = Gam[lane];
    if (lane == 0) gg[kC] = Gam[kC - 1];
  }
  __syncthreads();  // the LDS is restaged for the next item
  }
}

// ---------------------------------------------------------------- pass 2
template <int DK, int NC>
struct StateLds {
  static constexpr int SK = DK + 8;
  static constexpr int kWs = 0;                          // W      [C][SK] bf16
  static constexpr int kQs = kWs + kC * SK * 2;          // Q      [C][SK] bf16
  static constexpr int kKT = kQs + kC * SK * 2;          // Kt^T   [DK][SC] bf16
  static constexpr int kMs = kKT + DK * kSC * 2;         // M      [C][SC] bf16
  static constexpr int kSt = kMs + kC * kSC * 2;         // S^T    [NC][SK] bf16
  static constexpr int kDt = kSt + NC * SK * 2;          // D^T    [NC][SC] bf16
  static constexpr int kGam = kDt + NC * kSC * 2;        // gam    [C] f32
  static constexpr int kOs = kGam + kC * 4;              // O      [8 waves][16][NC / 2 + 8] bf16
  static constexpr int kBytes = kOs + kWaves * 16 * (NC / 2 + 8) * 2;
  static_assert(kBytes <= 160 * 1024, "LDS budget of one gfx950 workgroup");
};

// One workgroup of 8 waves per CU (the LDS holds one): two waves per SIMD may
// use 256 registers each, which keeps the staging arrays in registers.
template <typename IO, int DK, int NC, int DVT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 2))) void chunk_state_kernel(ScanParams p, const unsigned char* ws, size_t rec_bytes,
                                                               const int32_t* cs) {
  using L_ = StateLds<DK, NC>;
  constexpr int SK = L_::SK;
  constexpr int CT = NC / 16;                   // column tiles of the block
  constexpr int CTW = CT / 2;                   // column tiles per wave in the (token, column) products
  constexpr int STW = (DK / 16) * CT / kWaves;  // state tiles per wave
  static_assert(CT % 2 == 0 && STW >= 1, "block shape");
  static_assert(STW <= CT && CT % STW == 0, "a wave's state tiles lie in one row tile");
  extern __shared__ __align__(16) unsigned char smem[];
  bf16_t* Ws = reinterpret_cast<bf16_t*>(smem + L_::kWs);
  bf16_t* Qs = reinterpret_cast<bf16_t*>(smem + L_::kQs);
  bf16_t* KTs = reinterpret_cast<bf16_t*>(smem + L_::kKT);
  bf16_t* Ms = reinterpret_cast<bf16_t*>(smem + L_::kMs);
  bf16_t* St = reinterpret_cast<bf16_t*>(smem + L_::kSt);
  bf16_t* Dt = reinterpret_cast<bf16_t*>(smem + L_::kDt);
  float* Gam = reinterpret_cast<float*>(smem + L_::kGam);
  constexpr int kSO = NC / 2 + 8;  // bf16 row stride of a wave's output block

  const int tid = static_cast<int>(threadIdx.x);
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int rb = w & 3;
  const int chalf = w >> 2;
  bf16_t* Os = reinterpret_cast<bf16_t*>(smem + L_::kOs) + w * 16 * kSO;
  int unit = static_cast<int>(blockIdx.x);
  const int cb = unit % p.col_blocks;
  unit /= p.col_blocks;
  const int h = unit % p.h_v;
  const int n = unit / p.h_v;
  const int hq = h / p.ratio;
  const int J0 = cb * NC;
  const int d_v = p.d_v;
  const int T = p.total_tokens;
  const int t_begin = seq_lo(p.cu, n, T);
  const int t_end = seq_hi(p.cu, n, T);
  const int c_first = cs[n];
  const int nchunks = (t_end - t_begin + kC - 1) / kC;
  bool has_state;
  const int sidx = state_slot(p.slots, p.num_slots, n, &has_state);
  const size_t sbase = (static_cast<size_t>(sidx) * p.h_v + h) * static_cast<size_t>(DK) * d_v;
  const Rec rec(DK, 16 * DVT);

  // ---- state slice in accumulators: wave w owns tiles w*STW .. (row tile * CT + column tile)
  f32x4 S[STW];
#pragma unroll
  for (int e = 0; e < STW; ++e) {
    const int ri = (w * STW + e) / CT, cj = (w * STW + e) % CT;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * ri + acc_row(lane, i);
      const int col = J0 + 16 * cj + acc_col(lane);
      S[e][i] = (p.s0 != nullptr && has_state && col < d_v) ? p.s0[sbase + static_cast<size_t>(row) * d_v + col] : 0.0f;
    }
  }
  auto publish_state = [&]() __attribute__((always_inline)) {  // S^T (bf16) for the next chunk's W S and Q S
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
  IO* og = static_cast<IO*>(p.out);
  const size_t qk_stride = static_cast<size_t>(p.h_qk) * DK;
  const size_t v_stride = static_cast<size_t>(p.h_v) * d_v;

  // ---- register staging of one chunk (loaded one chunk ahead)
  constexpr int VPR = DK / 8;
  constexpr int R_IT = kC * VPR / kThreads;      // W and Q rows, Kt^T
  constexpr int M_IT = kC * (kC / 8) / kThreads;
  static_assert(R_IT >= 1 && M_IT >= 1, "block shape");
  // vector-typed staging arrays stay in registers (arrays of uint4 structs
  // were left in scratch memory by the compiler)
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  u32x4 rw[R_IT], rk[R_IT];
  uint4 rq[R_IT], rm[M_IT];
  f32x4 ru[CTW];
  float rgam = 0.0f, rgl = 0.0f;
  auto fetch = [&](int j) __attribute__((always_inline)) {
    const unsigned char* base = ws + (static_cast<size_t>(c_first + j) * p.h_v + h) * rec_bytes;
    const int c0 = t_begin + j * kC;
    const int Lc = min(kC, t_end - c0);
    const bf16_t* wg = reinterpret_cast<const bf16_t*>(base + rec.w);
    const bf16_t* ktg = reinterpret_cast<const bf16_t*>(base + rec.kt);
#pragma unroll
    for (int it = 0; it < R_IT; ++it) {
      const int v = tid + it * kThreads;
      const int t = v / VPR, c8 = (v % VPR) * 8;
      rw[it] = *reinterpret_cast<const u32x4*>(wg + t * DK + c8);
      rk[it] = reinterpret_cast<const u32x4*>(ktg)[v];  // Kt^T is [DK][C]: 8 consecutive per item
      rq[it] = make_uint4(0, 0, 0, 0);
      if (t < Lc)
        rq[it] = *reinterpret_cast<const uint4*>(qg + static_cast<size_t>(c0 + t) * qk_stride +
                                                 static_cast<size_t>(hq) * DK + c8);
    }
    const bf16_t* mg = reinterpret_cast<const bf16_t*>(base + rec.m);
#pragma unroll
    for (int it = 0; it < M_IT; ++it) rm[it] = *reinterpret_cast<const uint4*>(mg + (tid + it * kThreads) * 8);
    const float* ug = reinterpret_cast<const float*>(base + rec.u);
#pragma unroll
    for (int e = 0; e < CTW; ++e) {
      const int cj = cb * CT + chalf * CTW + e;  // column tile of the whole head
      ru[e] = cj < DVT ? *reinterpret_cast<const f32x4*>(ug + ((static_cast<size_t>(rb) * DVT + cj) * 64 + lane) * 4)
                       : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    const float* gg = reinterpret_cast<const float*>(base + rec.g);
    rgam = gg[lane];  // gam_t of token lane (used by wave 0)
    rgl = gg[kC];     // gam_last
  };
  if (nchunks > 0) fetch(0);

  for (int j = 0; j < nchunks; ++j) {
    const int c0 = t_begin + j * kC;
    const int Lc = min(kC, t_end - c0);

    // ================= a. stage W, Q, Kt^T, M, gam; U to registers; fetch the next chunk
#pragma unroll
    for (int it = 0; it < R_IT; ++it) {
      const int v = tid + it * kThreads;
      const int t = v / VPR, c8 = (v % VPR) * 8;
      *reinterpret_cast<u32x4*>(Ws + t * SK + c8) = rw[it];
      *reinterpret_cast<uint4*>(Qs + t * SK + c8) = rq[it];
      const int i = (v * 8) / kC, t8 = (v * 8) % kC;
      *reinterpret_cast<u32x4*>(KTs + i * kSC + t8) = rk[it];
    }
#pragma unroll
    for (int it = 0; it < M_IT; ++it) {
      const int v = tid + it * kThreads;
      const int t = (v * 8) / kC, s8 = (v * 8) % kC;
      *reinterpret_cast<uint4*>(Ms + t * kSC + s8) = rm[it];
    }
    if (w == 0) Gam[lane] = rgam;
    f32x4 U[CTW];
#pragma unroll
    for (int e = 0; e < CTW; ++e) U[e] = ru[e];
    const float gam_last = rgl;
    __syncthreads();
    if (j + 1 < nchunks) fetch(j + 1);  // in flight while this chunk computes

    // ================= b. X = W S, Y = Q S (shared B fragments); D = U - X
    f32x4 X[CTW], Y[CTW];
#pragma unroll
    for (int e = 0; e < CTW; ++e) X[e] = Y[e] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < DK; kk += 32) {
      const bf16x8 aw = frag(Ws + (16 * rb) * SK + kk, SK, lane);
      const bf16x8 aq = frag(Qs + (16 * rb) * SK + kk, SK, lane);
#pragma unroll
      for (int e = 0; e < CTW; ++e) {
        const int cj = chalf * CTW + e;
        const bf16x8 bs = frag(St + (16 * cj) * SK + kk, SK, lane);
        X[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, bs, X[e], 0, 0, 0);
        Y[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, bs, Y[e], 0, 0, 0);
      }
    }
#pragma unroll
    for (int e = 0; e < CTW; ++e) {
      const int cj = chalf * CTW + e;
      const int t = 16 * rb + acc_row(lane, 0);
      const int col = 16 * cj + acc_col(lane);
      uint2 pk;
      pk.x = static_cast<uint32_t>(to_bf16(U[e][0] - X[e][0])) | (static_cast<uint32_t>(to_bf16(U[e][1] - X[e][1])) << 16);
      pk.y = static_cast<uint32_t>(to_bf16(U[e][2] - X[e][2])) | (static_cast<uint32_t>(to_bf16(U[e][3] - X[e][3])) << 16);
      *reinterpret_cast<uint2*>(Dt + col * kSC + t) = pk;
#pragma unroll
      for (int i = 0; i < 4; ++i) Y[e][i] *= Gam[t + i];
    }
    __syncthreads();

    // ================= c. O = scale (gam Q S + M D); the A fragment (M rows) is shared by the wave's tiles
    const int kmax = (rb < 2) ? 32 : 64;  // M vanishes above the diagonal
    for (int kk = 0; kk < kmax; kk += 32) {
      const bf16x8 am = frag(Ms + (16 * rb) * kSC + kk, kSC, lane);
#pragma unroll
      for (int e = 0; e < CTW; ++e) {
        const int cj = chalf * CTW + e;
        Y[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, frag(Dt + (16 * cj) * kSC + kk, kSC, lane), Y[e], 0, 0, 0);
      }
    }
    // the wave's 16 x NC/2 output block goes through LDS and out in 16-byte rows
    if (og != nullptr) {
#pragma unroll
      for (int e = 0; e < CTW; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) Os[acc_row(lane, i) * kSO + 16 * e + acc_col(lane)] = to_bf16(p.scale * Y[e][i]);
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
      constexpr int VPRO = NC / 16;  // 8-element vectors per row of the block
#pragma unroll
      for (int it = 0; it < 16 * VPRO / 64; ++it) {
        const int v = lane + 64 * it;
        const int r = v / VPRO, c8 = (v % VPRO) * 8;
        const int t = 16 * rb + r;
        const int col = J0 + chalf * (NC / 2) + c8;
        if (t < Lc && col < d_v)
          *reinterpret_cast<uint4*>(og + static_cast<size_t>(c0 + t) * v_stride + static_cast<size_t>(h) * d_v + col) =
              *reinterpret_cast<const uint4*>(Os + r * kSO + c8);
      }
    }
    // ================= d. S <- gam_last S + Kt^T D; a wave's state tiles share one row tile (its A fragment)
#pragma unroll
    for (int e = 0; e < STW; ++e) S[e] = S[e] * gam_last;
#pragma unroll
    for (int kk = 0; kk < kC; kk += 32) {
      const bf16x8 ak = frag(KTs + (16 * ((w * STW) / CT)) * kSC + kk, kSC, lane);
#pragma unroll
      for (int e = 0; e < STW; ++e) {
        const int cj = (w * STW + e) % CT;
        S[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, frag(Dt + (16 * cj) * kSC + kk, kSC, lane), S[e], 0, 0, 0);
      }
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

template <typename K>
hipError_t set_lds(K kern, int bytes, bool* configured) {
  if (*configured) return hipSuccess;
  const hipError_t e =
      hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) *configured = true;
  return e;
}

int split_columns(int d_v) { return d_v > 64 ? 128 : 64; }

// Persistent grid of the preparation pass: one workgroup per compute unit.
int prep_workgroups() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  return cus;
}

template <typename IO, int DK, int DVT>
hipError_t launch_dvt(const ScanParams& p, unsigned char* ws, size_t rec_bytes, int32_t* cs, const int2* info,
                      int chunk_bound, hipStream_t stream) {
  if (chunk_bound > 0 && p.h_v > 0) {
    constexpr int bytes = PrepLds<DK, DVT>::kBytes;
    const int items = chunk_bound * p.h_v;
    const unsigned grid = static_cast<unsigned>(items < prep_workgroups() ? items : prep_workgroups());
    if (p.gates.raw) {
      static bool cfg = false;
      auto kern = chunk_prep_kernel<IO, DK, DVT, true>;
      hipError_t e = set_lds(kern, bytes, &cfg);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), bytes, stream, p, ws, rec_bytes, cs, info, items);
    } else {
      static bool cfg = false;
      auto kern = chunk_prep_kernel<IO, DK, DVT, false>;
      hipError_t e = set_lds(kern, bytes, &cfg);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), bytes, stream, p, ws, rec_bytes, cs, info, items);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const unsigned blocks = static_cast<unsigned>(p.num_seqs) * p.h_v * p.col_blocks;
  if (blocks == 0) return hipSuccess;
  if (split_columns(p.d_v) == 128) {
    static bool cfg = false;
    constexpr int bytes = StateLds<DK, 128>::kBytes;
    auto kern = chunk_state_kernel<IO, DK, 128, DVT>;
    hipError_t e = set_lds(kern, bytes, &cfg);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(kThreads), bytes, stream, p, ws, rec_bytes, cs);
  } else {
    static bool cfg = false;
    constexpr int bytes = StateLds<DK, 64>::kBytes;
    auto kern = chunk_state_kernel<IO, DK, 64, DVT>;
    hipError_t e = set_lds(kern, bytes, &cfg);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(kThreads), bytes, stream, p, ws, rec_bytes, cs);
  }
  return hipGetLastError();
}

int chunk_bound_of(int num_seqs, int total_tokens) {
  return num_seqs > 0 ? (total_tokens + kC - 1) / kC + num_seqs : 0;
}

}  // namespace

bool split_supported(int io_bf16, int d_k, int d_v, const GateArgs& gates, int window) {
  return chunked_supported(io_bf16, d_k, d_v, gates, window) && d_v <= 256;
}

int split_columns_per_block(int d_v) { return split_columns(d_v); }

// Workspace: cs [N + 1] int32, info [chunk bound] int2, then the records.
static size_t table_bytes(int num_seqs, int total_tokens) {
  return align256(static_cast<size_t>(num_seqs + 1) * 4) + align256(static_cast<size_t>(chunk_bound_of(num_seqs, total_tokens)) * 8);
}

size_t split_workspace_bytes(int num_seqs, int total_tokens, int h_v, int d_k, int d_v) {
  if (num_seqs <= 0) return 0;
  const int dvt = pad16(d_v) > 128 ? 16 : 8;
  const Rec rec(d_k, 16 * dvt);
  return table_bytes(num_seqs, total_tokens) +
         static_cast<size_t>(chunk_bound_of(num_seqs, total_tokens)) * h_v * rec.bytes;
}

hipError_t launch_prefill_split(ScanParams p, void* workspace, hipStream_t stream) {
  if (p.num_seqs <= 0) return hipSuccess;
  const int dvt = pad16(p.d_v) > 128 ? 16 : 8;
  const Rec rec(p.d_k, 16 * dvt);
  // total tokens: the caller's count (the kernels clamp the sequences to it)
  const int T = p.total_tokens;
  int32_t* cs = static_cast<int32_t*>(workspace);
  int2* info = reinterpret_cast<int2*>(static_cast<unsigned char*>(workspace) +
                                       align256(static_cast<size_t>(p.num_seqs + 1) * 4));
  unsigned char* recs = static_cast<unsigned char*>(workspace) + table_bytes(p.num_seqs, T);
  hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(1024), 0, stream, p.cu, p.num_seqs, T, cs, info);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int bound = chunk_bound_of(p.num_seqs, T);
  if (p.d_k == 128)
    return dvt == 16 ? launch_dvt<bf16_t, 128, 16>(p, recs, rec.bytes, cs, info, bound, stream)
                     : launch_dvt<bf16_t, 128, 8>(p, recs, rec.bytes, cs, info, bound, stream);
  return dvt == 16 ? launch_dvt<bf16_t, 64, 16>(p, recs, rec.bytes, cs, info, bound, stream)
                   : launch_dvt<bf16_t, 64, 8>(p, recs, rec.bytes, cs, info, bound, stream);
}

}  // namespace gdn
