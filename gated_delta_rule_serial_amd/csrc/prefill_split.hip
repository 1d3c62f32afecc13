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
// A chunk table (chunk_table_kernel) maps the packed sequences to chunks.  A
// preparation pass then forms, for all chunks of all sequences at once, what
// depends on one chunk alone, into a record per (chunk, value head) in a
// caller-provided workspace; a state pass walks each sequence's chunks with
// the state in MFMA accumulators.  The preparation pass fills the whole chip
// however few sequences and heads there are, and the serial chain per chunk
// shrinks to the products that involve S.  Two pairs of passes:
//   - chunk_trec_kernel + chunk_state_kernel (one workgroup per (sequence,
//     value head, block of 64 or 128 columns)): the record holds only T' =
//     T diag(beta gam), T'' = T diag(beta), M, gam and exp(G_last - G); the
//     state pass reads K, Q and V itself and forms U = T'' V, W S = T' (K S),
//     diag(gam) Q S and Kt^T D = K^T diag(exp(G_last - G)) D;
//   - chunk_prep_kernel + chunk_rows_kernel (few units at d_k = 128: each
//     16-column tile's state rows split over four waves): the record holds W,
//     diag(gam) Q, Kt^T, M, U and gam_last.
#include <type_traits>

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

// Shared operand fragments of the state pass, per (chunk, value head): W and
// diag(gam) Q as 16 x 32 blocks (4 token tiles x DK / 32 key blocks), Kt^T
// (DK / 16 key tiles x 2 token blocks), the six lower blocks of M and the six
// of T'' = T diag(beta) (the state pass forms U = T'' V itself).  Each is
// stored as the 64 lanes x 16 bytes one wave loads for a 16x16x32 MFMA, with
// the contraction index of a block permuted so that lane group g holds
// k = 4 g .. 4 g + 3 and 16 + 4 g .. 16 + 4 g + 3: the order in which two
// stacked accumulator tiles already hold the other operand (state rows, or
// the tokens of D), so that operand never leaves the registers.
__host__ __device__ constexpr int frags_w(int dk) { return 4 * (dk / 32); }
__host__ __device__ constexpr int frags_total(int dk) { return 2 * frags_w(dk) + 2 * (dk / 16) + 12; }
// M block (token tile tt, token block kb), kb <= tt / 2
__host__ __device__ constexpr int m_frag(int tt, int kb) { return tt < 2 ? tt : 2 + 2 * (tt - 2) + kb; }

// One (chunk, value head) record of the workspace.
struct Rec {
  size_t frag, g, bytes;
  __host__ __device__ explicit Rec(int dk) {
    frag = 0;                                                // fragments [frags_total][64 lanes] x 16 B
    g = frag + static_cast<size_t>(frags_total(dk)) * 1024;  // gam_last f32 (a 256-byte slot)
    bytes = align256(g + 256);
  }
};

// The smaller record of the column-block state pass, which reads K, Q and V
// itself: T' = T diag(beta gam), T'' = T diag(beta) and M, each as its six
// lower 16 x 32 blocks (the fragment order of M above), then a 1 KiB tail with
// gam [64] and the update factors exp(G_last - G) [64] in float32 (the last
// 512 bytes unused).  T' and T'' stand in for W = T' K and U = T'' V.
constexpr int kTFrags = 18;
constexpr size_t kTRecTail = static_cast<size_t>(kTFrags) * 1024;
constexpr size_t kTRecBytes = kTRecTail + 1024;


__device__ __forceinline__ int seq_lo(const int32_t* cu, int n, int T) { return min(max(cu[n], 0), T); }
__device__ __forceinline__ int seq_hi(const int32_t* cu, int n, int T) {
  return min(max(cu[n + 1], seq_lo(cu, n, T)), T);
}

// cs[n] = chunks of the sequences before n; cs[N] = all chunks; info[c] =
// (first token, tokens) of chunk c.  A thread writes the entries of its own
// short sequences; those of long ones (up to 256 of them) are written by the
// whole block, so that one long sequence does not leave a single thread
// writing hundreds of entries.
__global__ __launch_bounds__(1024) void chunk_table_kernel(const int32_t* cu, int num_seqs, int T, int32_t* cs,
                                                           int2* info) {
  constexpr int kLongChunks = 16, kMaxLong = 256;
  __shared__ int wsum[16];
  __shared__ int nlong;
  __shared__ int4 longs[kMaxLong];  // (first token, end, first chunk) of a long sequence
  const int tid = static_cast<int>(threadIdx.x);
  if (tid == 0) nlong = 0;
  const int per = (num_seqs + 1023) / 1024;
  const int a = min(tid * per, num_seqs), b = min(a + per, num_seqs);
  auto chunks = [&](int n) { return (seq_hi(cu, n, T) - seq_lo(cu, n, T) + kC - 1) / kC; };
  int sum = 0;
  for (int n = a; n < b; ++n) sum += chunks(n);
  // the chunk counts' prefix over the threads: within each wave by lane
  // shifts, then over the 16 waves' totals (one barrier)
  const int lane = tid & 63, wv = tid >> 6;
  int incl = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < wv; ++i) before += wsum[i];
  int run = before + incl - sum;
  for (int n = a; n < b; ++n) {
    cs[n] = run;
    const int lo = seq_lo(cu, n, T), hi = seq_hi(cu, n, T);
    const int cnt = (hi - lo + kC - 1) / kC;
    const int slot = cnt > kLongChunks ? atomicAdd(&nlong, 1) : kMaxLong;
    if (slot < kMaxLong) {
      longs[slot] = make_int4(lo, hi, run, 0);
      run += cnt;
    } else {
      for (int t = lo; t < hi; t += kC) info[run++] = make_int2(t, min(kC, hi - t));
    }
  }
  __syncthreads();
  const int m = min(nlong, kMaxLong);
  // the long sequences' bounds come from LDS: no global load waits between them
  for (int i = 0; i < m; ++i) {
    const int4 L = longs[i];
    for (int t = L.x + kC * tid; t < L.y; t += kC * 1024) info[L.z + (t - L.x) / kC] = make_int2(t, min(kC, L.y - t));
  }
  if (tid == 1023) cs[num_seqs] = before + incl;
}

// ---------------------------------------------------------------- pass 1
template <int DK>
struct PrepLds {
  static constexpr int SK = DK + 8;
  static constexpr int kKs = 0;                          // K rows  [C][SK] bf16
  static constexpr int kQs = kKs + kC * SK * 2;          // Q rows  [C][SK] bf16
  static constexpr int kKT = kQs + kC * SK * 2;          // K^T     [DK][SC] bf16
  static constexpr int kAf = kKT + DK * kSC * 2;         // A       [C][SA] f32 (later T', T'')
  static constexpr int kTf = kAf + kC * kSA * 4;         // T       [C][ST] f32
  static constexpr int kMs = kTf + kC * kST * 4;         // M       [C][SC] bf16
  static constexpr int kXs = kMs + kC * kSC * 2;         // solve scratch [4][16][20] f32
  static constexpr int kGd = kXs + 4 * 16 * 20 * 4;      // G       [C] f64
  static constexpr int kGam = kGd + kC * 8;              // gam     [C] f32
  static constexpr int kBet = kGam + kC * 4;             // beta    [C] f32
  static constexpr int kKf = kBet + kC * 4;              // exp(G_last - G) [C] f32
  static constexpr int kBytes = kKf + kC * 4;
  static_assert(2 * kC * kSC * 2 <= kC * kSA * 4, "T' and T'' must fit in the A buffer");
  static_assert(kBytes <= 160 * 1024, "LDS budget of one gfx950 workgroup");
};

// Persistent: one workgroup per CU walks the (chunk, value head) items
// blockIdx.x, + gridDim.x, ...; the next item's K and Q rows and gates are
// loaded into registers while the current one computes.
template <typename IO, int DK, bool RAW>
__global__ __launch_bounds__(kThreads) void chunk_prep_kernel(ScanParams p, unsigned char* ws, size_t rec_bytes,
                                                              const int32_t* cs, const int2* __restrict__ info, int items,
                                                              int nt_stores) {
  using L_ = PrepLds<DK>;
  constexpr int SK = L_::SK;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16_t* Ks = reinterpret_cast<bf16_t*>(smem + L_::kKs);
  bf16_t* Qs = reinterpret_cast<bf16_t*>(smem + L_::kQs);
  bf16_t* KT = reinterpret_cast<bf16_t*>(smem + L_::kKT);
  float* Af = reinterpret_cast<float*>(smem + L_::kAf);
  bf16_t* Tp = reinterpret_cast<bf16_t*>(smem + L_::kAf);
  bf16_t* Tpp = reinterpret_cast<bf16_t*>(smem + L_::kAf + kC * kSC * 2);
  float* Tf = reinterpret_cast<float*>(smem + L_::kTf);
  bf16_t* Ms = reinterpret_cast<bf16_t*>(smem + L_::kMs);
  float* Xs = reinterpret_cast<float*>(smem + L_::kXs);
  double* Gd = reinterpret_cast<double*>(smem + L_::kGd);
  float* Gam = reinterpret_cast<float*>(smem + L_::kGam);
  float* Bet = reinterpret_cast<float*>(smem + L_::kBet);
  float* Kf = reinterpret_cast<float*>(smem + L_::kKf);

  const int T = p.total_tokens;
  const int total = cs[p.num_seqs] * p.h_v;  // live items; the grid covers a bound
  const int n_items = items < total ? items : total;
  const int tid = static_cast<int>(threadIdx.x);
  // wave-uniform, and the compiler is told so: branches on w must skip
  // their MFMAs, which run whatever the execution mask
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const Rec rec(DK);
  const IO* qg = static_cast<const IO*>(p.q);
  const IO* kg = static_cast<const IO*>(p.k);
  const size_t qk_stride = static_cast<size_t>(p.h_qk) * DK;

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
  // unconditional (clamped) loads: a load under a condition becomes a choice
  // between old and new values that the compiler settles with a copy waiting
  // for the load, which would stall the wave right after the load is issued
  auto info_of = [&](int item) __attribute__((always_inline)) { return info[min(item, n_items - 1) / p.h_v]; };

  // ---- register staging of one item (vector-typed, so that it stays in registers)
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  constexpr int VPR = DK / 8;
  constexpr int KQ_IT = kC * VPR / kThreads;
  static_assert(KQ_IT >= 1, "block shape");
  u32x4 rk[KQ_IT], rq[KQ_IT];
  // gate inputs of token (chunk start + lane) as raw 16-bit patterns, and the
  // head's A_log, dt_bias: converted where they are used, so that no
  // conversion waits for the loads right after they are issued
  uint32_t rg = 0u, rbt = 0u;
  float rAl = 0.0f, rdt = 0.0f;
  auto fetch = [&](const Where& at) __attribute__((always_inline)) {
    const int hq = at.h / p.ratio;
#pragma unroll
    for (int it = 0; it < KQ_IT; ++it) {
      const int v = tid + it * kThreads;
      const int t = min(v / VPR, at.Lc - 1), c8 = (v % VPR) * 8;  // rows past the chunk: zeroed when staged
      const size_t off = static_cast<size_t>(at.t0 + t) * qk_stride + static_cast<size_t>(hq) * DK + c8;
      rk[it] = *reinterpret_cast<const u32x4*>(kg + off);
      rq[it] = *reinterpret_cast<const u32x4*>(qg + off);
    }
    {
      // gate inputs of token (chunk start + lane), clamped into the chunk (wave 0
      // uses them; every wave loads, so no wave keeps an old value)
      const int tl = at.t0 + min(lane, max(at.Lc - 1, 0));
      const size_t gi = static_cast<size_t>(tl) * p.h_v + at.h;
      const size_t bi = p.gates.beta_shared ? static_cast<size_t>(tl) : gi;
      const IO* bsrc = static_cast<const IO*>(RAW ? p.gates.b : p.gates.beta);
      const IO* gsrc = p.gates.decays ? static_cast<const IO*>(RAW ? p.gates.a : p.gates.g) : bsrc;
      rg = reinterpret_cast<const uint16_t*>(gsrc)[p.gates.decays ? gi : bi];
      rbt = reinterpret_cast<const uint16_t*>(bsrc)[bi];
      if constexpr (RAW) {
        rAl = p.gates.A_log[at.h];
        rdt = p.gates.dt_bias[at.h];
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

  // Blocks go round-robin over the 8 XCDs.  Where the grid allows, the ratio
  // value heads of one (chunk, q/k head) go to blocks 8 apart, on one XCD,
  // which run them at about the same time and read K and Q once through its L2.
  int item = static_cast<int>(blockIdx.x);
  {
    const int R = p.ratio, G = static_cast<int>(gridDim.x);
    if (R > 1 && G % (8 * R) == 0) {
      const int xcd = item % 8, j = item / 8;
      item = (j / R) * (8 * R) + xcd * R + j % R;
    }
  }
  if (item >= n_items) return;
  Where at = locate(item, info[item / p.h_v]);
  fetch(at);
  int2 next_info = info_of(item + static_cast<int>(gridDim.x));  // one item ahead of the fetch
  for (; item < n_items; item += static_cast<int>(gridDim.x)) {
    const int h = at.h;
    const int Lc = at.Lc;
    unsigned char* base = ws + (static_cast<size_t>(at.c) * p.h_v + h) * rec_bytes;

    // ================= 1. stage K and Q rows; gates and the prefix sum of the log-decay
#pragma unroll
    for (int it = 0; it < KQ_IT; ++it) {
      const int v = tid + it * kThreads;
      const int t = v / VPR, c8 = (v % VPR) * 8;
      const u32x4 zero = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(Ks + t * SK + c8) = t < Lc ? rk[it] : zero;
      *reinterpret_cast<u32x4*>(Qs + t * SK + c8) = t < Lc ? rq[it] : zero;
    }
    if (w == 0) {
      float g = 0.0f, b = 0.0f;
      if (lane < Lc) {
        if constexpr (RAW) {
          g = p.gates.decays ? gate_log_decay(widen_bits16<IO>(rg), rAl, rdt) : 0.0f;
          b = gate_sigmoid(widen_bits16<IO>(rbt));
        } else {
          g = p.gates.decays ? widen_bits16<IO>(rg) : 0.0f;
          b = widen_bits16<IO>(rbt);
        }
        g = fmaxf(g, kMinLogDecay);
      }
      const double G = wave_prefix_sum(static_cast<double>(g) * kLog2e, lane);
      Gd[lane] = G;
      Gam[lane] = fast_exp2(static_cast<float>(G));
      Bet[lane] = b;
      // the state-update factor exp(G_last - G_t); gates past the chunk's end
      // are 0, so G_last is the prefix at the last lane
      Kf[lane] = fast_exp2(static_cast<float>(__shfl(G, kC - 1) - G));
    }
    __syncthreads();

  // ================= 2. A = strictly lower (beta_t exp(G_t - G_s) k_t.k_s), K^T, and the
  // diagonal 16 x 16 blocks of T = (I + A)^-1.  Waves 0-3 form the diagonal
  // tile of A in block w and invert that block at once; waves 4-7 transpose K
  // and form the six tiles of A below the diagonal blocks.  The ten lower
  // tiles of M = lower (exp(G_t - G_s) q_t.k_s), which only the record reads,
  // are formed by the waves that the block substitution leaves idle.
  // exp(G_t - G_s) for the accumulator tile (token tile tb, token tile cb), 0 where s > t;
  // the lane's four rows are 16 tb + 4 g + i, read at once (no load waits inside a branch)
  auto tile_decay = [&](int tb, int cb) __attribute__((always_inline)) {
    const int s_ = 16 * cb + acc_col(lane);
    const int t0 = 16 * tb + acc_row(lane, 0);
    const double Gs = Gd[s_];
    const double2 ga = *reinterpret_cast<const double2*>(Gd + t0);
    const double2 gb = *reinterpret_cast<const double2*>(Gd + t0 + 2);
    const double gt[4] = {ga.x, ga.y, gb.x, gb.y};
    f32x4 dec;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = fast_exp2(static_cast<float>(gt[i] - Gs));  // selected away (even if infinite) where s > t
      dec[i] = s_ <= t0 + i ? e : 0.0f;
    }
    return dec;
  };
  auto store_a = [&](int tb, int cb, f32x4 pacc) __attribute__((always_inline)) {
    const f32x4 dec = tile_decay(tb, cb);
    const int s_ = 16 * cb + acc_col(lane);
    const int t0 = 16 * tb + acc_row(lane, 0);
    const f32x4 bt = *reinterpret_cast<const f32x4*>(Bet + t0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = bt[i] * dec[i] * pacc[i];
      Af[(t0 + i) * kSA + s_] = (s_ < t0 + i) ? a : 0.0f;
    }
  };
  auto store_m = [&](int tb, int cb, f32x4 racc) __attribute__((always_inline)) {
    const f32x4 dec = tile_decay(tb, cb);
    const int s_ = 16 * cb + acc_col(lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) Ms[(16 * tb + acc_row(lane, i)) * kSC + s_] = to_bf16(dec[i] * racc[i]);
  };
  if (w < 4) {
    f32x4 pacc = {0.0f, 0.0f, 0.0f, 0.0f};
    pacc = mma<DK>(pacc, Ks + 16 * w * SK, SK, Ks + 16 * w * SK, SK, lane);
    store_a(w, w, pacc);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the block is in LDS for this wave's reads
    __builtin_amdgcn_wave_barrier();
    // forward substitution, one column of the block per lane (lanes 16-63 repeat lanes 0-15)
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
  } else {
    for (int ix = tid - 4 * 64; ix < DK * (kC / 8); ix += 4 * 64) {
      const int i = ix % DK;
      const int t8 = (ix / DK) * 8;
      uint32_t wv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        wv[e] = static_cast<uint32_t>(Ks[(t8 + 2 * e) * SK + i]) | (static_cast<uint32_t>(Ks[(t8 + 2 * e + 1) * SK + i]) << 16);
      *reinterpret_cast<uint4*>(KT + i * kSC + t8) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    }
    // the tiles of A below the diagonal blocks, (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
    for (int q = w - 4; q < 6; q += 4) {
      const int tb = q < 1 ? 1 : (q < 3 ? 2 : 3);
      const int cb = q - tb * (tb - 1) / 2;
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      acc = mma<DK>(acc, Ks + 16 * tb * SK, SK, Ks + 16 * cb * SK, SK, lane);
      store_a(tb, cb, acc);
    }
  }
  // the next item's inputs, in flight while this one computes: issued once
  // the previous item's record stores have drained, so that the loads do not
  // queue behind them, and well ahead of this item's own stores
  {
    const int next = item + static_cast<int>(gridDim.x);
    if (next < n_items) {
      at = locate(next, next_info);
      fetch(at);
      next_info = info_of(next + static_cast<int>(gridDim.x));
    }
  }
  __syncthreads();

  // ================= 3. the blocks of T below the diagonal, by block substitution;
  // beside the first two steps, waves 3-7 form the lower tiles of M
  // ((0,0) (1,0) (1,1) (2,0) .. (3,3), five per step)
  for (int dist = 1; dist < 4; ++dist) {
    const int i = w + dist, j = w;
    const int mq = 5 * (dist - 1) + (w - 3);
    if (w >= 3 && mq < 10) {
      int tb = 0;
      while ((tb + 1) * (tb + 2) / 2 <= mq) ++tb;
      const int cb = mq - tb * (tb + 1) / 2;
      f32x4 racc = {0.0f, 0.0f, 0.0f, 0.0f};
      racc = mma<DK>(racc, Qs + 16 * tb * SK, SK, Ks + 16 * cb * SK, SK, lane);
      store_m(tb, cb, racc);
    }
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
  // T' = T diag(beta gam) and T'' = T diag(beta) in bf16, lower triangle, four columns per thread
  for (int e = tid; e < kC * kC / 4; e += kThreads) {
    const int t = e >> 4, s4 = (e & 15) * 4;
    const f32x4 tv = *reinterpret_cast<const f32x4*>(Tf + t * kST + s4);
    const f32x4 bs = *reinterpret_cast<const f32x4*>(Bet + s4);
    const f32x4 gm = *reinterpret_cast<const f32x4*>(Gam + s4);
    uint32_t wp[2], wpp[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      float a2[2], b2[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int c = 2 * h2 + k;
        const float x = (s4 + c <= t) ? tv[c] : 0.0f;
        b2[k] = x * bs[c];
        a2[k] = b2[k] * gm[c];
      }
      wp[h2] = static_cast<uint32_t>(to_bf16(a2[0])) | (static_cast<uint32_t>(to_bf16(a2[1])) << 16);
      wpp[h2] = static_cast<uint32_t>(to_bf16(b2[0])) | (static_cast<uint32_t>(to_bf16(b2[1])) << 16);
    }
    *reinterpret_cast<uint2*>(Tp + t * kSC + s4) = make_uint2(wp[0], wp[1]);
    *reinterpret_cast<uint2*>(Tpp + t * kSC + s4) = make_uint2(wpp[0], wpp[1]);
  }
  __syncthreads();

  // ================= 4. the record: W from MFMA accumulators, then diag(gam) Q, Kt^T, M and T'' from LDS
  {
    typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
    constexpr int KB = DK / 32;
    constexpr int FQ = frags_w(DK), FK = 2 * frags_w(DK), FM = FK + 2 * (DK / 16), FT = FM + 6, NF = frags_total(DK);
    u32x4_t* fr = reinterpret_cast<u32x4_t*>(base + rec.frag);
    auto put = [&](int f, u32x4_t piece) __attribute__((always_inline)) {
      if (nt_stores)
        __builtin_nontemporal_store(piece, fr + f * 64 + lane);
      else
        fr[f * 64 + lane] = piece;
    };
    auto bf2 = [](float a, float b) __attribute__((always_inline)) {
      return static_cast<uint32_t>(to_bf16(a)) | (static_cast<uint32_t>(to_bf16(b)) << 16);
    };
    // W^T = K^T T'^T per (key tile, token tile tw): accumulator element i of lane l
    // holds W[16 tw + l % 16][16 kt + 4 (l / 16) + i], so the tiles of key tiles
    // 2 kb and 2 kb + 1 stack into the W fragment (tw, kb) as it is stored
    const int tw = w & 3;
    const int kmax_w = tw < 2 ? 32 : 64;  // T' vanishes above the diagonal
#pragma unroll
    for (int e = 0; e < KB / 2; ++e) {
      const int kb = (w >> 2) * (KB / 2) + e;
      f32x4 lo = {0.0f, 0.0f, 0.0f, 0.0f}, hi = {0.0f, 0.0f, 0.0f, 0.0f};
      lo = mma_range(lo, KT + (32 * kb) * kSC, kSC, Tp + (16 * tw) * kSC, kSC, 0, kmax_w, lane);
      hi = mma_range(hi, KT + (32 * kb + 16) * kSC, kSC, Tp + (16 * tw) * kSC, kSC, 0, kmax_w, lane);
      put(tw * KB + kb, u32x4_t{bf2(lo[0], lo[1]), bf2(lo[2], lo[3]), bf2(hi[0], hi[1]), bf2(hi[2], hi[3])});
    }
    const int g = lane >> 4, r = lane & 15;
    // k values of this lane's slots, relative to the block: 4 g + e (e < 4), 16 + 4 g + (e - 4)
    auto slot_k = [&](int e) __attribute__((always_inline)) { return 4 * g + (e & 3) + 16 * (e >> 2); };
    auto pick = [&](const bf16_t* row, int kb) __attribute__((always_inline)) {
      const uint2 lo = *reinterpret_cast<const uint2*>(row + 32 * kb + 4 * g);
      const uint2 hi = *reinterpret_cast<const uint2*>(row + 32 * kb + 16 + 4 * g);
      return u32x4_t{lo.x, lo.y, hi.x, hi.y};
    };
    auto scaled = [&](u32x4_t x, auto factor) __attribute__((always_inline)) {
      u32x4_t y;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        y[q] = bf2(widen(static_cast<bf16_t>(x[q] & 0xffffu)) * factor(2 * q),
                   widen(static_cast<bf16_t>(x[q] >> 16)) * factor(2 * q + 1));
      return y;
    };
    for (int f = FQ + w; f < NF; f += kWaves) {
      u32x4_t piece;
      if (f < FK) {
        const int t = 16 * ((f - FQ) / KB) + r;
        const float gm = Gam[t];
        piece = scaled(pick(Qs + t * SK, (f - FQ) % KB), [&](int) { return gm; });
      } else if (f < FM) {
        const int kb = (f - FK) & 1;
        piece = scaled(pick(KT + (16 * ((f - FK) >> 1) + r) * kSC, kb), [&](int e) { return Kf[32 * kb + slot_k(e)]; });
      } else {
        // the six lower blocks of M, then of T'' (the same block order)
        const int mf = f < FT ? f - FM : f - FT;
        const int tt = mf < 2 ? mf : 2 + ((mf - 2) >> 1);
        const int kb = mf < 2 ? 0 : ((mf - 2) & 1);
        piece = pick((f < FT ? Ms : Tpp) + (16 * tt + r) * kSC, kb);
      }
      put(f, piece);
    }
    if (tid == 0) *reinterpret_cast<float*>(base + rec.g) = Gam[kC - 1];
  }
  __syncthreads();  // the LDS is restaged for the next item
  }
}

// ---------------------------------------------------------------- pass 1, small record
// The preparation pass of the column-block state pass (T', T'' and M
// record): four waves per workgroup and two workgroups per compute unit, so
// that one's barriers and the latency of the substitution overlap the other's
// products.  Two fit in the LDS because Q's rows hold the substitution's
// scratch once M is formed.
constexpr int kTWaves = 4;
constexpr int kTThreads = 64 * kTWaves;

template <int DK, int NH>
struct TPrepLds {
  static constexpr int SK = DK + 8;
  static constexpr int SA = kC + 4;                  // f32 row stride of A: 4 rows of a tile 16 banks apart
  static constexpr int kKs = 0;                      // K rows [C][SK] bf16
  static constexpr int kQs = kKs + kC * SK * 2;      // Q rows [C][SK] bf16, later the scratch [4][16][20] f32
  static constexpr int kAf = kQs + kC * SK * 2;      // A [C][SA] f32
  static constexpr int kTf = kAf + kC * SA * 4;      // T [C][ST] f32
  static constexpr int kMs = kTf + kC * kST * 4;     // M [C][SC] bf16
  static constexpr int kGd = kMs + kC * kSC * 2;     // G [NH][C] f64, one set per value head of a unit
  static constexpr int kGam = kGd + NH * kC * 8;     // gam [NH][C] f32
  static constexpr int kBet = kGam + NH * kC * 4;    // beta [NH][C] f32
  static constexpr int kKf = kBet + NH * kC * 4;     // exp(G_last - G) [NH][C] f32
  static constexpr int kBytes = kKf + NH * kC * 4;
  static_assert(4 * 16 * 20 * 4 <= kC * SK * 2, "the scratch fits in Q's rows");
  static_assert(2 * kBytes <= 160 * 1024, "two workgroups per gfx950 compute unit");
};

// Persistent: the workgroups walk the units blockIdx.x, + gridDim.x, ...;
// the next unit's K and Q rows and gates are loaded into registers while the
// current one computes.  A unit is a chunk and NH value heads that read the
// same q/k head (NH = 2 where the head ratio is even): their K K^T and Q K^T
// are one product, formed once and kept in registers, and each head then
// takes its own decay and gates (A, M), substitution and record in turn.
template <typename IO, int DK, bool RAW, int NH, bool PLAIN>
__global__ __launch_bounds__(kTThreads) void chunk_trec_kernel(ScanParams p, unsigned char* ws, const int32_t* cs,
                                                               const int2* __restrict__ info, int units) {
  using L_ = TPrepLds<DK, NH>;
  constexpr int SK = L_::SK;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16_t* Ks = reinterpret_cast<bf16_t*>(smem + L_::kKs);
  bf16_t* Qs = reinterpret_cast<bf16_t*>(smem + L_::kQs);
  float* Xs = reinterpret_cast<float*>(smem + L_::kQs);
  constexpr int kSA = L_::SA;  // this kernel's stride of A
  float* Af = reinterpret_cast<float*>(smem + L_::kAf);
  float* Tf = reinterpret_cast<float*>(smem + L_::kTf);
  bf16_t* Ms = reinterpret_cast<bf16_t*>(smem + L_::kMs);

  const int hpu = p.h_v / NH;                       // units per chunk
  const int total = cs[p.num_seqs] * hpu;           // live units; the grid covers a bound
  // PLAIN, the gated and linear rules (no delta correction): the record holds
  // T'' = I and T' = 0, so the state pass takes D = V
  constexpr bool plain = PLAIN;
  const int n_units = units < total ? units : total;
  const int tid = static_cast<int>(threadIdx.x);
  // wave-uniform, and the compiler is told so: branches on w must skip
  // their MFMAs, which run whatever the execution mask
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4, r = lane & 15;
  const IO* qg = static_cast<const IO*>(p.q);
  const IO* kg = static_cast<const IO*>(p.k);
  const size_t qk_stride = static_cast<size_t>(p.h_qk) * DK;

  // unit u is chunk c = u / hpu (first token, tokens from the chunk table),
  // value heads NH (u % hpu) .. + NH - 1
  struct Where {
    int c, h, t0, Lc;
  };
  auto locate = [&](int unit, int2 ci) __attribute__((always_inline)) {
    Where at;
    at.c = unit / hpu;
    at.h = NH * (unit % hpu);
    at.t0 = ci.x;
    at.Lc = ci.y;
    return at;
  };
  // unconditional (clamped) loads, so that no wait for them falls right after they are issued
  auto info_of = [&](int unit) __attribute__((always_inline)) { return info[min(unit, n_units - 1) / hpu]; };

  // ---- register staging of one unit's K and Q rows and gate inputs
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  constexpr int VPR = DK / 8;
  constexpr int KQ_IT = kC * VPR / kTThreads;
  static_assert(KQ_IT >= 1, "block shape");
  u32x4_t rk[KQ_IT], rq[KQ_IT];
  uint32_t rg[NH], rbt[NH];
  float rAl[NH], rdt[NH];
  auto fetch = [&](const Where& at) __attribute__((always_inline)) {
    const int hq = at.h / p.ratio;
#pragma unroll
    for (int it = 0; it < KQ_IT; ++it) {
      const int v = tid + it * kTThreads;
      const int t = min(v / VPR, at.Lc - 1), c8 = (v % VPR) * 8;  // rows past the chunk: zeroed when staged
      const size_t off = static_cast<size_t>(at.t0 + t) * qk_stride + static_cast<size_t>(hq) * DK + c8;
      rk[it] = *reinterpret_cast<const u32x4_t*>(kg + off);
      rq[it] = *reinterpret_cast<const u32x4_t*>(qg + off);
    }
    // gate inputs of token (chunk start + lane), clamped into the chunk
    const int tl = at.t0 + min(lane, max(at.Lc - 1, 0));
#pragma unroll
    for (int hs = 0; hs < NH; ++hs) {
      const int hh = at.h + hs;
      const size_t gi = static_cast<size_t>(tl) * p.h_v + hh;
      const size_t bi = p.gates.beta_shared ? static_cast<size_t>(tl) : gi;
      // a rule without the decay or the delta correction reads K's first
      // element in place of the gate it lacks (loaded, not used)
      const IO* bsrc = PLAIN ? kg : static_cast<const IO*>(RAW ? p.gates.b : p.gates.beta);
      const IO* gsrc = p.gates.decays ? static_cast<const IO*>(RAW ? p.gates.a : p.gates.g) : kg;
      rg[hs] = reinterpret_cast<const uint16_t*>(gsrc)[p.gates.decays ? gi : 0];
      rbt[hs] = reinterpret_cast<const uint16_t*>(bsrc)[PLAIN ? 0 : bi];
      if constexpr (RAW) {
        rAl[hs] = p.gates.A_log[hh];
        rdt[hs] = p.gates.dt_bias[hh];
      } else {
        rAl[hs] = rdt[hs] = 0.0f;
      }
    }
  };

  // the upper tiles of M stay zero for every item
  for (int e = tid; e < 6 * 256; e += kTThreads) {
    const int tile = e >> 8;
    const int tb = tile < 3 ? 0 : (tile < 5 ? 1 : 2);
    const int cs_ = tile < 3 ? tile + 1 : (tile < 5 ? tile - 1 : 3);
    const int t = 16 * tb + ((e & 255) >> 4), s = 16 * cs_ + (e & 15);
    Ms[t * kSC + s] = 0;
  }

  // exp(G_t - G_s) for the accumulator tile (token tile tb, token tile cb), 0
  // where s > t, from the prefix sums Gd of one head; the lane's four rows are
  // 16 tb + 4 g + i, read at once
  auto tile_decay = [&](const double* Gd, int tb, int cb) __attribute__((always_inline)) {
    const int s_ = 16 * cb + acc_col(lane);
    const int t0 = 16 * tb + acc_row(lane, 0);
    const double Gs = Gd[s_];
    const double2 ga = *reinterpret_cast<const double2*>(Gd + t0);
    const double2 gb = *reinterpret_cast<const double2*>(Gd + t0 + 2);
    const double gt[4] = {ga.x, ga.y, gb.x, gb.y};
    f32x4 dec;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = fast_exp2(static_cast<float>(gt[i] - Gs));  // selected away (even if infinite) where s > t
      dec[i] = s_ <= t0 + i ? e : 0.0f;
    }
    return dec;
  };
  // The twenty tile products of a unit: the lower tiles of K K^T (A, with
  // beta and the decay) and of Q K^T (M, with the decay).  Wave w forms the
  // K K^T tiles of token tile w ((w, cb), cb <= w) and the Q K^T tiles of
  // token tile 3 - w ((3 - w, cb), cb <= 3 - w), five each: it holds the
  // fragments of its own K and Q rows and reads each K tile cb once for both
  // families (K tile w is its own B operand), 18 tile reads from LDS per unit
  // instead of the 40 of one pair of operand tiles per product.  The raw
  // products stay in registers, indexed by their column tile (rawA[cb] for
  // cb <= w, rawM[cb] for cb <= 3 - w); each head's epilogue reads them.
  f32x4 rawA[4], rawM[4];
  auto products = [&]() __attribute__((always_inline)) {
    constexpr int NK = DK / 32;
    const int wm = 3 - w;
    bf16x8 ka[NK], qa[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      ka[kk] = frag(Ks + 16 * w * SK + 32 * kk, SK, lane);
      qa[kk] = frag(Qs + 16 * wm * SK + 32 * kk, SK, lane);
    }
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      if (cb > w && cb > wm) break;
      bf16x8 kb[NK];
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) kb[kk] = cb == w ? ka[kk] : frag(Ks + 16 * cb * SK + 32 * kk, SK, lane);
      if (cb <= w) {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kk], kb[kk], acc, 0, 0, 0);
        rawA[cb] = acc;
      }
      if (cb <= wm) {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kk], kb[kk], acc, 0, 0, 0);
        rawM[cb] = acc;
      }
    }
  };
  // No A or T tile above the diagonal is ever read (the solve reads below the
  // diagonal of its block, the block substitution the lower blocks, the record
  // masks the upper part), so in a pair of heads the second head's diagonal
  // block w waits there: its A tile, formed with the first head's tiles, and
  // its T block, solved beside the first head's, sit in the upper tile U(w) of
  // Af and of Tf, (0,1), (0,2), (0,3) and (1,2) for w = 0 .. 3.
  static_assert(kST == L_::SA, "A and T share the row stride");
  const int upper_off = (w < 3 ? 0 : 16 * kSA) + 16 * (w < 3 ? w + 1 : 2);
  // one head's A and M tiles from the raw products, in the order products() left
  // them; with diag_next also the next head's diagonal A tile, into U(w)
  auto epilogue = [&](int hs, bool diag_next) __attribute__((always_inline)) {
    const double* Gd = reinterpret_cast<const double*>(smem + L_::kGd) + hs * kC;
    const float* Bet = reinterpret_cast<const float*>(smem + L_::kBet) + hs * kC;
    const int wm = 3 - w;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      if (cb > w && cb > wm) break;
#pragma unroll
      for (int fam = 0; fam < 2; ++fam) {
        const int tb = fam == 0 ? w : wm;
        if (cb > tb) continue;
        const f32x4 acc = fam == 0 ? rawA[cb] : rawM[cb];
        const f32x4 dec = tile_decay(Gd, tb, cb);
        const int s_ = 16 * cb + acc_col(lane);
        const int t0 = 16 * tb + acc_row(lane, 0);
        if (fam == 0) {
          const f32x4 bt = *reinterpret_cast<const f32x4*>(Bet + t0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float a = bt[i] * dec[i] * acc[i];
            Af[(t0 + i) * kSA + s_] = (s_ < t0 + i) ? a : 0.0f;
          }
          if (NH == 2 && diag_next && cb == tb) {
            const f32x4 dec1 = tile_decay(Gd + kC, tb, cb);
            const f32x4 bt1 = *reinterpret_cast<const f32x4*>(Bet + kC + t0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float a = bt1[i] * dec1[i] * acc[i];
              Af[upper_off + acc_row(lane, i) * kSA + acc_col(lane)] = (s_ < t0 + i) ? a : 0.0f;
            }
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) Ms[(t0 + i) * kSC + s_] = to_bf16(dec[i] * acc[i]);
        }
      }
    }
  };

  // Blocks go round-robin over the 8 XCDs.  Where the grid allows, the units
  // of one (chunk, q/k head) go to blocks 8 apart, on one XCD, which run them
  // at about the same time and read K and Q once through its L2.
  int unit = static_cast<int>(blockIdx.x);
  {
    const int R = p.ratio / NH, G = static_cast<int>(gridDim.x);
    if (R > 1 && G % (8 * R) == 0) {
      const int xcd = unit % 8, j = unit / 8;
      unit = (j / R) * (8 * R) + xcd * R + j % R;
    }
  }
  if (unit >= n_units) return;
  Where at = locate(unit, info[unit / hpu]);
  fetch(at);
  int2 next_info = info_of(unit + static_cast<int>(gridDim.x));  // one unit ahead of the fetch
  for (; unit < n_units; unit += static_cast<int>(gridDim.x)) {
    const int h0 = at.h;
    const int c = at.c;
    const int Lc = at.Lc;

    // ================= 1. stage K and Q rows; per head: gates and the prefix sum of the log-decay
#pragma unroll
    for (int it = 0; it < KQ_IT; ++it) {
      const int v = tid + it * kTThreads;
      const int t = v / VPR, c8 = (v % VPR) * 8;
      const u32x4_t zero = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4_t*>(Ks + t * SK + c8) = t < Lc ? rk[it] : zero;
      *reinterpret_cast<u32x4_t*>(Qs + t * SK + c8) = t < Lc ? rq[it] : zero;
    }
    if (w == 0) {
#pragma unroll
      for (int hs = 0; hs < NH; ++hs) {
        float gv = 0.0f, b = 0.0f;
        if (lane < Lc) {
          if constexpr (RAW) {
            gv = p.gates.decays ? gate_log_decay(widen_bits16<IO>(rg[hs]), rAl[hs], rdt[hs]) : 0.0f;
            b = gate_sigmoid(widen_bits16<IO>(rbt[hs]));
          } else {
            gv = p.gates.decays ? widen_bits16<IO>(rg[hs]) : 0.0f;
            b = widen_bits16<IO>(rbt[hs]);
          }
          gv = fmaxf(gv, kMinLogDecay);
          if (PLAIN) b = 1.0f;
        }
        const double G = wave_prefix_sum(static_cast<double>(gv) * kLog2e, lane);
        reinterpret_cast<double*>(smem + L_::kGd)[hs * kC + lane] = G;
        reinterpret_cast<float*>(smem + L_::kGam)[hs * kC + lane] = fast_exp2(static_cast<float>(G));
        reinterpret_cast<float*>(smem + L_::kBet)[hs * kC + lane] = b;
        // the state-update factor exp(G_last - G_t); gates past the chunk's end
        // are 0, so G_last is the prefix at the last lane
        reinterpret_cast<float*>(smem + L_::kKf)[hs * kC + lane] = fast_exp2(static_cast<float>(__shfl(G, kC - 1) - G));
      }
    }
    __syncthreads();

    // ================= 2. the twenty tile products (once for the unit's heads)
    products();
#pragma unroll
    for (int hs = 0; hs < NH; ++hs) {
      const float* Gam = reinterpret_cast<const float*>(smem + L_::kGam) + hs * kC;
      const float* Bet = reinterpret_cast<const float*>(smem + L_::kBet) + hs * kC;
      const float* Kf = reinterpret_cast<const float*>(smem + L_::kKf) + hs * kC;
      unsigned char* base = ws + (static_cast<size_t>(c) * p.h_v + h0 + hs) * kTRecBytes;

      // ---- this head's A and M tiles, then the diagonal 16 x 16 block w of
      // T = (I + A)^-1 by forward substitution, one column per lane: lanes
      // 0-15 this head's, lanes 16-31 in a pair the second head's (from and to
      // the upper tiles U(w)), the other lanes repeat them.  The second head
      // of a pair moves its solved block into place.
      epilogue(hs, hs == 0);
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the diagonal block is in LDS for this wave's reads
      __builtin_amdgcn_wave_barrier();
      if (plain) {
        // no delta correction: T = I, nothing to solve
      } else if (NH == 2 && hs == 1) {
        if (lane < 16) {
#pragma unroll
          for (int rr = 0; rr < 16; ++rr)
            Tf[(16 * w + rr) * kST + 16 * w + lane] = Tf[upper_off + rr * kST + lane];
        }
      } else {
        const int cc = lane & 15;
        const int boff = NH == 2 && (lane & 16) ? upper_off : (16 * w) * kSA + 16 * w;
        const float* Ab = Af + boff;
        float d[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          float x0 = (rr == cc) ? 1.0f : 0.0f, x1 = 0.0f;
#pragma unroll
          for (int s2 = 0; s2 < rr; s2 += 2) {
            x0 = fmaf(-Ab[rr * kSA + s2], d[s2], x0);
            if (s2 + 1 < rr) x1 = fmaf(-Ab[rr * kSA + s2 + 1], d[s2 + 1], x1);
          }
          d[rr] = x0 + x1;
        }
        if (lane < (NH == 2 ? 32 : 16)) {
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) Tf[boff + rr * kST + cc] = d[rr];
        }
      }
      // the next unit's inputs, in flight while this one computes
      if (hs == 0) {
        const int next = unit + static_cast<int>(gridDim.x);
        if (next < n_units) {
          at = locate(next, next_info);
          fetch(at);
          next_info = info_of(next + static_cast<int>(gridDim.x));
        }
      }
      __syncthreads();

      // ================= 3. the blocks of T below the diagonal, by block
      // substitution: T_ij = -T_ii sum_{k = j .. i-1} A_ik T_kj
      for (int dist = 1; dist < (plain ? 1 : 4); ++dist) {
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

      // ================= 4. the record: T' = T diag(beta gam) and T'' = T diag(beta)
      // formed in bf16 straight into their fragments (lower triangle), the M
      // blocks, then gam and exp(G_last - G)
      {
        u32x4_t* fr = reinterpret_cast<u32x4_t*>(base);
        for (int f = w; f < 12; f += kTWaves) {
          const int mf = f % 6;
          const int tt = mf < 2 ? mf : 2 + ((mf - 2) >> 1);
          const int kb = mf < 2 ? 0 : ((mf - 2) & 1);
          const int t = 16 * tt + r;
          if (f < 6) {
            uint32_t wp[4], wpp[4];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const int s4 = 32 * kb + 16 * hh + 4 * g;
              const f32x4 tv = *reinterpret_cast<const f32x4*>(Tf + t * kST + s4);
              const f32x4 bs = *reinterpret_cast<const f32x4*>(Bet + s4);
              const f32x4 gm = *reinterpret_cast<const f32x4*>(Gam + s4);
#pragma unroll
              for (int h2 = 0; h2 < 2; ++h2) {
                float a2[2], b2[2];
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                  const int cix = 2 * h2 + k;
                  // without the delta correction T = I: T'' = I and T' = 0 (D = V)
                  const float x = plain ? (s4 + cix == t ? 1.0f : 0.0f) : (s4 + cix <= t) ? tv[cix] : 0.0f;
                  b2[k] = x * bs[cix];
                  a2[k] = plain ? 0.0f : b2[k] * gm[cix];
                }
                wp[2 * hh + h2] = static_cast<uint32_t>(to_bf16(a2[0])) | (static_cast<uint32_t>(to_bf16(a2[1])) << 16);
                wpp[2 * hh + h2] = static_cast<uint32_t>(to_bf16(b2[0])) | (static_cast<uint32_t>(to_bf16(b2[1])) << 16);
              }
            }
            __builtin_nontemporal_store(u32x4_t{wp[0], wp[1], wp[2], wp[3]}, fr + f * 64 + lane);
            __builtin_nontemporal_store(u32x4_t{wpp[0], wpp[1], wpp[2], wpp[3]}, fr + (f + 6) * 64 + lane);
          } else {
            const bf16_t* row = Ms + t * kSC;
            const uint2 lo = *reinterpret_cast<const uint2*>(row + 32 * kb + 4 * g);
            const uint2 hi = *reinterpret_cast<const uint2*>(row + 32 * kb + 16 + 4 * g);
            __builtin_nontemporal_store(u32x4_t{lo.x, lo.y, hi.x, hi.y}, fr + (f + 6) * 64 + lane);
          }
        }
        if (tid < 32) {
          const f32x4 v4 = *reinterpret_cast<const f32x4*>((tid < 16 ? Gam : Kf) + 4 * (tid & 15));
          __builtin_nontemporal_store(v4, reinterpret_cast<f32x4*>(base + kTRecTail) + tid);
        }
      }
      __syncthreads();  // A, M and T are rewritten by the next head or unit
    }
  }
}

// ---------------------------------------------------------------- pass 2
constexpr int kStateWaves = 4;
constexpr int kStateTouchAhead = 1;  // one-buffer state pass: chunks between a line's touch and its load

// Global and LDS address spaces, as the direct global-to-LDS load takes them.
#define GDN_GLOBAL(ptr) ((const __attribute__((address_space(1))) void*)(ptr))
#define GDN_LDS(ptr) ((__attribute__((address_space(3))) void*)(ptr))

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane i passes the address of four consecutive 16-bit elements (piece
// i) and receives element i % 4 of pieces i / 4, 4 + i / 4, 8 + i / 4 and
// 12 + i / 4: when lane i points at row i / 4, columns 4 (i % 4) .. +3 of a
// 4 x 16 block, it receives column i of the four rows (checked on the hardware).
__device__ __forceinline__ s16x4 lds_read_tr(const bf16_t* ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<bf16_t*>(ptr)));
}

// LDS of the column-block state pass, per chunk buffer: the chunk's K and Q
// rows (all d_k keys of the q/k head), its V rows over the block's columns
// and its record.  Rows are stored as 16-byte pieces, piece c of row t at
// position c ^ row_swizzle(t).  The swizzle is a permutation of t's low four
// bits (t1 t0 into bits 2-1, t2 into bit 0, t3 kept), so that both kinds of
// read below touch distinct banks: 16 consecutive rows at one piece (the
// operand rows of K and Q) and 4 consecutive rows at two neighbouring pieces
// (the transposing reads).
__device__ __forceinline__ int row_swizzle(int t, int pieces) {
  return (((t & 3) << 1) | ((t >> 2) & 1) | (t & 8)) & (pieces - 1);
}

template <int DK, int SL>
struct StateLds {
  static constexpr int NC = kStateWaves * 16 * SL;  // columns per workgroup
  static constexpr int kK = 0;                       // K rows [C][DK] bf16
  static constexpr int kQ = kK + kC * DK * 2;        // Q rows [C][DK] bf16
  static constexpr int kV = kQ + kC * DK * 2;        // V rows [C][NC] bf16
  static constexpr int kF = kV + kC * NC * 2;        // record
  static constexpr int kBytes = kF + static_cast<int>(kTRecBytes);
  static constexpr int NK = kC * DK * 2 / 1024;      // 1 KiB global-to-LDS loads per chunk: K (and Q)
  static constexpr int NV = kC * NC * 2 / 1024;      // V
  static constexpr int NR = static_cast<int>(kTRecBytes / 1024);  // record
  static constexpr int NI = 2 * NK + NV + NR;
};

// One workgroup of four waves (one per SIMD) per (sequence, value head, block
// of 64 SL columns).  Wave w owns state columns 16 SL w .. +16 SL - 1 for all
// DK rows, as MFMA accumulators that never leave its registers.  Per chunk,
// with the chunk's K, Q, V and record in LDS:
//     U  = T'' V                       (V read transposed)
//     X  = T' (K S)   D = U - X        (K S packed to bf16 as the B operand)
//     O  = scale (diag(gam) (Q S) + M D)
//     S <- gam_last S + K^T diag(exp(G_last - G)) D   (K read transposed)
// Two stacked accumulator tiles, packed to bf16, are directly the B operand
// of the next product: the contraction index of every A operand (the K and Q
// rows, the record's blocks, K^T) is read in the matching permuted order.
// The next chunk's K, Q, V and record travel straight from memory into the
// second LDS buffer (global-to-LDS loads, no registers) while this chunk
// computes, so a chunk costs one barrier.  The ratio value heads of a q/k head
// and the column blocks of a head sit on one XCD and share K and Q in its L2.
// NORM (128-column blocks, d_v <= 128): the workgroup owns whole output rows
// and stores the gated RMSNorm of O instead of O.  Each wave sums the squares
// of its scaled Y per token with DPP over the 16 lanes of a row and writes
// them to a per-chunk LDS slot (double-buffered by chunk parity); after the
// chunk's barrier the row stores of the next chunk add the four waves'
// partials and apply the norm, with the gate rows loaded a chunk ahead.
// ONE (64-column blocks, no norm): one chunk buffer, and two workgroups per
// compute unit, so that one's loads and barriers overlap the other's products:
// each chunk starts with the output stores of the one before and a touch of
// the next chunk's lines (into L2), and ends with a barrier, the next chunk's
// loads and a second barrier.  The stores go first so that no output store is
// waited for with the loads, and their LDS reads wait for no load.
template <typename IO, int DK, int SL, bool NORM, bool ONE>
__global__ __launch_bounds__(64 * kStateWaves) __attribute__((amdgpu_waves_per_eu(ONE ? 2 : 1, ONE ? 2 : 1))) void
chunk_state_kernel(ScanParams p, const unsigned char* ws, const int32_t* cs) {
  static_assert(!NORM || SL == 2, "the fused norm needs 128-column blocks");
  static_assert(!ONE || (SL == 1 && !NORM), "one buffer: 64-column blocks without the norm");
  using L_ = StateLds<DK, SL>;
  constexpr int KB = DK / 32;   // key blocks of 32
  constexpr int RT = DK / 16;   // state row tiles
  constexpr int NC = L_::NC;
  constexpr int CPK = DK / 8;   // 16-byte pieces per K / Q row
  constexpr int CPV = NC / 8;   // 16-byte pieces per V row
  constexpr int kSO = 16 * SL;  // bf16 row stride of a wave's output block
  constexpr int ISS = (L_::NI + kStateWaves - 1) / kStateWaves;  // loads issued per wave and chunk
  // two chunk buffers, each region a distinct object, so that the compiler
  // keeps the loads into one buffer apart from the reads of the other (and
  // puts no wait for them before those reads)
  __shared__ __align__(16) bf16_t k0[kC * DK], k1[ONE ? 8 : kC * DK], q0[kC * DK], q1[ONE ? 8 : kC * DK];
  __shared__ __align__(16) bf16_t v0[kC * NC], v1[ONE ? 8 : kC * NC];
  __shared__ __align__(16) bf16x8 f0[kTRecBytes / 16], f1[ONE ? 1 : kTRecBytes / 16];
  struct Buf {
    bf16_t *k, *q, *v;
    bf16x8* f;
  };
  auto buf_of = [&](auto par) __attribute__((always_inline)) {
    if constexpr (ONE || decltype(par)::value == 0)
      return Buf{k0, q0, v0, f0};
    else
      return Buf{k1, q1, v1, f1};
  };
  __shared__ __align__(16) bf16_t out_blk[kStateWaves * kC * kSO];  // each wave's output block
  __shared__ float ss_blk[NORM ? 2 * kStateWaves * kC : 1];          // [chunk parity][wave][token] sums of squares
  static_assert((ONE ? 1 : 2) * L_::kBytes + sizeof(out_blk) + sizeof(ss_blk) <= (ONE ? 80 : 160) * 1024,
                "LDS budget of one gfx950 compute unit");
  static_assert(sizeof(k0) + sizeof(q0) + sizeof(v0) + sizeof(f0) == L_::kBytes, "buffer layout");

  const int tid = static_cast<int>(threadIdx.x);
  // wave-uniform, and the compiler is told so
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  bf16_t* Os = out_blk + w * kC * kSO;
  // blocks go round-robin over the 8 XCDs: the ratio value heads of a q/k head
  // and their column blocks are placed 8 apart, on one XCD
  const int xcd = static_cast<int>(blockIdx.x) % 8, r = static_cast<int>(blockIdx.x) / 8;
  const int per_group = p.ratio * p.col_blocks;
  const int group = (r / per_group) * 8 + xcd;  // (sequence, q/k head)
  if (group >= p.num_seqs * p.h_qk) return;     // the grid is padded to whole rounds of 8 groups
  const int unit = group * p.ratio + (r % per_group) / p.col_blocks;
  const int cb = r % p.col_blocks;
  const int h = unit % p.h_v;
  // the host's order of the sequences, where it gives one (a permutation)
  const int n = p.num_ordered == p.num_seqs ? static_cast<int>(p.seq_order[unit / p.h_v]) : unit / p.h_v;
  const int hq = h / p.ratio;
  const int d_v = p.d_v;
  const int T = p.total_tokens;
  const int t_begin = seq_lo(p.cu, n, T);
  const int t_end = seq_hi(p.cu, n, T);
  const int c_first = cs[n];
  const int nchunks = (t_end - t_begin + kC - 1) / kC;
  const int Jw = cb * NC + 16 * SL * w;  // first column of the wave
  bool has_state;
  const int sidx = state_slot(p.slots, p.num_slots, n, &has_state);
  const size_t sbase = (static_cast<size_t>(sidx) * p.h_v + h) * static_cast<size_t>(DK) * d_v;

  // ---- the wave's state slice: row tile ri, column tile sl
  f32x4 S[RT][SL];
#pragma unroll
  for (int ri = 0; ri < RT; ++ri)
#pragma unroll
    for (int sl = 0; sl < SL; ++sl) {
      const int col = Jw + 16 * sl + acc_col(lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * ri + acc_row(lane, i);
        S[ri][sl][i] = (p.s0 != nullptr && has_state && col < d_v) ? p.s0[sbase + static_cast<size_t>(row) * d_v + col] : 0.0f;
      }
    }

  const IO* kg = static_cast<const IO*>(p.k);
  const IO* qg = static_cast<const IO*>(p.q);
  const IO* vg = static_cast<const IO*>(p.v);
  IO* og = static_cast<IO*>(p.out);
  const size_t qk_stride = static_cast<size_t>(p.h_qk) * DK;
  const size_t v_stride = static_cast<size_t>(p.h_v) * d_v;
  // This wave's loads of a chunk, e = 0 .. ISS - 1, each 1 KiB with lane l
  // writing bytes 16 l .. +15: K pieces w + 4 e (e < EQ), Q pieces, V pieces,
  // then record pieces, so that the kind of load e is fixed at compile time.
  // The row in the chunk and the offset of each lane's 16 bytes are the same
  // for every chunk.  Rows past the sequence repeat its last row (their
  // contributions vanish: beta = 0 there); columns past d_v repeat the last 8
  // (their reads are zeroed below).
  constexpr int EQ = L_::NK / kStateWaves, EV = 2 * EQ, ER = EV + L_::NV / kStateWaves;
  static_assert(L_::NK % kStateWaves == 0 && L_::NV % kStateWaves == 0, "whole loads per wave");
  static_assert(ISS == ER + (L_::NR + kStateWaves - 1) / kStateWaves, "loads per wave");
  int ld_row[ISS], ld_off[ISS];
#pragma unroll
  for (int e = 0; e < ISS; ++e) {
    ld_row[e] = 0;
    if (e < EV) {
      const int s = 64 * (w + kStateWaves * (e < EQ ? e : e - EQ)) + lane;
      const int t = s / CPK, c = (s % CPK) ^ row_swizzle(t, CPK);
      ld_row[e] = t;
      ld_off[e] = hq * DK + 8 * c;  // elements
    } else if (e < ER) {
      const int s = 64 * (w + kStateWaves * (e - EV)) + lane;
      const int t = s / CPV, c = (s % CPV) ^ row_swizzle(t, CPV);
      ld_row[e] = t;
      ld_off[e] = h * d_v + min(cb * NC + 8 * c, d_v - 8);  // elements
    } else {
      ld_off[e] = (64 * (w + kStateWaves * (e - ER)) + lane) * 16;  // bytes of the record
    }
  }
  auto issue = [&](int j, const Buf& dst, int e) __attribute__((always_inline)) {
    const int c0 = t_begin + j * kC;
    const size_t row = static_cast<size_t>(c0 + min(ld_row[e], t_end - 1 - c0));
    if (e < EQ) {
      __builtin_amdgcn_global_load_lds(GDN_GLOBAL(kg + row * qk_stride + ld_off[e]),
                                       GDN_LDS(dst.k + 512 * (w + kStateWaves * e)), 16, 0, 0);
    } else if (e < EV) {
      __builtin_amdgcn_global_load_lds(GDN_GLOBAL(qg + row * qk_stride + ld_off[e]),
                                       GDN_LDS(dst.q + 512 * (w + kStateWaves * (e - EQ))), 16, 0, 0);
    } else if (e < ER) {
      __builtin_amdgcn_global_load_lds(GDN_GLOBAL(vg + row * v_stride + ld_off[e]),
                                       GDN_LDS(dst.v + 512 * (w + kStateWaves * (e - EV))), 16, 0, 0);
    } else {
      const int f = w + kStateWaves * (e - ER);
      const unsigned char* rec = ws + (static_cast<size_t>(c_first + j) * p.h_v + h) * kTRecBytes;
      if (e + 1 < ISS || f < L_::NR)
        __builtin_amdgcn_global_load_lds(GDN_GLOBAL(rec + ld_off[e]), GDN_LDS(dst.f + 64 * f), 16, 0, 0);
    }
  };
  auto issue_all = [&](int j, const Buf& dst) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < ISS; ++e) issue(j, dst, e);
  };
  // ONE: the chunk's loads are issued only after its predecessor is done, so
  // their latency would be paid in full every chunk.  Instead, at the start of
  // chunk j every workgroup touches its share of the 128-byte lines of chunk
  // j + kStateTouchAhead (one 4-byte load per line and thread): the K and Q
  // rows split over the per_group workgroups of the q/k head, the record over
  // the column blocks of the value head, the V rows its own (at most 256 lines:
  // any beyond are left to the loads).  The lines then come from L2 when the
  // chunk's loads are issued.  A touch's value is used at the next touch, long
  // after it has landed, so no early wait falls on it.
  constexpr int kLinesKQ = kC * DK * 2 / 128;  // K lines of a chunk (as many Q lines)
  constexpr int kLinesV = kC * NC * 2 / 128;
  constexpr int kLinesF = static_cast<int>(kTRecBytes / 128);
  const int member = r % per_group;
  const int n_kq = (2 * kLinesKQ - member + per_group - 1) / per_group;
  const int n_f = (kLinesF - cb + p.col_blocks - 1) / p.col_blocks;
  const int n_touch = n_kq + kLinesV + n_f;
  int tv = 0;
  auto touch_line = [&](int j, int x) __attribute__((always_inline)) {
    x = min(x, n_touch - 1);
    const int c0 = t_begin + j * kC;
    const int i = member + per_group * x;  // K then Q lines, when x < n_kq
    const int ikq = i < kLinesKQ ? i : i - kLinesKQ;
    const int xv = x - n_kq;              // V rows, then record lines
    const int xf = cb + p.col_blocks * (xv - kLinesV);
    const int row = x < n_kq ? ikq / (kLinesKQ / kC) : min(xv, kC - 1);
    const size_t trow = static_cast<size_t>(c0 + min(row, t_end - 1 - c0));
    const unsigned char* a =
        x < n_kq ? reinterpret_cast<const unsigned char*>((i < kLinesKQ ? kg : qg) + trow * qk_stride + hq * DK) +
                       128 * (ikq % (kLinesKQ / kC))
        : xv < kLinesV ? reinterpret_cast<const unsigned char*>(vg + trow * v_stride + h * d_v + min(cb * NC, d_v - 8))
                       : ws + (static_cast<size_t>(c_first + j) * p.h_v + h) * kTRecBytes + 128 * static_cast<size_t>(xf);
    return *reinterpret_cast<const int*>(a);
  };
  auto touch = [&](int j) __attribute__((always_inline)) {
    asm volatile("" ::"v"(tv));  // the previous touch's value, used
    tv = touch_line(min(j, nchunks - 1), tid);
    __builtin_amdgcn_sched_barrier(0);  // issued here, not sunk to the chunk's end
  };
  // A operand of rows 16 tt + (l % 16) of a K or Q buffer, keys 32 kb + 4 g .. +3
  // and 32 kb + 16 + 4 g .. +3 (g = l / 16)
  auto rows_frag = [&](const bf16_t* X, int tt, int kb) __attribute__((always_inline)) {
    const int t = 16 * tt + (lane & 15);
    const int sw = row_swizzle(t, CPK);
    const int c0 = 4 * kb + (g >> 1), half = 4 * (g & 1);
    const uint2 lo = *reinterpret_cast<const uint2*>(X + t * DK + 8 * (c0 ^ sw) + half);
    const uint2 hi = *reinterpret_cast<const uint2*>(X + t * DK + 8 * ((c0 + 2) ^ sw) + half);
    return __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
  };
  // operand over tokens, read transposed: lane l gets column col0 + l % 16 of
  // token rows 32 kb + 4 g .. +3 (elements 0-3) and 32 kb + 16 + 4 g .. +3
  auto tr_frag = [&](const bf16_t* X, int row_elems, int pieces, int col0, int kb) __attribute__((always_inline)) {
    const int i = lane & 15;
    const int col = col0 + 4 * (i & 3);
    const int c = col >> 3, half = col & 7;
    const int t0 = 32 * kb + 4 * g + (i >> 2);
    const s16x4 a = lds_read_tr(X + t0 * row_elems + 8 * (c ^ row_swizzle(t0, pieces)) + half);
    const s16x4 b = lds_read_tr(X + (t0 + 16) * row_elems + 8 * (c ^ row_swizzle(t0 + 16, pieces)) + half);
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    return __builtin_bit_cast(bf16x8, s16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]});
  };
  auto pack = [](f32x4 a, f32x4 b) __attribute__((always_inline)) {
    bf16x8 rr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rr[i] = static_cast<__bf16>(a[i]);
      rr[4 + i] = static_cast<__bf16>(b[i]);
    }
    return rr;
  };
  // swizzled output block: the 8-column piece pc of row t sits at piece pc ^ ((t / 4) % (2 SL))
  auto out_at = [](int t, int c) __attribute__((always_inline)) {
    return t * kSO + ((((c >> 3) ^ (t >> 2)) & (2 * SL - 1)) << 3) + (c & 7);
  };
  // the fused norm: this lane's 8-column piece of every row it stores is
  // columns Jw + 8 (lane % 4) .. +7; their scale once, and the gate rows of
  // the chunk in flight (loaded a chunk ahead, clamped into the sequence)
  const int nc8 = 8 * (lane & 3);
  const int ncol = Jw + nc8 < d_v ? Jw + nc8 : 0;
  RawSlice<IO, 8> n_scale;
  RawSlice<IO, 8> n_gate[4];
  if constexpr (NORM) n_scale.load(static_cast<const IO*>(p.norm.scale) + ncol);
  auto load_gate = [&](int j) __attribute__((always_inline)) {
    if constexpr (NORM) {
      const IO* gp = static_cast<const IO*>(p.norm.gate);
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int t = min(t_begin + j * kC + (lane >> 2) + 16 * it, t_end - 1);
        n_gate[it].load(gp + static_cast<size_t>(t) * v_stride + static_cast<size_t>(h) * d_v + ncol);
      }
    }
  };
  // the output block of chunk j (its scaled Y, kept in registers until no
  // global-to-LDS load is in flight) through the wave's LDS block, in 16-byte rows
  f32x4 Yp[4][SL];
  auto store_out = [&](int j) __attribute__((always_inline)) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int sl = 0; sl < SL; ++sl)
#pragma unroll
        for (int i = 0; i < 4; ++i) Os[out_at(16 * tt + acc_row(lane, i), 16 * sl + acc_col(lane))] = to_bf16(Yp[tt][sl][i]);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    const int c0 = t_begin + j * kC;
    const int Lc = min(kC, t_end - c0);
    constexpr int VPRO = 2 * SL;  // 8-column pieces per row
#pragma unroll
    for (int it = 0; it < kC * VPRO / 64; ++it) {
      const int v = lane + 64 * it;
      const int t = v / VPRO, c8 = (v % VPRO) * 8;
      if constexpr (NORM) {
        // y = o / sqrt(mean(o^2) + eps) scale act(gate) over the four waves' columns
        const float* ssj = ss_blk + (j & 1) * kStateWaves * kC;
        float ss = 0.0f;
#pragma unroll
        for (int ww = 0; ww < kStateWaves; ++ww) ss += ssj[ww * kC + t];
        const float inv = __builtin_amdgcn_rsqf(fmaf(ss, p.norm.inv_n, p.norm.eps));
        RawSlice<IO, 8> ro;
        const uint4 ow = *reinterpret_cast<const uint4*>(Os + out_at(t, c8));
        ro.w[0] = ow.x;
        ro.w[1] = ow.y;
        ro.w[2] = ow.z;
        ro.w[3] = ow.w;
        float o8[8], g8[8], s8[8], y8[8];
        ro.widen_to(o8);
        n_gate[it].widen_to(g8);
        n_scale.widen_to(s8);
#pragma unroll
        for (int e = 0; e < 8; ++e) y8[e] = gated_norm(o8[e], inv, s8[e], g8[e], p.norm.silu);
        if (t < Lc && Jw + c8 < d_v)
          store_slice<IO, 8>(og + static_cast<size_t>(c0 + t) * v_stride + static_cast<size_t>(h) * d_v + Jw + c8, y8);
      } else {
        if (t < Lc && Jw + c8 < d_v)
          *reinterpret_cast<uint4*>(og + static_cast<size_t>(c0 + t) * v_stride + static_cast<size_t>(h) * d_v + Jw + c8) =
              *reinterpret_cast<const uint4*>(Os + out_at(t, c8));
      }
    }
  };

  auto chunk = [&](int j, auto par) __attribute__((always_inline)) {
    const Buf cur = buf_of(par);
    const Buf nxt = buf_of(std::integral_constant<int, 1 - decltype(par)::value>{});
    // the next chunk's loads are spread over this chunk's products (a burst
    // would stall the wave on the memory pipeline while its MFMAs wait)
    const bool more = j + 1 < nchunks;
    if constexpr (ONE) touch(j + kStateTouchAhead);
    if (og != nullptr && j > 0) store_out(j - 1);
    if (og != nullptr) load_gate(j);
    const bf16_t* Kc = cur.k;
    const bf16_t* Qc = cur.q;
    const bf16_t* Vc = cur.v;
    const bf16x8* Fc = cur.f + lane;
    const float* tail = reinterpret_cast<const float*>(cur.f + kTRecTail / 16);

    // ================= a. U = T'' V, V over tokens as the B operand (columns past d_v read as 0)
    f32x4 U[4][SL];
    {
      bf16x8 VB[2][SL];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int sl = 0; sl < SL; ++sl) {
          VB[kb][sl] = tr_frag(Vc, NC, CPV, 16 * (SL * w + sl), kb);
          if (Jw + 16 * sl + (lane & 15) >= d_v) VB[kb][sl] = bf16x8{};
        }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
        for (int sl = 0; sl < SL; ++sl) U[tt][sl] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb <= tt / 2; ++kb) {
          const bf16x8 a = Fc[(6 + m_frag(tt, kb)) * 64];
#pragma unroll
          for (int sl = 0; sl < SL; ++sl) U[tt][sl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, VB[kb][sl], U[tt][sl], 0, 0, 0);
        }
      }
    }

    // ================= b. K S and Q S, the state (bf16) as the B operand from registers
    bf16x8 SB[KB][SL];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int sl = 0; sl < SL; ++sl) SB[kb][sl] = pack(S[2 * kb][sl], S[2 * kb + 1][sl]);
    // the next chunk's loads (the last chunk reloads itself into the idle
    // buffer) are spread over the 4 KB steps; the K and Q operands are read P
    // steps ahead
    const int jn = more ? j + 1 : j;
    constexpr int NSTEP = 4 * KB, P = 4;
    bf16x8 rk[P], rq[P];
#pragma unroll
    for (int q = 0; q < P; ++q) {
      rk[q] = rows_frag(Kc, q / KB, q % KB);
      rq[q] = rows_frag(Qc, q / KB, q % KB);
    }
    f32x4 X[4][SL], Y[4][SL];
#pragma unroll
    for (int step = 0; step < NSTEP; ++step) {
      const int tt = step / KB, kb = step % KB;
      if (kb == 0) {
#pragma unroll
        for (int sl = 0; sl < SL; ++sl) X[tt][sl] = Y[tt][sl] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
      if constexpr (!ONE) {
#pragma unroll
        for (int e = (step * ISS) / NSTEP; e < ((step + 1) * ISS) / NSTEP; ++e) issue(jn, nxt, e);
      }
      const bf16x8 ak = rk[step % P], aq = rq[step % P];
      if (step + P < NSTEP) {
        rk[step % P] = rows_frag(Kc, (step + P) / KB, (step + P) % KB);
        rq[step % P] = rows_frag(Qc, (step + P) / KB, (step + P) % KB);
      }
#pragma unroll
      for (int sl = 0; sl < SL; ++sl) {
        X[tt][sl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, SB[kb][sl], X[tt][sl], 0, 0, 0);
        Y[tt][sl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, SB[kb][sl], Y[tt][sl], 0, 0, 0);
      }
    }

    // ================= c. D = U - T' (K S), packed as the B operand over tokens, plain and scaled by exp(G_last - G)
    bf16x8 DB[2][SL], DW[2][SL];
    {
      bf16x8 XB[2][SL];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int sl = 0; sl < SL; ++sl) XB[kb][sl] = pack(X[2 * kb][sl], X[2 * kb + 1][sl]);
      f32x4 D[4][SL];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
        for (int sl = 0; sl < SL; ++sl) D[tt][sl] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb <= tt / 2; ++kb) {
          const bf16x8 a = Fc[m_frag(tt, kb) * 64];
#pragma unroll
          for (int sl = 0; sl < SL; ++sl) D[tt][sl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, XB[kb][sl], D[tt][sl], 0, 0, 0);
        }
#pragma unroll
        for (int sl = 0; sl < SL; ++sl) D[tt][sl] = U[tt][sl] - D[tt][sl];
      }
      f32x4 kf[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) kf[tt] = *reinterpret_cast<const f32x4*>(tail + 64 + 16 * tt + 4 * g);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int sl = 0; sl < SL; ++sl) {
          DB[kb][sl] = pack(D[2 * kb][sl], D[2 * kb + 1][sl]);
          DW[kb][sl] = pack(D[2 * kb][sl] * kf[2 * kb], D[2 * kb + 1][sl] * kf[2 * kb + 1]);
        }
    }

    // ================= d. O = scale (diag(gam) Q S + M D), stored at the start of the next chunk
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const f32x4 gm = *reinterpret_cast<const f32x4*>(tail + 16 * tt + 4 * g);
#pragma unroll
      for (int sl = 0; sl < SL; ++sl) Y[tt][sl] = Y[tt][sl] * gm;
#pragma unroll
      for (int kb = 0; kb <= tt / 2; ++kb) {
        const bf16x8 am = Fc[(12 + m_frag(tt, kb)) * 64];
#pragma unroll
        for (int sl = 0; sl < SL; ++sl) Y[tt][sl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, DB[kb][sl], Y[tt][sl], 0, 0, 0);
      }
    }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int sl = 0; sl < SL; ++sl) Yp[tt][sl] = p.scale * Y[tt][sl];
    if constexpr (NORM) {
      // per-token sums of squares over this wave's columns: lane l holds rows
      // 4 (l / 16) + i of column l % 16 in each tile; the 16 lanes of a row group add up
      float* ssw = ss_blk + ((j & 1) * kStateWaves + w) * kC;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float q = 0.0f;
#pragma unroll
          for (int sl = 0; sl < SL; ++sl) q = fmaf(Yp[tt][sl][i], Yp[tt][sl][i], q);
          q = group_sum<16>(q);
          if ((lane & 15) == 0) ssw[16 * tt + acc_row(lane, i)] = q;
        }
    }

    // ================= e. S <- gam_last S + K^T (exp(G_last - G) D), K over tokens as the A operand
    const float gl = tail[kC - 1];
#pragma unroll
    for (int ri = 0; ri < RT; ++ri) {
#pragma unroll
      for (int sl = 0; sl < SL; ++sl) S[ri][sl] = S[ri][sl] * gl;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 ak = tr_frag(Kc, DK, CPK, 16 * ri, kb);
#pragma unroll
        for (int sl = 0; sl < SL; ++sl) S[ri][sl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, DW[kb][sl], S[ri][sl], 0, 0, 0);
      }
    }
    if constexpr (ONE) {
      __syncthreads();  // every wave is done with this chunk's K, Q, V and record
      if (more) issue_all(j + 1, nxt);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's share of the next buffer has landed
    __syncthreads();                     // the next buffer is complete; this one may be refilled
  };

  if (nchunks > 0) issue_all(0, buf_of(std::integral_constant<int, 0>{}));
  // on every path, so that no load of the initial state is left in flight
  // into the chunk loop (a wait for it there would also wait for the touches)
  __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();
  if constexpr (ONE) {
    for (int j = 1; j < kStateTouchAhead && j < nchunks; ++j) touch(j);
  }
  for (int j = 0; j < nchunks; j += 2) {
    chunk(j, std::integral_constant<int, 0>{});
    if (j + 1 < nchunks) chunk(j + 1, std::integral_constant<int, 1>{});
  }
  if (og != nullptr && nchunks > 0) store_out(nchunks - 1);
  if constexpr (ONE) asm volatile("" ::"v"(tv));

  // ---- final state
  if (p.sN != nullptr && has_state) {
#pragma unroll
    for (int ri = 0; ri < RT; ++ri)
#pragma unroll
      for (int sl = 0; sl < SL; ++sl) {
        const int col = Jw + 16 * sl + acc_col(lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * ri + acc_row(lane, i);
          if (col < d_v) p.sN[sbase + static_cast<size_t>(row) * d_v + col] = S[ri][sl][i];
        }
      }
  }
}

// The state pass for few (sequence, head) units, at d_k = 128: one workgroup
// of four waves per (sequence, value head, 16-column tile), wave w owning
// state rows [32 w, 32 w + 32) of the tile as two accumulator tiles.  Where
// the column-block form above would leave most compute units idle (32 heads
// of one sequence fill 64 of them), this form puts a head's 16-column tiles on
// as many compute units, and each wave loads only the fragments of its own
// key block, straight into registers.  Per chunk, with two barriers:
//  1. every wave forms its partial W S over its rows -> LDS; after the first
//     barrier, its partial diag(gam) Q S -> LDS (double-buffered by chunk parity);
//  2. wave w sums the partials of token tile w: D = U - W S -> LDS;
//  3. after the second barrier every wave packs D and updates its rows,
//     S <- gam_last S + Kt^T D, and wave w writes the output of token tile w,
//     O = scale ((sum of the Q S partials) + M D).
constexpr int kRowWaves = 4;
constexpr int kRowTouchAhead = 3;  // chunks between a record's touch and its use

__global__ __launch_bounds__(64 * kRowWaves) void chunk_rows_kernel(ScanParams p, const unsigned char* ws,
                                                                   size_t rec_bytes, const int32_t* cs, int units8) {
  constexpr int DK = 128;
  constexpr int KB = DK / 32;
  constexpr int FQ = frags_w(DK), FK = 2 * frags_w(DK), FM = FK + 2 * (DK / 16), FT = FM + 6;
  __shared__ __align__(16) f32x4 xpart[2][kRowWaves][4][64];  // [buffer][wave][token tile][lane]
  __shared__ __align__(16) f32x4 ypart[2][kRowWaves][4][64];
  __shared__ __align__(16) f32x4 dt[4][64];                    // D per token tile

  const int unit = static_cast<int>(blockIdx.x) % units8;
  const int ct = static_cast<int>(blockIdx.x) / units8;
  if (unit >= p.num_seqs * p.h_v) return;  // the grid is padded to whole rounds of 8 units
  const int n = unit / p.h_v, h = unit % p.h_v;
  const int d_v = p.d_v;
  const int T = p.total_tokens;
  const int tid = static_cast<int>(threadIdx.x);
  // w is wave-uniform, and the compiler is told so: a branch on it must skip
  // its MFMAs, which run whatever the execution mask
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = 16 * ct + acc_col(lane);
  const bool col_ok = col < d_v;
  const Rec rec(DK);
  bf16_t* og = static_cast<bf16_t*>(p.out);
  const size_t v_stride = static_cast<size_t>(p.h_v) * d_v;

  bool has_state = true;
  const int sidx = state_slot(p.slots, p.num_slots, n, &has_state);
  const size_t sbase = (static_cast<size_t>(sidx) * p.h_v + h) * DK * d_v;
  f32x4 S[2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      S[r][i] = (p.s0 != nullptr && has_state && col_ok)
                    ? p.s0[sbase + static_cast<size_t>(32 * w + 16 * r + acc_row(lane, i)) * d_v + col]
                    : 0.0f;

  const int t_begin = seq_lo(p.cu, n, T), t_end = seq_hi(p.cu, n, T);
  const int nchunks = (t_end - t_begin + kC - 1) / kC;
  const int c_first = cs[n];
  // loads of a chunk past the last are clamped to the last
  auto record = [&](int j) __attribute__((always_inline)) {
    return ws + (static_cast<size_t>(c_first + min(j, nchunks - 1)) * p.h_v + h) * rec_bytes;
  };
  auto frag = [&](const unsigned char* rb, int f) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8*>(rb + rec.frag + (static_cast<size_t>(f) * 64 + lane) * 16);
  };
  auto pack = [](f32x4 a, f32x4 b) __attribute__((always_inline)) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[i] = static_cast<__bf16>(a[i]);
      r[4 + i] = static_cast<__bf16>(b[i]);
    }
    return r;
  };
  // W and diag(gam) Q of this wave's key block: the next chunk's are loaded
  // as soon as this chunk's products have read them; the operands used after
  // the second barrier (Kt^T, M, U, gam_last) at the top of their own chunk
  bf16x8 Wf[4], Qf[4];
  auto load_w = [&](int j) __attribute__((always_inline)) {
    const unsigned char* rb = record(j);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) Wf[tt] = frag(rb, tt * KB + w);
  };
  auto load_q = [&](int j) __attribute__((always_inline)) {
    const unsigned char* rb = record(j);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) Qf[tt] = frag(rb, FQ + tt * KB + w);
  };
  // The chunk's V rows over this column tile (64 x 16, 32-byte rows) pass
  // through LDS, double-buffered by chunk parity: every lane loads 16 bytes at
  // the top of the chunk before (waves 0 and 1 write them, before that chunk's
  // second barrier), and each wave reads its B operand of U = T'' V
  // transposed: lane l gets column l % 16 of tokens 32 kb + 4 g .. +3 and
  // 32 kb + 16 + 4 g .. +3 (g = l / 16), the permuted order of the record's
  // fragments.  Rows past the sequence repeat its last row (T'' is zero
  // there); columns past d_v repeat the last 8.
  __shared__ __align__(16) bf16_t vbuf[2][kC * 16];
  const int v_row = 32 * (w & 1) + (lane >> 1);
  const bf16_t* vg = static_cast<const bf16_t*>(p.v) + static_cast<size_t>(h) * d_v + min(16 * ct + 8 * (lane & 1), d_v - 8);
  u32x4 vrow;
  auto load_v = [&](int j) __attribute__((always_inline)) {
    const int c0 = t_begin + kC * min(j, nchunks - 1);
    vrow = *reinterpret_cast<const u32x4*>(vg + static_cast<size_t>(min(c0 + v_row, t_end - 1)) * v_stride);
  };
  auto store_v = [&](int j) __attribute__((always_inline)) {
    if (w < 2) *reinterpret_cast<u32x4*>(vbuf[j & 1] + v_row * 16 + 8 * (lane & 1)) = vrow;
  };
  auto v_operand = [&](int j, int kb) __attribute__((always_inline)) {
    const bf16_t* vb = vbuf[j & 1] + (32 * kb + 4 * (lane >> 4) + ((lane & 15) >> 2)) * 16 + 4 * (lane & 3);
    const s16x4 a = lds_read_tr(vb);
    const s16x4 b = lds_read_tr(vb + 16 * 16);
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    return __builtin_bit_cast(bf16x8, s16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]});
  };
  // U of token tile w and this column tile, T'' (its lower blocks, loaded with
  // the chunk's other operands a chunk ahead; the second block is loaded by
  // every wave, used by waves 2 and 3) times the V rows: formed at the end of
  // the chunk before, off the chain from S to the next S
  bf16x8 TA[2];
  f32x4 Uw;
  auto load_t = [&](int j) __attribute__((always_inline)) {
    const unsigned char* rb = record(j);
    TA[0] = frag(rb, FT + m_frag(w, 0));
    TA[1] = frag(rb, FT + m_frag(w, 1));
  };
  auto form_u = [&](int j) __attribute__((always_inline)) {
    Uw = __builtin_amdgcn_mfma_f32_16x16x32_bf16(TA[0], v_operand(j, 0), (f32x4{0.0f, 0.0f, 0.0f, 0.0f}), 0, 0, 0);
    if (w >= 2) Uw = __builtin_amdgcn_mfma_f32_16x16x32_bf16(TA[1], v_operand(j, 1), Uw, 0, 0, 0);
  };
  // The column tiles of a unit share each chunk's record through one L2 (they
  // sit units8 blocks apart: on one XCD).  Each tile touches its share of the
  // record kRowTouchAhead chunks ahead, one 4-byte load per 128-byte line, so
  // the record comes in from HBM while earlier chunks compute; the touch is
  // issued after the chunk's other loads and its value consumed a chunk
  // later, so no wait falls on it early (loads complete in issue order).
  const int ntiles = (d_v + 15) / 16;
  const int lines = static_cast<int>(rec_bytes / 128);
  const int per_tile = (lines + ntiles - 1) / ntiles;
  // Threads past the tile's record lines touch the tile's V rows of the same
  // chunk (the line that holds its 16 columns of each row), which nothing
  // else brings in ahead of the gathers of load_v.
  const bool touching = per_tile + kC <= 64 * kRowWaves;
  int touched = 0, tv = 0;
  auto touch = [&](int j) __attribute__((always_inline)) {
    touched += tv;
    const int line = min(ct * per_tile + tid, lines - 1);
    const int vrow = min(t_begin + kC * min(j, nchunks - 1) + (tid - per_tile), t_end - 1);
    const unsigned char* a =
        tid < per_tile ? record(j) + static_cast<size_t>(line) * 128
                       : reinterpret_cast<const unsigned char*>(static_cast<const bf16_t*>(p.v) + static_cast<size_t>(vrow) * v_stride +
                                                                static_cast<size_t>(h) * d_v + 16 * ct);
    tv = *reinterpret_cast<const int*>(a);
  };

  auto chunk = [&](int j) __attribute__((always_inline)) {
    const int t0 = t_begin + kC * j;
    const int Lc = min(kC, t_end - t0);
    const unsigned char* rb = record(j);
    const int buf = j & 1;
    load_v(j + 1);  // first: its wait, before the second barrier, then covers no later load

    bf16x8 KtA[2][2];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) KtA[r][kb] = frag(rb, FK + 2 * (2 * w + r) + kb);
    // the second block of M is used by waves 2 and 3 only, but loaded by all
    // (m_frag(w, 1) is block w itself for w < 2): a load chosen by a branch
    // would be waited for, with every load before it, where it joins
    bf16x8 MA[2];
    MA[0] = frag(rb, FM + m_frag(w, 0));
    MA[1] = frag(rb, FM + m_frag(w, 1));
    const float gam_last = *reinterpret_cast<const float*>(rb + rec.g);

    // ---- 1. partials over this wave's rows (U of token tile w folded into
    //      wave w's W S partial of that tile: the partials sum to -D)
    const bf16x8 SB = pack(S[0], S[1]);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const f32x4 x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Wf[tt], SB, (f32x4{0.0f, 0.0f, 0.0f, 0.0f}), 0, 0, 0);
      xpart[buf][w][tt][lane] = tt == w ? x - Uw : x;
    }
    load_w(j + 1);
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
      ypart[buf][w][tt][lane] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Qf[tt], SB, (f32x4{0.0f, 0.0f, 0.0f, 0.0f}), 0, 0, 0);
    load_q(j + 1);
    load_t(j + 1);
    if (touching) touch(j + kRowTouchAhead);

    // ---- 2. D of token tile w
    {
      f32x4 x = xpart[buf][0][w][lane];
#pragma unroll
      for (int ww = 1; ww < kRowWaves; ++ww) x += xpart[buf][ww][w][lane];
      dt[w][lane] = -x;
    }
    store_v(j + 1);
    __syncthreads();

    // ---- 3. D as the B operand over tokens; the output of tile w; the state update
    bf16x8 DB[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) DB[kb] = pack(dt[2 * kb][lane], dt[2 * kb + 1][lane]);
    if (og != nullptr) {
      f32x4 y = ypart[buf][0][w][lane];
#pragma unroll
      for (int ww = 1; ww < kRowWaves; ++ww) y += ypart[buf][ww][w][lane];
      y = __builtin_amdgcn_mfma_f32_16x16x32_bf16(MA[0], DB[0], y, 0, 0, 0);
      if (w >= 2) y = __builtin_amdgcn_mfma_f32_16x16x32_bf16(MA[1], DB[1], y, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * w + acc_row(lane, i);
        if (t < Lc && col_ok)
          og[static_cast<size_t>(t0 + t) * v_stride + static_cast<size_t>(h) * d_v + col] = to_bf16(p.scale * y[i]);
      }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      f32x4 sacc = S[r] * gam_last;
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(KtA[r][0], DB[0], sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(KtA[r][1], DB[1], sacc, 0, 0, 0);
      S[r] = sacc;
    }
    form_u(j + 1);  // the next chunk's V rows are in LDS since the second barrier
  };

  if (nchunks > 0) {
    load_w(0);
    load_q(0);
    load_t(0);
    load_v(0);
    store_v(0);
    __syncthreads();
    form_u(0);
    for (int j = 0; j < nchunks; ++j) chunk(j);
  }

  // keeps the touches alive (never true: the host rejects negative token counts)
  if (p.total_tokens < 0 && touched + tv == 1) og[0] = 0;
  if (p.sN != nullptr && has_state && col_ok) {
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        p.sN[sbase + static_cast<size_t>(32 * w + 16 * r + acc_row(lane, i)) * d_v + col] = S[r][i];
  }
}

template <typename K>
hipError_t set_lds(K kern, int bytes) {
  return ensure_dynamic_lds(reinterpret_cast<const void*>(kern), bytes);
}


// Persistent grid of the preparation pass: one workgroup per compute unit.
int prep_workgroups() { return device_compute_units(); }

// Columns per state-pass workgroup: 128 (two per wave), or 64 while the
// 64-column workgroups take at most two rounds of the compute units (one per
// unit): the smaller blocks fill units left idle, and in a second round they
// take the places freed by short sequences (the 8-sequence packed workload:
// 1.07 against 1.10 ms).
// The row-split state pass (16-column tiles) at d_k = 128 while its
// workgroups take at most one round of the compute units: 32 heads of one
// 4096-token sequence 0.196 against 0.244 ms, 8 heads 0.124 against 0.173 ms;
// at two rounds (2 sequences x 32 heads) the column blocks are faster
// (0.52 against 0.60 ms).
bool split_rows(int d_k, int d_v, int units) {
  return d_k == 128 && static_cast<int64_t>(units) * ((d_v + 15) / 16) <= device_compute_units();
}

int split_columns(int d_v, int units) {
  return d_v > 64 && static_cast<int64_t>(units) * ((d_v + 63) / 64) > 2 * static_cast<int64_t>(prep_workgroups()) ? 128 : 64;
}


template <typename IO, int DK>
hipError_t launch_prep(const ScanParams& p, unsigned char* ws, size_t rec_bytes, const int32_t* cs, const int2* info,
                       int items, int nt, hipStream_t stream) {
  constexpr int bytes = PrepLds<DK>::kBytes;
  const unsigned grid = static_cast<unsigned>(items < prep_workgroups() ? items : prep_workgroups());
  if (p.gates.raw) {
    auto kern = chunk_prep_kernel<IO, DK, true>;
    hipError_t e = set_lds(kern, bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), bytes, stream, p, ws, rec_bytes, cs, info, items, nt);
  } else {
    auto kern = chunk_prep_kernel<IO, DK, false>;
    hipError_t e = set_lds(kern, bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), bytes, stream, p, ws, rec_bytes, cs, info, items, nt);
  }
  return hipGetLastError();
}

// The small-record preparation pass: two workgroups per compute unit.
template <typename IO, int DK>
hipError_t launch_trec(const ScanParams& p, unsigned char* ws, const int32_t* cs, const int2* info, int items,
                       hipStream_t stream) {
  // value heads of one q/k head in pairs where the ratio is even
  const bool pairs = p.ratio % 2 == 0;
  const int units = pairs ? items / 2 : items;
  const int slots = 2 * prep_workgroups();
  const unsigned grid = static_cast<unsigned>(units < slots ? units : slots);
  auto launch = [&](auto kern, int bytes) {
    hipError_t e = set_lds(kern, bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kTThreads), bytes, stream, p, ws, cs, info, units);
    return hipGetLastError();
  };
  auto by_rule = [&](auto raw, auto nh) {
    constexpr bool R = decltype(raw)::value;
    constexpr int N = decltype(nh)::value;
    return p.gates.deltas ? launch(chunk_trec_kernel<IO, DK, R, N, false>, TPrepLds<DK, N>::kBytes)
                          : launch(chunk_trec_kernel<IO, DK, R, N, true>, TPrepLds<DK, N>::kBytes);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  if (pairs)
    return p.gates.raw ? by_rule(T_{}, std::integral_constant<int, 2>{}) : by_rule(F_{}, std::integral_constant<int, 2>{});
  return p.gates.raw ? by_rule(T_{}, std::integral_constant<int, 1>{}) : by_rule(F_{}, std::integral_constant<int, 1>{});
}

// The row-split state pass reads the full record (W, diag(gam) Q, Kt^T, M,
// T'') and V; the column-block pass reads K, Q and V itself and the T', T'', M
// record.
template <typename IO, int DK>
hipError_t launch_split_passes(const ScanParams& p, unsigned char* ws, size_t rec_bytes, int32_t* cs, const int2* info,
                      int chunk_bound, hipStream_t stream) {
  const int units = p.num_seqs * p.h_v;
  // the row-split pair forms its record for the delta rules only
  const bool rows = DK == 128 && p.gates.deltas && split_rows(p.d_k, p.d_v, units);
  if (chunk_bound > 0 && p.h_v > 0) {
    const int items = chunk_bound * p.h_v;
    // Nontemporal record stores ahead of the column-block state pass (the
    // 8-sequence packed workload 1.07-1.08 against 1.09-1.10 ms); ahead of
    // the row-split pass they cost about 1 % (one 4096-token sequence).
    const hipError_t e = rows ? launch_prep<IO, DK>(p, ws, rec_bytes, cs, info, items, 0, stream)
                              : launch_trec<IO, DK>(p, ws, cs, info, items, stream);
    if (e != hipSuccess) return e;
  }
  if (units == 0) return hipSuccess;
  if constexpr (DK == 128) {
    if (rows) {
      const int units8 = (units + 7) / 8 * 8;
      const unsigned rblocks = static_cast<unsigned>(units8) * static_cast<unsigned>((p.d_v + 15) / 16);
      hipLaunchKernelGGL(chunk_rows_kernel, dim3(rblocks), dim3(64 * kRowWaves), 0, stream, p, ws, rec_bytes, cs, units8);
      return hipGetLastError();
    }
  }
  const unsigned groups8 = static_cast<unsigned>((p.num_seqs * p.h_qk + 7) / 8 * 8);
  const unsigned blocks = groups8 * static_cast<unsigned>(p.ratio) * static_cast<unsigned>(p.col_blocks);
  if (p.norm.gate != nullptr && split_fuses_norm(p.d_v, units))
    hipLaunchKernelGGL((chunk_state_kernel<IO, DK, 2, true, false>), dim3(blocks), dim3(64 * kStateWaves), 0, stream, p, ws, cs);
  else if (split_columns(p.d_v, units) == 128)
    hipLaunchKernelGGL((chunk_state_kernel<IO, DK, 2, false, false>), dim3(blocks), dim3(64 * kStateWaves), 0, stream, p, ws, cs);
  else
    hipLaunchKernelGGL((chunk_state_kernel<IO, DK, 1, false, true>), dim3(blocks), dim3(64 * kStateWaves), 0, stream, p, ws, cs);
  return hipGetLastError();
}

// Bytes of one (chunk, value head) record for the state pass that runs.
size_t record_bytes(int d_k, int d_v, int units, bool deltas) {
  if (deltas && split_rows(d_k, d_v, units)) return Rec(d_k).bytes;
  return kTRecBytes;
}

int chunk_bound_of(int num_seqs, int total_tokens) {
  return num_seqs > 0 ? (total_tokens + kC - 1) / kC + num_seqs : 0;
}

}  // namespace

// Any of the four rules: without the delta correction the small-record
// preparation writes T'' = I and T' = 0 (the column-block state pass then
// takes D = V), so those rules run the column-block pair whatever the units.
bool split_supported(int io_bf16, int d_k, int d_v, const GateArgs& gates, int window) {
  return io_bf16 && (d_k == 64 || d_k == 128) && d_v % 8 == 0 && d_v <= 256 && !gates.per_key && window == 0;
}

int split_columns_per_block(int d_v, int units) { return split_columns(d_v, units); }

bool split_takes_rows_kernel(int d_k, int d_v, int units, bool deltas) { return deltas && split_rows(d_k, d_v, units); }

// The fused norm needs 128-column blocks; it is taken where the column rule
// picks them anyway.  There it beats the separate norm pass (16 x 2048 tokens:
// 1.093 against 1.125 ms; 32 x 1024: 1.083 against 1.094 ms); where 64-column
// blocks or the row-split pass would run, forcing 128-column blocks costs more
// than the pass saves (8 packed sequences: 1.26 against 1.18 ms; one
// 4096-token sequence: 0.41 against 0.20 ms).
bool split_fuses_norm(int d_v, int units) { return d_v <= 128 && split_columns(d_v, units) == 128; }

// Workspace: cs [N + 1] int32, info [chunk bound] int2, then the records.
static size_t table_bytes(int num_seqs, int total_tokens) {
  return align256(static_cast<size_t>(num_seqs + 1) * 4) + align256(static_cast<size_t>(chunk_bound_of(num_seqs, total_tokens)) * 8);
}

int chunk_table_bound(int num_seqs, int total_tokens) { return chunk_bound_of(num_seqs, total_tokens); }
size_t chunk_table_bytes(int num_seqs, int total_tokens) { return num_seqs > 0 ? table_bytes(num_seqs, total_tokens) : 0; }

hipError_t launch_chunk_table(const int32_t* cu, int num_seqs, int total_tokens, void* workspace, hipStream_t stream) {
  int32_t* cs = static_cast<int32_t*>(workspace);
  int2* info = reinterpret_cast<int2*>(static_cast<unsigned char*>(workspace) +
                                       align256(static_cast<size_t>(num_seqs + 1) * 4));
  hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(1024), 0, stream, cu, num_seqs, total_tokens, cs, info);
  return hipGetLastError();
}

size_t split_workspace_bytes(int num_seqs, int total_tokens, int h_v, int d_k, int d_v, bool deltas) {
  if (num_seqs <= 0) return 0;
  return table_bytes(num_seqs, total_tokens) + static_cast<size_t>(chunk_bound_of(num_seqs, total_tokens)) * h_v *
                                                   record_bytes(d_k, d_v, num_seqs * h_v, deltas);
}

hipError_t launch_prefill_split(ScanParams p, void* workspace, hipStream_t stream) {
  if (p.num_seqs <= 0) return hipSuccess;
  const size_t rec_bytes = record_bytes(p.d_k, p.d_v, p.num_seqs * p.h_v, p.gates.deltas != 0);
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
    return launch_split_passes<bf16_t, 128>(p, recs, rec_bytes, cs, info, bound, stream);
  return launch_split_passes<bf16_t, 64>(p, recs, rec_bytes, cs, info, bound, stream);
}

}  // namespace gdn
