// gated_rmsnorm.hip -- gated RMSNorm (gfx950), the operation after the gated
// delta-rule recurrence in its block.
//
// Definition ([P1] onnxruntime-ep-mlx, src/ops/ssm.rs, `gated_rms_norm_op`):
// each row is split into groups of `group` consecutive elements; per group,
// in float32,
//     y = x / sqrt(mean(x^2) + eps) * scale * act(gate)
// with act = silu (gate * sigmoid(gate)) or sigmoid, narrowed once to the
// I/O dtype.
//
// HBM-bound (x and gate read once, y written once).  A team of TL lanes
// (a power of two up to 64) owns one group; lane l of a team holds vectors
// l, l + TL, ... (NV of them, 16 bytes each when the group is a multiple of
// 16 bytes, single elements otherwise), so a team reads TL * 16 contiguous
// bytes per step.  The sum of squares is reduced across the team with DPP
// row operations.  Waves walk the groups grid-stride.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxNV = 8;

// U groups per team per iteration (U * NV vectors of x and of the gate in
// flight per lane).
template <typename IO, int V, int TL, int NV, bool SILU, int U = (NV >= 4 ? 1 : 4 / NV)>
__global__ __launch_bounds__(kThreads) void rmsnorm_kernel(NormParams p) {
  const int lane = static_cast<int>(threadIdx.x) % 64;
  const int wave = static_cast<int>(threadIdx.x) / 64;
  const int tl = lane % TL;
  constexpr int kTeams = 64 / TL;
  const int team = lane / TL;
  const int nvec = p.group / V;
  const IO* __restrict__ xg = static_cast<const IO*>(p.x);
  const IO* __restrict__ gg = static_cast<const IO*>(p.gate);
  const IO* __restrict__ sg = static_cast<const IO*>(p.scale);
  IO* __restrict__ yg = static_cast<IO*>(p.y);
  const float inv_n = 1.0f / static_cast<float>(p.group);

  // a wave takes U * kTeams consecutive groups per iteration (team u * kTeams +
  // team), so each load instruction covers kTeams consecutive groups; every
  // lane runs the same number of iterations (the DPP reduction needs the whole
  // wave), and a team past the end repeats the last group
  const int64_t per_wave = static_cast<int64_t>(U) * kTeams;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * (kThreads / 64) * per_wave;
  const int64_t first = (static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + wave) * per_wave;
  for (int64_t base = first; base < p.groups; base += stride) {
    // Loads are unconditional, from clamped (existing) groups and vectors:
    // under a condition, the compiler could no longer count the loads issued
    // after a given one and would wait for every memory operation, stores
    // included, before each use.  Vectors past the group read as zero below.
    // This lane's scale elements (the same for every group) are loaded first
    // in every iteration: most waves run one iteration, and a load before the
    // loop would cost them a second full memory latency.  They come from
    // cache after the first; the empty asm keeps the load in the loop.
    int opaque_zero = 0;
    asm volatile("" : "+s"(opaque_zero));
    const IO* sgi = sg + opaque_zero;
    RawSlice<IO, V> rs[NV], rx[U][NV], rg[U][NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) rs[k].load(sgi + static_cast<size_t>(min(k * TL + tl, nvec - 1)) * V);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t grp = base + u * kTeams + team;
      const size_t off = static_cast<size_t>(grp < p.groups ? grp : p.groups - 1) * p.group;
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int vi = min(k * TL + tl, nvec - 1);
        rx[u][k].load(xg + off + static_cast<size_t>(vi) * V);
        rg[u][k].load(gg + off + static_cast<size_t>(vi) * V);
      }
    }
    // every load of the iteration is issued before the first use waits
    __builtin_amdgcn_sched_barrier(0);
    float sc[NV][V];
#pragma unroll
    for (int k = 0; k < NV; ++k) rs[k].widen_to(sc[k]);
    // Stores are unconditional too (a load used only under a condition is
    // sunk into it and waited for there): a lane past the end computes and
    // stores the clamped vector it loaded, with that group's norm, which
    // repeats its owner's store bit for bit.
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t grp = base + u * kTeams + team;
      const size_t off = static_cast<size_t>(grp < p.groups ? grp : p.groups - 1) * p.group;
      float xv[NV][V];
      float ss = 0.0f;
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        rx[u][k].widen_to(xv[k]);
        float part = 0.0f;
#pragma unroll
        for (int e = 0; e < V; ++e) part = fmaf(xv[k][e], xv[k][e], part);
        ss += k * TL + tl < nvec ? part : 0.0f;
      }
      ss = group_sum<TL>(ss);
      // v_rsq_f32 (about 1 ulp); the argument is at least eps
      const float inv = __builtin_amdgcn_rsqf(fmaf(ss, inv_n, p.eps));
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int vi = min(k * TL + tl, nvec - 1);
        float gv[V], out[V];
        rg[u][k].widen_to(gv);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const float s = fast_sigmoid(gv[e]);
          const float act = SILU ? gv[e] * s : s;
          out[e] = xv[k][e] * inv * sc[k][e] * act;
        }
        IO* yo = yg + off + static_cast<size_t>(vi) * V;
        if constexpr (V * sizeof(IO) == 16) {
          store_slice<IO, V>(yo, out);
        } else {
#pragma unroll
          for (int e = 0; e < V; ++e) narrow_store(yo + e, out[e]);
        }
      }
    }
  }
}

// Team size and vectors per lane for a group of nvec vectors.
void shape_for(int nvec, int* tl, int* nv) {
  int t = 1;
  while (t < nvec && t < 64) t *= 2;
  int v = 1;
  while (v * t < nvec) v *= 2;
  *tl = t;
  *nv = v;
}

template <typename IO, int V, int TL, bool SILU>
hipError_t launch_act(const NormParams& p, int nv, unsigned grid, hipStream_t stream) {
  switch (nv) {
    case 1: hipLaunchKernelGGL((rmsnorm_kernel<IO, V, TL, 1, SILU>), dim3(grid), dim3(kThreads), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((rmsnorm_kernel<IO, V, TL, 2, SILU>), dim3(grid), dim3(kThreads), 0, stream, p); break;
    case 4: hipLaunchKernelGGL((rmsnorm_kernel<IO, V, TL, 4, SILU>), dim3(grid), dim3(kThreads), 0, stream, p); break;
    default: hipLaunchKernelGGL((rmsnorm_kernel<IO, V, TL, kMaxNV, SILU>), dim3(grid), dim3(kThreads), 0, stream, p); break;
  }
  return hipGetLastError();
}

template <typename IO, int V, int TL>
hipError_t launch_tl(const NormParams& p, int nv, unsigned grid, hipStream_t stream) {
  return p.activation == 1 ? launch_act<IO, V, TL, true>(p, nv, grid, stream)
                           : launch_act<IO, V, TL, false>(p, nv, grid, stream);
}

template <typename IO, int V>
hipError_t launch_v(const NormParams& p, hipStream_t stream) {
  int tl, nv;
  shape_for(p.group / V, &tl, &nv);
  const int u = nv >= 4 ? 1 : 4 / nv;
  const int64_t teams_per_block = (kThreads / 64) * (64 / tl) * u;
  const int64_t want = (p.groups + teams_per_block - 1) / teams_per_block;
  const unsigned grid = static_cast<unsigned>(want < 16384 ? want : 16384);
  switch (tl) {
    case 1: return launch_tl<IO, V, 1>(p, nv, grid, stream);
    case 2: return launch_tl<IO, V, 2>(p, nv, grid, stream);
    case 4: return launch_tl<IO, V, 4>(p, nv, grid, stream);
    case 8: return launch_tl<IO, V, 8>(p, nv, grid, stream);
    case 16: return launch_tl<IO, V, 16>(p, nv, grid, stream);
    case 32: return launch_tl<IO, V, 32>(p, nv, grid, stream);
    default: return launch_tl<IO, V, 64>(p, nv, grid, stream);
  }
}

template <typename IO>
hipError_t launch_io(const NormParams& p, hipStream_t stream) {
  constexpr int V = 16 / static_cast<int>(sizeof(IO));
  if (p.groups == 0) return hipSuccess;
  if (p.group % V == 0) return launch_v<IO, V>(p, stream);
  return launch_v<IO, 1>(p, stream);
}

}  // namespace

bool gated_rmsnorm_supported(int io_dtype, int group) {
  const int v = io_dtype == 0 ? 4 : 8;
  const int nvec = group % v == 0 ? group / v : group;
  return group >= 1 && nvec <= 64 * kMaxNV;
}

hipError_t launch_gated_rmsnorm(NormParams p, int io_dtype, hipStream_t stream) {
  if (io_dtype == 1) return launch_io<bf16_t>(p, stream);
  if (io_dtype == 2) return launch_io<f16_t>(p, stream);
  return launch_io<float>(p, stream);
}

}  // namespace gdn
