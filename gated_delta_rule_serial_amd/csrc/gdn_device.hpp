// gdn_device.hpp -- device helpers shared by the libgdn kernels (gfx950).
//
// I/O element types, widening loads of short row slices, 64-lane wavefront
// reductions built from DPP row operations, and the gate prologue math.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

using bf16_t = uint16_t;  // bfloat16 storage
using f16_t = _Float16;   // IEEE binary16 storage

// ---------------------------------------------------------------- scalars
__device__ __forceinline__ float widen(float x) { return x; }
__device__ __forceinline__ float widen(bf16_t x) { return __uint_as_float(static_cast<uint32_t>(x) << 16); }
__device__ __forceinline__ float widen(f16_t x) { return static_cast<float>(x); }

// Widen the 16-bit pattern in the low half of `bits` as an element of IO.
template <typename IO>
__device__ __forceinline__ float widen_bits16(uint32_t bits) {
  if constexpr (__is_same(IO, f16_t)) return static_cast<float>(__builtin_bit_cast(f16_t, static_cast<uint16_t>(bits)));
  else return __uint_as_float(bits << 16);
}

// Narrowing rounds to nearest even (gfx950 v_cvt_pk_bf16_f32, v_cvt_f16_f32
// in the default rounding mode).
__device__ __forceinline__ void narrow_store(float* p, float x) { *p = x; }
__device__ __forceinline__ void narrow_store(bf16_t* p, float x) {
  *p = __builtin_bit_cast(bf16_t, static_cast<__bf16>(x));
}
__device__ __forceinline__ void narrow_store(f16_t* p, float x) { *p = static_cast<f16_t>(x); }

template <typename IO>
__device__ __forceinline__ float load1(const IO* p) { return widen(*p); }

// Two floats narrowed (round to nearest even) into one 32-bit word, the first
// in the low half.
template <typename IO>
__device__ __forceinline__ uint32_t narrow_pair(float a, float b) {
  if constexpr (__is_same(IO, f16_t)) {
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<f16_t>(a))) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<f16_t>(b))) << 16);
  } else {
    // one v_cvt_pk_bf16_f32 for the pair
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const f32x2 ab = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(ab, bf16x2));
  }
}

// Narrow N floats and store them with 16-byte stores; p is 16-byte aligned
// and N * sizeof(IO) a multiple of 16.
template <typename IO, int N>
__device__ __forceinline__ void store_slice(IO* p, const float* v) {
  static_assert((N * static_cast<int>(sizeof(IO))) % 16 == 0, "whole 16-byte stores only");
  if constexpr (sizeof(IO) == 4) {
#pragma unroll
    for (int c = 0; c < N / 4; ++c)
      reinterpret_cast<float4*>(p)[c] = make_float4(v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]);
  } else {
#pragma unroll
    for (int c = 0; c < N / 8; ++c) {
      uint4 w;
      w.x = narrow_pair<IO>(v[8 * c + 0], v[8 * c + 1]);
      w.y = narrow_pair<IO>(v[8 * c + 2], v[8 * c + 3]);
      w.z = narrow_pair<IO>(v[8 * c + 4], v[8 * c + 5]);
      w.w = narrow_pair<IO>(v[8 * c + 6], v[8 * c + 7]);
      reinterpret_cast<uint4*>(p)[c] = w;
    }
  }
}

// ---------------------------------------------------------------- row slices
// Load N consecutive I/O elements starting at p (aligned to N elements) and
// widen them to float.  N is a power of two, 1 .. 16.
template <int N>
__device__ __forceinline__ void load_slice(const float* p, float* dst) {
  if constexpr (N >= 4) {
#pragma unroll
    for (int c = 0; c < N / 4; ++c) {
      const float4 x = reinterpret_cast<const float4*>(p)[c];
      dst[4 * c + 0] = x.x;
      dst[4 * c + 1] = x.y;
      dst[4 * c + 2] = x.z;
      dst[4 * c + 3] = x.w;
    }
  } else if constexpr (N == 2) {
    const float2 x = *reinterpret_cast<const float2*>(p);
    dst[0] = x.x;
    dst[1] = x.y;
  } else {
    dst[0] = *p;
  }
}

__device__ __forceinline__ void unpack2(uint32_t w, float* dst) {
  dst[0] = __uint_as_float(w << 16);
  dst[1] = __uint_as_float(w & 0xffff0000u);
}

template <int N>
__device__ __forceinline__ void load_slice(const bf16_t* p, float* dst) {
  if constexpr (N >= 8) {
#pragma unroll
    for (int c = 0; c < N / 8; ++c) {
      const uint4 x = reinterpret_cast<const uint4*>(p)[c];
      unpack2(x.x, dst + 8 * c + 0);
      unpack2(x.y, dst + 8 * c + 2);
      unpack2(x.z, dst + 8 * c + 4);
      unpack2(x.w, dst + 8 * c + 6);
    }
  } else if constexpr (N == 4) {
    const uint2 x = *reinterpret_cast<const uint2*>(p);
    unpack2(x.x, dst + 0);
    unpack2(x.y, dst + 2);
  } else if constexpr (N == 2) {
    unpack2(*reinterpret_cast<const uint32_t*>(p), dst);
  } else {
    dst[0] = widen(*p);
  }
}

// Bounds-checked variant: element e is read only when e < limit (else 0).
template <int N, typename IO>
__device__ __forceinline__ void load_slice_masked(const IO* p, int limit, float* dst) {
#pragma unroll
  for (int e = 0; e < N; ++e) dst[e] = (e < limit) ? widen(p[e]) : 0.0f;
}

// A row slice of N I/O elements held in its packed (loaded, not yet widened)
// form.  Keeping the packed words lets a load be issued many steps before its
// value is consumed: the wait for the data lands at widen(), not at load().
template <typename IO, int N>
struct RawSlice {
  static constexpr int kBytes = N * static_cast<int>(sizeof(IO));
  static constexpr int kWords = kBytes >= 4 ? kBytes / 4 : 1;
  uint32_t w[kWords];

  // p must be aligned to min(kBytes, 16) bytes.
  __device__ __forceinline__ void load(const IO* p) {
    if constexpr (kBytes >= 16) {
#pragma unroll
      for (int c = 0; c < kBytes / 16; ++c) {
        const uint4 x = reinterpret_cast<const uint4*>(p)[c];
        w[4 * c + 0] = x.x;
        w[4 * c + 1] = x.y;
        w[4 * c + 2] = x.z;
        w[4 * c + 3] = x.w;
      }
    } else if constexpr (kBytes == 8) {
      const uint2 x = *reinterpret_cast<const uint2*>(p);
      w[0] = x.x;
      w[1] = x.y;
    } else if constexpr (kBytes == 4) {
      w[0] = *reinterpret_cast<const uint32_t*>(p);
    } else {
      w[0] = *reinterpret_cast<const uint16_t*>(p);
    }
  }

  // Element e is read only when e < limit; the rest read as zero.
  __device__ __forceinline__ void load_masked(const IO* p, int limit) {
#pragma unroll
    for (int c = 0; c < kWords; ++c) w[c] = 0u;
#pragma unroll
    for (int e = 0; e < N; ++e) {
      if (e < limit) {
        if constexpr (sizeof(IO) == 4) {
          w[e] = reinterpret_cast<const uint32_t*>(p)[e];
        } else {
          const uint32_t h = reinterpret_cast<const uint16_t*>(p)[e];
          w[e / 2] |= (e & 1) ? (h << 16) : h;
        }
      }
    }
  }

  __device__ __forceinline__ void widen_to(float* dst) const {
    if constexpr (sizeof(IO) == 4) {
#pragma unroll
      for (int e = 0; e < N; ++e) dst[e] = __uint_as_float(w[e]);
    } else {
#pragma unroll
      for (int e = 0; e < N; ++e) {
        const uint32_t word = w[e / 2];
        dst[e] = widen_bits16<IO>((e & 1) ? (word >> 16) : (word & 0xffffu));
      }
    }
  }
};

// One I/O scalar in packed form (see RawSlice).
template <typename IO>
struct RawScalar {
  uint32_t w;
  __device__ __forceinline__ void load(const IO* p) {
    if constexpr (sizeof(IO) == 4) w = *reinterpret_cast<const uint32_t*>(p);
    else w = *reinterpret_cast<const uint16_t*>(p);
  }
  __device__ __forceinline__ float value() const {
    if constexpr (sizeof(IO) == 4) return __uint_as_float(w);
    else return widen_bits16<IO>(w);
  }
};

// Streaming (non-temporal) 16-byte accesses: data touched once per kernel,
// e.g. the decode state, bypasses cache retention.
typedef float vfloat4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_stream4(const float* p) {
  const vfloat4 x = __builtin_nontemporal_load(reinterpret_cast<const vfloat4*>(p));
  return make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void store_stream4(float* p, float4 x) {
  const vfloat4 y = {x.x, x.y, x.z, x.w};
  __builtin_nontemporal_store(y, reinterpret_cast<vfloat4*>(p));
}

__device__ __forceinline__ float readlane(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// ---------------------------------------------------------------- DPP
// dpp_ctrl encodings (GCN/CDNA DPP): quad_perm selectors and row mirrors.
constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <- lane 7-i within each 8
constexpr int kRowMirror = 0x140;     // lane i <- lane 15-i within each 16

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Inclusive prefix sum of a double over the 64 lanes of a wave, without LDS:
// Hillis-Steele steps inside each 16-lane row (DPP row_shr 1, 2, 4, 8 on both
// halves; lanes shifted in from outside the row read 0), then each row adds
// the totals of the rows before it (read from lanes 15, 31, 47).
template <int N>
__device__ __forceinline__ double dpp_row_shr(double x) {
  const unsigned long long b = __builtin_bit_cast(unsigned long long, x);
  const unsigned lo = static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(b), 0x110 + N, 0xF, 0xF, false));
  const unsigned hi = static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(b >> 32), 0x110 + N, 0xF, 0xF, false));
  return __builtin_bit_cast(double, static_cast<unsigned long long>(lo) | (static_cast<unsigned long long>(hi) << 32));
}
__device__ __forceinline__ double readlane(double x, int lane) {
  const unsigned long long b = __builtin_bit_cast(unsigned long long, x);
  const unsigned lo = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(b), lane));
  const unsigned hi = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(b >> 32), lane));
  return __builtin_bit_cast(double, static_cast<unsigned long long>(lo) | (static_cast<unsigned long long>(hi) << 32));
}
__device__ __forceinline__ double wave_prefix_sum(double x, int lane) {
  x += dpp_row_shr<1>(x);
  x += dpp_row_shr<2>(x);
  x += dpp_row_shr<4>(x);
  x += dpp_row_shr<8>(x);
  const double r0 = readlane(x, 15), r1 = readlane(x, 31), r2 = readlane(x, 47);
  const int row = lane >> 4;
  double before = 0.0;
  if (row >= 1) before += r0;
  if (row >= 2) before += r1;
  if (row >= 3) before += r2;
  return x + before;
}

// x + (x of lane i ^ 16) and x + (x of lane i ^ 32) with the gfx950 lane
// swaps (VALU, no LDS): v_permlane16_swap exchanges the odd 16-lane rows of
// its first operand with the even rows of its second, v_permlane32_swap the
// upper half of the first with the lower half of the second; with both
// operands holding x, their sum is the pairwise sum in every lane.  The
// instructions are written out because the compiler's builtins return one
// operand for both results.  The s_nop pairs cover the hazards around a
// lane swap that reads a just-written register.
__device__ __forceinline__ float xor16_sum(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return a + b;
}
__device__ __forceinline__ float xor32_sum(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return a + b;
}

// Two independent sums over all 64 lanes, interleaved step by step so that
// each chain's dependent DPP and lane-swap steps fill the other's hazard
// slots; every lane receives both sums.
__device__ __forceinline__ void wave_sum2(float& x, float& y) {
  x += dpp<kQuadSwap1>(x);
  y += dpp<kQuadSwap1>(y);
  x += dpp<kQuadSwap2>(x);
  y += dpp<kQuadSwap2>(y);
  x += dpp<kRowHalfMirror>(x);
  y += dpp<kRowHalfMirror>(y);
  x += dpp<kRowMirror>(x);
  y += dpp<kRowMirror>(y);
  float x1 = x, x2 = x, y1 = y, y2 = y;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\tv_permlane16_swap_b32 %2, %3\n\ts_nop 1"
               : "+v"(x1), "+v"(x2), "+v"(y1), "+v"(y2));
  x = x1 + x2;
  y = y1 + y2;
  x1 = x2 = x;
  y1 = y2 = y;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\tv_permlane32_swap_b32 %2, %3\n\ts_nop 1"
               : "+v"(x1), "+v"(x2), "+v"(y1), "+v"(y2));
  x = x1 + x2;
  y = y1 + y2;
}

// Two independent sums over aligned groups of G = 16, 32 or 64 lanes,
// interleaved as in wave_sum2.
template <int G>
__device__ __forceinline__ void group_sum2(float& x, float& y) {
  static_assert(G == 16 || G == 32 || G == 64, "group_sum2 takes groups of 16, 32 or 64 lanes");
  if constexpr (G == 64) {
    wave_sum2(x, y);
  } else {
    x += dpp<kQuadSwap1>(x);
    y += dpp<kQuadSwap1>(y);
    x += dpp<kQuadSwap2>(x);
    y += dpp<kQuadSwap2>(y);
    x += dpp<kRowHalfMirror>(x);
    y += dpp<kRowHalfMirror>(y);
    x += dpp<kRowMirror>(x);
    y += dpp<kRowMirror>(y);
    if constexpr (G == 32) {
      float x1 = x, x2 = x, y1 = y, y2 = y;
      asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\tv_permlane16_swap_b32 %2, %3\n\ts_nop 1"
                   : "+v"(x1), "+v"(x2), "+v"(y1), "+v"(y2));
      x = x1 + x2;
      y = y1 + y2;
    }
  }
}

// Sum over aligned groups of G consecutive lanes (G = 1, 2, 4, 8, 16, 32,
// 64); every lane of a group receives the group's sum.  Every lane of the
// wave must be active.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (G >= 2) x += dpp<kQuadSwap1>(x);
  if constexpr (G >= 4) x += dpp<kQuadSwap2>(x);
  if constexpr (G >= 8) x += dpp<kRowHalfMirror>(x);
  if constexpr (G >= 16) x += dpp<kRowMirror>(x);
  if constexpr (G >= 32) x = xor16_sum(x);
  if constexpr (G >= 64) x = xor32_sum(x);
  static_assert(G <= 64, "group_sum supports groups of at most 64 lanes");
  return x;
}

// ---------------------------------------------------------------- gates
// Logistic function with exp evaluated only at non-positive arguments.
__device__ __forceinline__ float gate_sigmoid(float x) {
  if (x >= 0.0f) return 1.0f / (1.0f + expf(-x));
  const float e = expf(x);
  return e / (1.0f + e);
}

// Logistic function from the hardware exp2 and reciprocal (v_exp_f32,
// v_rcp_f32; about one ulp each): 1 / (1 + 2^(-x log2(e))).  Saturates
// cleanly: 2^(+large) = inf gives 0, 2^(-large) = 0 gives 1.  For the
// elementwise epilogues, where the precise division would cost as much time
// as the memory traffic.
__device__ __forceinline__ float fast_sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}

// One element of the gated RMSNorm ([P1] `gated_rms_norm_op`): x times the
// row's 1 / sqrt(mean(x^2) + eps), the per-element scale and the gate's
// activation (silu: g sigmoid(g); else sigmoid(g)), with the epilogues'
// hardware sigmoid.
__device__ __forceinline__ float gated_norm(float x, float inv, float scale, float g, int silu) {
  const float s = fast_sigmoid(g);
  return x * inv * scale * (silu ? g * s : s);
}

// softplus(x) = max(x, 0) + log1p(exp(-|x|)), overflow-free.
__device__ __forceinline__ float gate_softplus(float x) {
  return fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x)));
}

// Log-decay of the raw gate: -exp(A_log) * softplus(a + dt_bias).
__device__ __forceinline__ float gate_log_decay(float a, float A_log, float dt_bias) {
  return -expf(A_log) * gate_softplus(a + dt_bias);
}

}  // namespace gdn
