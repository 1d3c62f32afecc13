// chunk_mfma.hpp -- MFMA fragment helpers shared by the chunked prefill
// kernels (gfx950).
//
// Operand layouts of the two matrix instructions used (checked on the
// hardware):
//   v_mfma_f32_16x16x32_bf16: lane l supplies A[l % 16][8 (l / 16) .. +7] and
//     B[8 (l / 16) .. +7][l % 16]; accumulator element i of lane l is
//     D[4 (l / 16) + i][l % 16].
//   v_mfma_f32_16x16x4_f32: lane l supplies A[l % 16][l / 16] and
//     B[l / 16][l % 16]; same accumulator layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_device.hpp"

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 2^x in one v_exp_f32; used with log-decays pre-scaled by log2(e).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16_t to_bf16(float x) { return __builtin_bit_cast(bf16_t, static_cast<__bf16>(x)); }

// Operand fragment of a 16x16x32 MFMA: lane l reads row (l % 16), k = 8 (l / 16) .. +7,
// of a bf16 matrix stored with k contiguous (row stride `stride` elements).
__device__ __forceinline__ bf16x8 frag(const bf16_t* base, int stride, int lane) {
  return *reinterpret_cast<const bf16x8*>(base + (lane & 15) * stride + 8 * (lane >> 4));
}

// acc += A (16 x K) * B (K x 16).  A: rows of a (stride sa), k contiguous.
// B: column n of B is row n of b (stride sb), k contiguous.
template <int K>
__device__ __forceinline__ f32x4 mma(f32x4 acc, const bf16_t* a, int sa, const bf16_t* b, int sb, int lane) {
#pragma unroll
  for (int kk = 0; kk < K; kk += 32)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag(a + kk, sa, lane), frag(b + kk, sb, lane), acc, 0, 0, 0);
  return acc;
}

// Same with the k range [k0, k1) chosen at run time (multiples of 32).
__device__ __forceinline__ f32x4 mma_range(f32x4 acc, const bf16_t* a, int sa, const bf16_t* b, int sb, int k0,
                                           int k1, int lane) {
  for (int kk = k0; kk < k1; kk += 32)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag(a + kk, sa, lane), frag(b + kk, sb, lane), acc, 0, 0, 0);
  return acc;
}

// acc += A (16 x 16) * B (16 x 16) in f32 (16x16x4 f32 MFMA); both row-major
// in LDS: A[m][k] at a[m * sa + k], B[k][n] at b[k * sb + n].
__device__ __forceinline__ f32x4 mma_f32(f32x4 acc, const float* a, int sa, const float* b, int sb, int lane) {
#pragma unroll
  for (int k0 = 0; k0 < 16; k0 += 4)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[(lane & 15) * sa + k0 + (lane >> 4)],
                                               b[(k0 + (lane >> 4)) * sb + (lane & 15)], acc, 0, 0, 0);
  return acc;
}

// Accumulator element i of lane l sits at row 4 (l / 16) + i, column l % 16.
__device__ __forceinline__ int acc_row(int lane, int i) { return 4 * (lane >> 4) + i; }
__device__ __forceinline__ int acc_col(int lane) { return lane & 15; }

}  // namespace gdn
