// ms_mfma.hpp: 16x16 tiles on the f32 MFMA of gfx950, shared by the matrix-scan
// kernels and its gradient.
//
// v_mfma_f32_16x16x4_f32 on a wave of 64 lanes, lane 16 r + c. Four of them
// make one 16x16x16 product D = A X + C, with
//   A: lane (r, c) holds A[c][4r .. 4r+3]   (row c, four consecutive columns)
//   X: lane (r, c) holds X[4r .. 4r+3][c]   (column c, four consecutive rows)
//   C, D: lane (r, c) holds D[4r .. 4r+3][c], the same order as X,
// so a chain h <- a h + b feeds each result back with no data movement.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sx {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.0f, 0.0f, 0.0f, 0.0f}; }

__device__ __forceinline__ f32x4 mfma_16x16x16(f32x4 a, f32x4 x, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], x[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], x[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], x[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], x[3], c, 0, 0, 0);
  return c;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats to two bf16 (round to nearest even), packed low then high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// The upper halves (bf16 patterns) of two f32 bit patterns, packed low then high.
__device__ __forceinline__ uint32_t upper_halves(uint32_t lo, uint32_t hi) {
  return __builtin_amdgcn_perm(hi, lo, 0x07060302u);
}

// D = A X + C as above, for an A given in bf16 (lane (r, c): A[c][4r .. 4r+3], two
// per word, the lower index in the low half) and X, C in f32, with every product
// of an entry of A and an entry of X exact: X is cut into three bf16 parts,
// X = hi + mid + lo exactly. hi is X truncated to bf16 (its low 16 bits cleared),
// mid the same of what is left, and what is left after that has at most eight
// significant bits, so lo is that remainder itself. Products of bf16 values are
// exact in f32, so the result carries the rounding of f32 sums only, as the f32
// MFMA does. Three v_mfma_f32_16x16x16_bf16 (the f32 16x16x4's operand layout
// with all of K in one instruction), smallest part first, each taking the last
// one's result as its accumulator. They stay one opcode on purpose: a
// v_mfma_f32_16x16x32_bf16 that took a 16x16x16's result as its accumulator
// (hi and mid in one instruction) was measured to read the accumulator before
// that result had landed, dropping the lo product.
__device__ __forceinline__ f32x4 mfma_16x16x16_bf16a(uint2 a, f32x4 x, f32x4 c) {
  uint32_t u[4], m1[4], lo[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    u[q] = __float_as_uint(x[q]);
    const float r1 = x[q] - __uint_as_float(u[q] & 0xffff0000u);  // exact
    m1[q] = __float_as_uint(r1);
    lo[q] = __float_as_uint(r1 - __uint_as_float(m1[q] & 0xffff0000u));  // exact; low 16 bits are zero
  }
  const s16x4_t av = __builtin_bit_cast(s16x4_t, a);
  const uint2 h2 = make_uint2(upper_halves(u[0], u[1]), upper_halves(u[2], u[3]));
  const uint2 m2 = make_uint2(upper_halves(m1[0], m1[1]), upper_halves(m1[2], m1[3]));
  const uint2 l2 = make_uint2(upper_halves(lo[0], lo[1]), upper_halves(lo[2], lo[3]));
  c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, __builtin_bit_cast(s16x4_t, l2), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, __builtin_bit_cast(s16x4_t, m2), c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, __builtin_bit_cast(s16x4_t, h2), c, 0, 0, 0);
}

// 4 x 4 transpose inside each quad of lanes: lane j of a quad holds x[v] = M[j][v]
// and receives M[v][j]. Two exchange levels (partner j ^ 1, then j ^ 2), each
// taking the partner's register v ^ bit where lane and register differ in that bit.
__device__ __forceinline__ f32x4 quad_transpose(f32x4 x, int j) {
  f32x4 y, z;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float pv = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x[v ^ 1]), 0xB1, 0xF, 0xF, false));
    y[v] = ((j ^ v) & 1) ? pv : x[v];
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float pv = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(y[v ^ 2]), 0x4E, 0xF, 0xF, false));
    z[v] = ((j ^ v) & 2) ? pv : y[v];
  }
  return z;
}

}  // namespace sx
