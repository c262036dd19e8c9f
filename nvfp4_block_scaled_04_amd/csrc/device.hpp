// Device-side helpers shared by the NVFP4 kernels (gfx950 only).
//
// NVFP4 as used here (README "NVFP4 MegaMoE Kernel", "What We Have", grouped
// GEMM): E2M1 element codes (bit 3 = sign, magnitudes 0 .5 1 1.5 2 3 4 6),
// one OCP E4M3 scale (bias 7, max 448, subnormal step 2^-9) per 16 elements,
// fp32 global scale.  The encoders below are written from the bit layouts of
// the formats; every operation rounds to nearest even.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr float kUnderflow = 0.01171875f;   // 6 * 2^-9: E2M1 max * E4M3 min subnormal
constexpr float kGsNumerator = 2688.0f;     // 448 * 6: E4M3 max * E2M1 max
constexpr float kE4m3Max = 448.0f;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Two floats -> two bf16 (lo in the low half), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// E4M3 byte of t, 2^-9 <= t <= 448, nearest with ties to even.
// Normal range (t >= 2^-6): round the fp32 mantissa to 3 bits on the bit
// pattern (the carry moves into the exponent) and rebias 127 -> 7.
// Subnormal range: t = k * 2^-9 with k = rint(t * 512) in 1..8 (k = 8 is the
// smallest normal, byte 0x08, so the two ranges meet without a seam).
__device__ __forceinline__ uint32_t e4m3_encode(float t) {
  const uint32_t sub = (uint32_t)__builtin_rintf(t * 512.0f);
  uint32_t u = __float_as_uint(t);
  u += 0x7FFFFu + ((u >> 20) & 1u);
  const uint32_t nrm = (u >> 20) - (120u << 3);
  return t < 0.015625f ? sub : nrm;   // both computed: a select, not a branch
}

// value of an E4M3 byte with sign bit clear (never the NaN byte here)
__device__ __forceinline__ float e4m3_decode(uint32_t b) {
  uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const float sub = (float)m * 0.001953125f;   // m * 2^-9, exact
  const float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return e == 0 ? sub : nrm;
}

// Eight fp32 values -> eight E2M1 codes (value i in bits 4i..4i+3):
// v_cvt_scalef32_pk_fp4_f32 (scale 1) rounds to nearest with ties to the
// even code, saturates at 6 and takes the sign bit from the value (so -0
// gives code 8).
__device__ __forceinline__ uint32_t e2m1_pack8(float v0, float v1, float v2, float v3, float v4,
                                               float v5, float v6, float v7) {
  uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v0, v1, 1.0f, 0);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, v2, v3, 1.0f, 1);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, v4, v5, 1.0f, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, v6, v7, 1.0f, 3);
}

// x / 6 rounded to nearest even, equal to the IEEE division for every fp32
// x >= 2^-125 (checked exhaustively against it; below, where the quotient is
// subnormal, the two can differ in the last place): the product with
// RN(1/6), then one FMA correction by the remainder, which the FMA computes
// exactly.  Callers use it where x >= 6 * 2^-9, or where the result is
// discarded.
__device__ __forceinline__ float div6_rn(float x) {
  const float c = 0.16666667f;                 // RN(1/6), 0x3E2AAAAB
  const float q0 = x * c;
  const float r = __builtin_fmaf(-q0, 6.0f, x);
  return __builtin_fmaf(r, c, q0);
}

// One 16-element block -> (8 bytes of packed codes, scale byte).
// x[i] are the fp32 values, gs the global scale.  Operation order:
// a_s = amax*gs; zero/underflow (amax == 0 or a_s < 6*2^-9) -> all zero;
// t = a_s/6; sf = E4M3(min(t,448)); r = gs/dec(sf);
// code_i = sign(x_i) | E2M1(min(|x_i*r|, 6)) (x_i*r has the sign of x_i).
__device__ __forceinline__ void quantize_block16(const float (&x)[16], float gs, uint32_t& lo,
                                                 uint32_t& hi, uint32_t& sf) {
#pragma clang fp contract(off)
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const float a_s = amax * gs;
  lo = 0u; hi = 0u; sf = 0u;
  if (amax == 0.0f || a_s < kUnderflow) return;
  const float t = fminf(a_s / 6.0f, kE4m3Max);
  sf = e4m3_encode(t);
  const float r = gs / e4m3_decode(sf);
  lo = e2m1_pack8(x[0] * r, x[1] * r, x[2] * r, x[3] * r, x[4] * r, x[5] * r, x[6] * r, x[7] * r);
  hi = e2m1_pack8(x[8] * r, x[9] * r, x[10] * r, x[11] * r, x[12] * r, x[13] * r, x[14] * r,
                  x[15] * r);
}

}  // namespace nvfp4
