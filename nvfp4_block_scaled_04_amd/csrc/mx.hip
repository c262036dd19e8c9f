// Re-encoding of NVFP4 data to MXFP4 for the block-scaled FP4 matrix
// instructions of gfx950 (v_mfma_scale_f32_32x32x64_f8f6f4).
//
// NVFP4 (README "NVFP4 MegaMoE Kernel", "What We Have", grouped GEMM): E2M1
// codes with one E4M3 scale per 16 elements.  The matrix instruction takes
// E2M1 codes with one power-of-two (E8M0) scale per 32 elements, the OCP MX
// layout.  Per 32-block (NVFP4 blocks 2j and 2j+1 of a row):
//   u_i = E2M1(q_i) * E4M3(sf)            exact in fp32 (<= 6 significant bits)
//   amax = max |u_i|; all zero -> scale byte 0, codes 0;
//   X = 2^(floor(log2 amax) - 2)          (MX conversion rule, E2M1 emax 2)
//   code_i = E2M1(u_i / X)                nearest, ties to even, saturating
//                                         at 6, sign bit kept
// The E8M0 byte of block j is written to bytes 2j and 2j+1 of a scale row of
// C/16 bytes: the MX scales then have the NVFP4 scale layout and every scale
// load and weight packing step of the GEMM applies unchanged.
#include "internal.hpp"
#include "device.hpp"

namespace nvfp4 {

namespace {

// one thread per 32-block: 16 code bytes + 2 scale bytes in, the same out
__global__ __launch_bounds__(256) void mx_reencode_kernel(const uint4* __restrict__ q,
                                                          const uint16_t* __restrict__ sf,
                                                          int64_t nblocks,
                                                          uint4* __restrict__ q_mx,
                                                          uint16_t* __restrict__ sc_mx) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const uint4 c = q[b];
  const uint32_t s2 = sf[b];
  const float s0 = e4m3_decode(s2 & 0x7Fu), s1 = e4m3_decode((s2 >> 8) & 0x7Fu);
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  float u[32];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const float s = d < 2 ? s0 : s1;
    // codes 8d .. 8d+7 of the block, two per conversion (byte p of the
    // dword); E2M1 -> fp32 is exact and keeps the sign of -0; the product
    // with the E4M3 scale is exact
    const auto v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 0);
    const auto v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 1);
    const auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 2);
    const auto v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 3);
    u[8 * d + 0] = v0[0] * s; u[8 * d + 1] = v0[1] * s;
    u[8 * d + 2] = v1[0] * s; u[8 * d + 3] = v1[1] * s;
    u[8 * d + 4] = v2[0] * s; u[8 * d + 5] = v2[1] * s;
    u[8 * d + 6] = v3[0] * s; u[8 * d + 7] = v3[1] * s;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(u[i]));
  uint4 o = make_uint4(0, 0, 0, 0);
  uint32_t sb = 0;
  if (amax > 0.0f) {
    // amax >= 2^-10 is a normal fp32: floor(log2 amax) is its exponent field - 127
    const uint32_t ef = (__float_as_uint(amax) >> 23) & 0xFFu;
    sb = ef - 2u;                                       // E8M0 byte: (ef - 127 - 2) + 127
    const float inv = __uint_as_float((254u - sb) << 23);   // 1/X = 2^(127 - sb)
    uint32_t r[4];
#pragma unroll
    for (int d = 0; d < 4; ++d)
      r[d] = e2m1_pack8(u[8 * d] * inv, u[8 * d + 1] * inv, u[8 * d + 2] * inv,
                        u[8 * d + 3] * inv, u[8 * d + 4] * inv, u[8 * d + 5] * inv,
                        u[8 * d + 6] * inv, u[8 * d + 7] * inv);
    o = make_uint4(r[0], r[1], r[2], r[3]);
  }
  q_mx[b] = o;
  sc_mx[b] = (uint16_t)(sb | (sb << 8));
}

}  // namespace

hipError_t launch_mx_reencode(const uint8_t* q, const uint8_t* sf, int64_t rows, int64_t cols,
                              uint8_t* q_mx, uint8_t* sc_mx, hipStream_t stream) {
  const int64_t nblocks = rows * (cols / 32);
  if (nblocks == 0) return hipSuccess;
  mx_reencode_kernel<<<(unsigned)((nblocks + 255) / 256), 256, 0, stream>>>(
      reinterpret_cast<const uint4*>(q), reinterpret_cast<const uint16_t*>(sf), nblocks,
      reinterpret_cast<uint4*>(q_mx), reinterpret_cast<uint16_t*>(sc_mx));
  return hipGetLastError();
}

}  // namespace nvfp4
