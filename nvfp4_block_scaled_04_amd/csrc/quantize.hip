// BF16 -> NVFP4 quantisation kernels (gfx950).
//
// README "NVFP4 MegaMoE Kernel", "What We Have" (bridge layer): BF16 -> NVFP4
// with a global scale, and a variant with a pre-computed global scale;
// "Correctness Bugs Fixed" bugs 3 and 4: zero blocks get scale 0, underflow
// blocks are zeroed; CURRENT_BUG.md "What Works": the activation global scale
// is recomputed per call.
//
// Launches for a per-call global scale: one group (the forward's tokens, a
// dense A operand) takes two,
//   amax_partial   grid (P, 1):    chunk maxima of |x| -> ws[P]
//   quantize_gs    capped grid:    every block reduces ws to the global scale
//                                  2688 / max (1 if 0) and quantises 16-element
//                                  blocks grid-stride (32 B in, 9 B out each);
// several groups (weight preparation) three: amax_partial over (P, groups),
// gs_finalize per group, then quantize with the per-group scales.  With a
// given scale only quantize runs.  Max is exact, so the partial split cannot
// change the result.
#include "internal.hpp"
#include "steps.hpp"

namespace nvfp4 {

namespace {

constexpr int kThreads = kStepThreads;

// vec_per_group data vectors per group; group g starts rows_per_group rows
// (rows.ld vectors each) after group g - 1
__global__ __launch_bounds__(kThreads) void amax_partial_kernel(
    const uint4* __restrict__ x, Rows rows, int64_t rows_per_group, int64_t vec_per_group,
    int parts, float* __restrict__ partial) {
  const int g = blockIdx.y;
  const int p = blockIdx.x;
  const int64_t per = (vec_per_group + parts - 1) / parts;
  const int64_t lo = (int64_t)p * per;
  const int64_t hi = lo + per < vec_per_group ? lo + per : vec_per_group;
  __shared__ float red[kThreads / 64];
  const float m = block_max(thread_amax(x + (int64_t)g * rows_per_group * rows.ld, rows, lo, hi), red);
  if (threadIdx.x == 0) partial[(int64_t)g * parts + p] = m;
}

__global__ __launch_bounds__(kThreads) void gs_finalize_kernel(const float* __restrict__ partial,
                                                               int parts, float* __restrict__ gs_out) {
  const int g = blockIdx.x;
  __shared__ float red[kThreads / 64];
  const float gs = gs_from_partials(partial + (int64_t)g * parts, parts, red);
  if (threadIdx.x == 0) gs_out[g] = gs;
}

__global__ __launch_bounds__(kThreads) void quantize_gs_kernel(
    const uint4* __restrict__ x, Rows rows, int64_t nblocks, const float* __restrict__ partial,
    int parts, float* __restrict__ gs_out, uint2* __restrict__ q, uint8_t* __restrict__ sf) {
  __shared__ float red[kThreads / 64];
  quantize_gs_body(x, rows, nblocks, partial, parts, gs_out, q, sf, blockIdx.x, gridDim.x, red);
}

// One thread per 16-element block.  blocks_per_group = rows_per_group*cols/16.
__global__ __launch_bounds__(kThreads) void quantize_kernel(
    const uint4* __restrict__ x, Rows rows, int64_t nblocks, int64_t blocks_per_group,
    const float* __restrict__ gs, const float* __restrict__ gs_copy_src, int groups,
    float* __restrict__ gs_copy_dst, uint2* __restrict__ q, uint8_t* __restrict__ sf) {
  const int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (gs_copy_dst != nullptr && b < groups) gs_copy_dst[b] = gs_copy_src[b];
  if (b >= nblocks) return;
  quantize_at(x, rows, b, gs[b / blocks_per_group], q, sf);
}

// Quantise-and-scatter: every block reduces the chunk maxima to the global
// scale (block 0 stores it), then takes 16-element blocks of token rows
// grid-stride; a block is quantised once (same rule as quantize_kernel) and
// written to the k expert-order rows of its token (rows past offsets[E]
// skipped).
__global__ __launch_bounds__(kThreads) void quantize_scatter_kernel(
    const uint4* __restrict__ x, int64_t T, int64_t blocks_per_row, int k,
    const int32_t* __restrict__ inv_perm, const int32_t* __restrict__ offsets, int E,
    const float* __restrict__ partial, int parts, float* __restrict__ gs_out,
    uint2* __restrict__ q, uint8_t* __restrict__ sf) {
  __shared__ float red[kThreads / 64];
  const float g = gs_from_partials(partial, parts, red);
  if (blockIdx.x == 0 && threadIdx.x == 0) gs_out[0] = g;
  const int32_t n_valid = offsets[E];
  const int64_t nblocks = T * blocks_per_row;
  for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblocks;
       b += (int64_t)gridDim.x * kThreads) {
    const int64_t t = b / blocks_per_row, blk = b - t * blocks_per_row;
    const uint4 v0 = x[2 * b], v1 = x[2 * b + 1];
    const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    float xs[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      xs[2 * j] = bf16_to_f32(w[j] & 0xFFFFu);
      xs[2 * j + 1] = bf16_to_f32(w[j] >> 16);
    }
    uint32_t lo, hi, s;
    quantize_block16(xs, g, lo, hi, s);
    for (int j = 0; j < k; ++j) {
      const int32_t d = inv_perm[t * k + j];
      if (d >= n_valid) continue;
      q[(int64_t)d * blocks_per_row + blk] = make_uint2(lo, hi);
      sf[(int64_t)d * blocks_per_row + blk] = (uint8_t)s;
    }
  }
}

}  // namespace

hipError_t launch_quantize_scatter(const void* x, int64_t T, int64_t H, int k,
                                   const int32_t* inv_perm, const int32_t* offsets, int E,
                                   uint8_t* q, uint8_t* sf, float* gs_out, float* ws,
                                   hipStream_t stream) {
  if (T == 0) {
    fill_f32(gs_out, 1.0f, 1, stream);
    return hipGetLastError();
  }
  const int parts = quantize_parts(1, T, H);
  amax_partial_kernel<<<dim3(parts, 1), kThreads, 0, stream>>>(
      static_cast<const uint4*>(x), Rows{H / 8, H / 8}, T, T * H / 8, parts, ws);
  const int64_t nblocks = T * (H / 16);
  quantize_scatter_kernel<<<(unsigned)quant_grid(nblocks), kThreads, 0, stream>>>(
      static_cast<const uint4*>(x), T, H / 16, k, inv_perm, offsets, E, ws, parts, gs_out,
      reinterpret_cast<uint2*>(q), sf);
  return hipGetLastError();
}

int quantize_parts(int64_t groups, int64_t rows_per_group, int64_t cols) {
  // chunks per group for the amax pass: enough blocks to fill the chip,
  // at most one chunk per 2048 vectors, capped at 1024
  const int64_t vec = rows_per_group * cols / 8;
  if (groups <= 0 || vec <= 0) return 0;
  int64_t p = (2048 + groups - 1) / groups;
  int64_t cap = (vec + 2047) / 2048;
  if (p > cap) p = cap;
  if (p > 1024) p = 1024;
  if (p < 1) p = 1;
  return (int)p;
}

hipError_t launch_quantize(const void* x, int64_t groups, int64_t rows_per_group, int64_t cols,
                           int64_t ld_x, const float* gs_in, uint8_t* q, uint8_t* sf,
                           float* gs_out, float* ws, hipStream_t stream) {
  const int64_t rows = groups * rows_per_group;
  const int64_t nblocks = rows * (cols / 16);
  const uint4* xv = static_cast<const uint4*>(x);
  const Rows rv{cols / 8, ld_x / 8};
  if (groups == 0) return hipSuccess;
  const int parts = quantize_parts(groups, rows_per_group, cols);
  if (gs_in == nullptr && groups == 1 && parts > 0) {
    // one group: the quantising blocks reduce the chunk maxima themselves
    amax_partial_kernel<<<dim3(parts, 1), kThreads, 0, stream>>>(xv, rv, rows, rows * cols / 8,
                                                                  parts, ws);
    quantize_gs_kernel<<<(unsigned)quant_grid(nblocks), kThreads, 0, stream>>>(
        xv, rv, nblocks, ws, parts, gs_out, reinterpret_cast<uint2*>(q), sf);
    return hipGetLastError();
  }
  const float* gs = gs_in;
  if (gs_in == nullptr) {
    if (parts > 0) {
      amax_partial_kernel<<<dim3(parts, (unsigned)groups), kThreads, 0, stream>>>(
          xv, rv, rows_per_group, rows_per_group * cols / 8, parts, ws);
      gs_finalize_kernel<<<(unsigned)groups, kThreads, 0, stream>>>(ws, parts, gs_out);
    } else {
      // empty groups: global scale 1
      fill_f32(gs_out, 1.0f, groups, stream);
    }
    gs = gs_out;
  }
  const int64_t need = nblocks > groups ? nblocks : groups;
  if (need == 0) return hipGetLastError();
  const unsigned grid = (unsigned)((need + kThreads - 1) / kThreads);
  const bool copy = gs_in != nullptr && gs_out != gs_in;
  quantize_kernel<<<grid, kThreads, 0, stream>>>(
      xv, rv, nblocks, rows_per_group * (cols / 16) > 0 ? rows_per_group * (cols / 16) : 1,
      gs, gs_in, (int)groups, copy ? gs_out : nullptr, reinterpret_cast<uint2*>(q), sf);
  return hipGetLastError();
}

}  // namespace nvfp4
