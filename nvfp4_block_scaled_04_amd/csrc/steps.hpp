// Block- and wave-level bodies of the steps that precede the GEMMs: the
// global amax of x, the global scale, the token quantisation, and the
// routing histogram and its scan over chunks.  The stand-alone kernels
// (quantize.hip, route.hip) and the forward's fused prologue (prologue.hip)
// run the same code, so the two paths give identical bytes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"

namespace nvfp4 {

constexpr int kStepThreads = 256;   // block size of every kernel built from these bodies

// Max over the block (kStepThreads threads); every thread gets the result.
// red: kStepThreads / 64 floats of LDS, used once per kernel.
__device__ __forceinline__ float block_max(float m, float* red) {
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kStepThreads / 64; ++i) r = fmaxf(r, red[i]);
  return r;
}

// Rows of a bf16 tensor in 16-byte vectors: rv vectors of data per row, rows
// ld vectors apart (ld == rv: contiguous).  at(i) is the position of data
// vector i (row-major).
struct Rows {
  int64_t rv, ld;
  __device__ __forceinline__ int64_t at(int64_t i) const {
    if (ld == rv) return i;
    const int64_t row = i / rv;
    return row * ld + (i - row * rv);
  }
};

// This thread's max |x| over the data vectors [lo, hi) (8 values each),
// block-strided.  Max is exact, so any split of the range gives the same
// global result.
__device__ __forceinline__ float thread_amax(const uint4* __restrict__ x, Rows rows, int64_t lo,
                                             int64_t hi) {
  float m = 0.0f;
  for (int64_t i = lo + threadIdx.x; i < hi; i += kStepThreads) {
    const uint4 v = x[rows.at(i)];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m = fmaxf(m, fabsf(bf16_to_f32(w[j] & 0xFFFFu)));
      m = fmaxf(m, fabsf(bf16_to_f32(w[j] >> 16)));
    }
  }
  return m;
}

// The global scale from the chunk maxima of one group: 2688 / amax, or 1
// when every element is zero (README "NVFP4 MegaMoE Kernel", "What We Have",
// bridge layer: BF16 -> NVFP4 with a global scale).  Every thread gets it.
__device__ __forceinline__ float gs_from_partials(const float* __restrict__ partial, int parts,
                                                 float* red) {
  float m = 0.0f;
  for (int i = threadIdx.x; i < parts; i += kStepThreads) m = fmaxf(m, partial[i]);
  const float r = block_max(m, red);
  return (r == 0.0f) ? 1.0f : kGsNumerator / r;
}

// 16-element block b of x (data vectors 2b and 2b + 1, one row) -> 8 bytes
// of codes and a scale byte, with global scale g
__device__ __forceinline__ void quantize_at(const uint4* __restrict__ x, Rows rows, int64_t b,
                                            float g, uint2* __restrict__ q,
                                            uint8_t* __restrict__ sf) {
  const int64_t v = rows.at(2 * b);
  const uint4 v0 = x[v], v1 = x[v + 1];
  const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  float xs[16];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    xs[2 * j] = bf16_to_f32(w[j] & 0xFFFFu);
    xs[2 * j + 1] = bf16_to_f32(w[j] >> 16);
  }
  uint32_t lo, hi, s;
  quantize_block16(xs, g, lo, hi, s);
  q[b] = make_uint2(lo, hi);
  sf[b] = (uint8_t)s;
}

// Grid of the quantisation with an in-kernel global scale: every block
// reduces the chunk maxima itself, so the grid is capped (the blocks then
// stride over the 16-element blocks) to keep that reduction a few MB of L2
// reads at most.
constexpr int64_t kQuantMaxBlocks = 2048;
inline int64_t quant_grid(int64_t nblocks) {
  const int64_t g = (nblocks + kStepThreads - 1) / kStepThreads;
  return g < kQuantMaxBlocks ? g : kQuantMaxBlocks;
}

// Quantisation of one group of nblocks 16-element blocks whose global scale
// follows from the chunk maxima: block `blk` of `nblk` reduces them, block 0
// stores the scale, and the 16-element blocks are taken grid-stride.
__device__ __forceinline__ void quantize_gs_body(const uint4* __restrict__ x, Rows rows,
                                                 int64_t nblocks, const float* __restrict__ partial,
                                                 int parts, float* __restrict__ gs_out,
                                                 uint2* __restrict__ q, uint8_t* __restrict__ sf,
                                                 int64_t blk, int64_t nblk, float* red) {
  const float g = gs_from_partials(partial, parts, red);
  if (blk == 0 && threadIdx.x == 0) gs_out[0] = g;
  for (int64_t b = blk * kStepThreads + threadIdx.x; b < nblocks; b += nblk * kStepThreads)
    quantize_at(x, rows, b, g, q, sf);
}

// routing bucket of an expert id: ids outside [0, E) share bucket E
__device__ __forceinline__ int bucket_of(int32_t id, int E) {
  return (id >= 0 && id < E) ? id : E;
}

// LDS histogram of ids[lo, hi) over the E + 1 buckets, stored as column c
// of the bucket-major hist[b][C].  cnt: E + 1 ints of LDS.
__device__ __forceinline__ void chunk_hist(const int32_t* __restrict__ ids, int64_t lo, int64_t hi,
                                           int E, int32_t* cnt, int32_t* __restrict__ hist,
                                           int64_t C, int64_t c) {
  const int nb = E + 1;
  for (int b = threadIdx.x; b < nb; b += kStepThreads) cnt[b] = 0;
  __syncthreads();
  for (int64_t f = lo + threadIdx.x; f < hi; f += kStepThreads) atomicAdd(&cnt[bucket_of(ids[f], E)], 1);
  __syncthreads();
  for (int b = threadIdx.x; b < nb; b += kStepThreads) hist[(int64_t)b * C + c] = cnt[b];
}

// inclusive prefix sum over the 64 lanes of a wave
__device__ __forceinline__ int32_t wave_incl_scan(int32_t v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  return v;
}

// One wave: row h[0:C) of the histogram (one bucket's count per chunk)
// becomes the bucket's rows in earlier chunks (exclusive scan); *total gets
// the bucket's row count.
__device__ __forceinline__ void scan_bucket(int32_t* __restrict__ h, int64_t C,
                                            int32_t* __restrict__ total, int lane) {
  int32_t run = 0;
  for (int64_t c0 = 0; c0 < C; c0 += 64) {
    const int64_t c = c0 + lane;
    const int32_t v = c < C ? h[c] : 0;
    const int32_t incl = wave_incl_scan(v, lane);
    if (c < C) h[c] = run + incl - v;
    run += __shfl(incl, 63, 64);
  }
  if (lane == 0) *total = run;
}

}  // namespace nvfp4
