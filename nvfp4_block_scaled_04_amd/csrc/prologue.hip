// The forward's steps before its GEMMs in three launches (gfx950).
//
// README "NVFP4 MegaMoE Kernel", "What We Have", MoE runner: quantise the
// activations with a per-call global scale, count the rows of every expert,
// compute the expert offsets and the expert-order permutation.  Run as
// separate kernels these are six launches (chunk maxima, global scale,
// quantisation, histogram, scan, scatter) plus one counter clear per GEMM;
// each launch in a dependent chain costs a few microseconds of dispatch,
// which at decode sizes is more than the work.  The independent steps share
// launches instead:
//   prologue_a  blocks [0, C):        routing histogram of chunk c (LDS)
//               blocks [C, C + P):    chunk maxima of |x|
//               block 0 also clears both GEMMs' scheduler counters
//   prologue_b  blocks [0, S):        one wave per bucket scans the histogram
//                                     over chunks (bucket offsets per chunk)
//               blocks [S, S + Q):    every block reduces the chunk maxima to
//                                     the global scale (block 0 stores it)
//                                     and quantises 16-element blocks of x,
//                                     grid-stride
//   route_scatter (route.hip)         the stable permutation
// Each role runs the same block body as its stand-alone kernel (steps.hpp),
// so the bytes are the same as those of nvfp4_quantize + nvfp4_moe_route.
#include "internal.hpp"
#include "steps.hpp"

namespace nvfp4 {

namespace {

__global__ __launch_bounds__(kStepThreads) void prologue_a_kernel(
    const int32_t* __restrict__ ids, int64_t M, int64_t chunk, int64_t C, int E,
    int32_t* __restrict__ hist, const uint4* __restrict__ x, int64_t vecs, int parts,
    float* __restrict__ partial, int* __restrict__ sched, int sched_ints) {
  extern __shared__ int32_t cnt[];
  __shared__ float red[kStepThreads / 64];
  const int64_t b = blockIdx.x;
  if (b == 0 && (int)threadIdx.x < sched_ints) sched[threadIdx.x] = 0;
  if (b < C) {
    const int64_t lo = b * chunk;
    const int64_t hi = lo + chunk < M ? lo + chunk : M;
    chunk_hist(ids, lo, hi, E, cnt, hist, C, b);
  } else {
    const int64_t p = b - C;
    const int64_t per = (vecs + parts - 1) / parts;
    const int64_t lo = p * per;
    const int64_t hi = lo + per < vecs ? lo + per : vecs;
    const float m = block_max(thread_amax(x, Rows{vecs, vecs}, lo, hi), red);
    if (threadIdx.x == 0) partial[p] = m;
  }
}

__global__ __launch_bounds__(kStepThreads) void prologue_b_kernel(
    int32_t* __restrict__ hist, int64_t C, int32_t* __restrict__ total, int E, int64_t scan_blocks,
    const uint4* __restrict__ x, Rows rows, int64_t nblocks, const float* __restrict__ partial,
    int parts, float* __restrict__ gs_out, uint2* __restrict__ q, uint8_t* __restrict__ sf) {
  __shared__ float red[kStepThreads / 64];
  const int64_t b = blockIdx.x;
  if (b < scan_blocks) {
    const int64_t bucket = b * (kStepThreads / 64) + (threadIdx.x >> 6);
    if (bucket <= E) scan_bucket(hist + bucket * C, C, total + bucket, threadIdx.x & 63);
  } else {
    quantize_gs_body(x, rows, nblocks, partial, parts, gs_out, q, sf, b - scan_blocks,
                     (int64_t)gridDim.x - scan_blocks, red);
  }
}

}  // namespace

hipError_t launch_forward_prologue(const void* x, int64_t T, int64_t H, const int32_t* topk_ids,
                                   int k, int E, uint8_t* a_q, uint8_t* a_sf, float* gs_a,
                                   float* qws, void* rws, int32_t* offsets, int32_t* perm,
                                   int32_t* inv_perm, int32_t* invalid_count, int* sched,
                                   int sched_ints, hipStream_t stream) {
  if (T <= 0 || sched_ints > kStepThreads) return hipErrorInvalidValue;
  const int64_t M = T * k;
  const int64_t chunk = route_chunk(M);
  const int64_t C = (M + chunk - 1) / chunk;
  const int parts = quantize_parts(1, T, H);
  int32_t* hist = static_cast<int32_t*>(rws);
  int32_t* total = hist + C * (int64_t)(E + 1);
  const size_t lds_hist = (size_t)(E + 1) * sizeof(int32_t);
  prologue_a_kernel<<<(unsigned)(C + parts), kStepThreads, lds_hist, stream>>>(
      topk_ids, M, chunk, C, E, hist, static_cast<const uint4*>(x), T * H / 8, parts, qws, sched,
      sched_ints);
  const int64_t nblocks = T * (H / 16);
  const int64_t scan_blocks = (E + 1 + kStepThreads / 64 - 1) / (kStepThreads / 64);
  prologue_b_kernel<<<(unsigned)(scan_blocks + quant_grid(nblocks)), kStepThreads, 0, stream>>>(
      hist, C, total, E, scan_blocks, static_cast<const uint4*>(x), Rows{H / 8, H / 8}, nblocks,
      qws, parts, gs_a, reinterpret_cast<uint2*>(a_q), a_sf);
  return launch_route_scatter(topk_ids, M, E, rws, offsets, perm, inv_perm, invalid_count, stream);
}

}  // namespace nvfp4
