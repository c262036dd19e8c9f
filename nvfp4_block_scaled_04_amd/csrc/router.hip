// Router: top-k of the expert logits and a softmax over the k chosen.
//
// The pages take routing ids and weights as inputs to the MoE runner (its
// last step scatters "with routing weights"); the tiny workload fixes the
// router as top-k of the logits followed by a softmax over those k.  The
// choice: the k largest logits in decreasing order, equal logits in
// increasing expert id, w_j = exp(l_j - l_max) / sum_i exp(l_i - l_max) in
// fp32.
//
// One wave per token.  Lane l holds logits l, l + 64, ... (up to 16 per
// lane, E <= 1024); each of the k rounds takes the wave-wide largest
// remaining value (lowest id among equals) with a butterfly reduction and
// retires it; lane j keeps round j's winner for the softmax and the store.
#include "internal.hpp"
#include "device.hpp"

namespace nvfp4 {

namespace {

constexpr int kRouterMaxPerLane = 16;    // E <= 1024

// (value, id) of the better of two candidates: larger value, then lower id
__device__ __forceinline__ void better(float& v, int& id, float v2, int id2) {
  if (v2 > v || (v2 == v && id2 < id)) {
    v = v2;
    id = id2;
  }
}

__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ logits,
                                                          int64_t T, int E, int k,
                                                          int32_t* __restrict__ topk_ids,
                                                          float* __restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;                          // the whole wave
  const float* row = logits + t * E;
  float v[kRouterMaxPerLane];
#pragma unroll
  for (int i = 0; i < kRouterMaxPerLane; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : -INFINITY;         // logits are finite: padding never wins
  }
  float my_v = 0.0f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    // this lane's best remaining candidate
    float bv = v[0];
    int bid = lane;
#pragma unroll
    for (int i = 1; i < kRouterMaxPerLane; ++i) better(bv, bid, v[i], lane + 64 * i);
    // wave-wide best
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oid = __shfl_xor(bid, off);
      better(bv, bid, ov, oid);
    }
    // retire it (its owner lane), keep it in lane j
#pragma unroll
    for (int i = 0; i < kRouterMaxPerLane; ++i)
      if (lane + 64 * i == bid) v[i] = -INFINITY;
    if (lane == j) {
      my_v = bv;
      my_id = bid;
    }
  }
  // softmax over the chosen logits; round 0's winner is the maximum
  const float vmax = __shfl(my_v, 0);
  const float ex = lane < k ? __expf(my_v - vmax) : 0.0f;
  float sum = ex;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane < k) {
    topk_ids[t * k + lane] = my_id;
    topk_w[t * k + lane] = ex / sum;
  }
}

}  // namespace

hipError_t launch_router_topk(const float* logits, int64_t T, int E, int k, int32_t* topk_ids,
                              float* topk_w, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int64_t blocks = (T + 3) / 4;
  router_topk_kernel<<<(unsigned)blocks, 256, 0, stream>>>(logits, T, E, k, topk_ids, topk_w);
  return hipGetLastError();
}

}  // namespace nvfp4
