// Routing-weighted combine of expert outputs back to tokens (gfx950).
//
// README "NVFP4 MegaMoE Kernel", "What We Have", MoE runner step 6: scatter
// with routing weights.  Written as a gather so no atomics are needed and the
// result is deterministic:
//   out[t][n] = bf16( sum_{j<k} w[t][j] * y[inv_perm[t*k+j]][n] ),
// fp32 accumulation in slot order; rows d >= offsets[E] (invalid expert ids)
// contribute nothing.  One block per token; each thread moves 16 bytes
// (8 BF16) per row, so every wave reads 1 KiB contiguous spans.  y is read
// once and out written once: both go through non-temporal accesses, which
// keep them from displacing other lines in the caches (6% faster at
// T=8192, H=7168, k=8 than plain accesses).
#include "internal.hpp"
#include "device.hpp"

namespace nvfp4 {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 128;
constexpr int kBatch = 8;                   // rows whose loads are in flight together

__global__ __launch_bounds__(kThreads) void combine_kernel(
    const uint4* __restrict__ y, const int32_t* __restrict__ inv_perm,
    const float* __restrict__ topk_w, const int32_t* __restrict__ offsets, int k, int E,
    int64_t H, uint4* __restrict__ out) {
  const int64_t t = blockIdx.x;
  const int64_t hv = H / 8;                 // 16-byte vectors per row
  const int32_t n_valid = offsets[E];
  for (int64_t v = threadIdx.x; v < hv; v += kThreads) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j0 = 0; j0 < k; j0 += kBatch) {
      // issue the batch's row loads first, then accumulate in slot order
      uint4 r[kBatch];
      float w[kBatch];
      bool ok[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int j = j0 + b;
        const int32_t d = j < k ? inv_perm[t * k + j] : n_valid;
        ok[b] = d < n_valid;          // slots past k and invalid expert ids add nothing
        w[b] = ok[b] ? topk_w[t * k + j] : 0.0f;
        if (ok[b]) {
          const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(y + (int64_t)d * hv + v));
          r[b] = make_uint4(q[0], q[1], q[2], q[3]);
        } else {
          r[b] = make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        if (!ok[b]) continue;
        const uint32_t p[4] = {r[b].x, r[b].y, r[b].z, r[b].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = fmaf(w[b], bf16_to_f32(p[i] & 0xFFFFu), acc[2 * i]);
          acc[2 * i + 1] = fmaf(w[b], bf16_to_f32(p[i] >> 16), acc[2 * i + 1]);
        }
      }
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    const u32x4 oq = {o.x, o.y, o.z, o.w};
    __builtin_nontemporal_store(oq, reinterpret_cast<u32x4*>(out + t * hv + v));
  }
}

}  // namespace

hipError_t launch_combine(const void* y, const int32_t* inv_perm, const float* topk_w,
                          const int32_t* offsets, int64_t T, int k, int E, int64_t H, void* out,
                          hipStream_t stream) {
  if (T == 0) return hipSuccess;
  combine_kernel<<<(unsigned)T, kThreads, 0, stream>>>(
      static_cast<const uint4*>(y), inv_perm, topk_w, offsets, k, E, H, static_cast<uint4*>(out));
  return hipGetLastError();
}

}  // namespace nvfp4
