// Expert offsets and the stable expert-order permutation (gfx950).
//
// README "NVFP4 MegaMoE Kernel", "Correctness Bugs Fixed" bug 5: experts are
// counted by a histogram (bincount), not an O(n x E) mask.  "Key Lessons" 4:
// quantise the compact rows, then place them.
//
// The flat pairs f = t*k + j are cut into C chunks of `chunk` entries.
//   route_hist     grid C:  LDS histogram of each chunk -> hist[b][c], bucket-
//                           major (bucket E collects ids outside [0, E))
//   route_scan     grid E+1, one wave per bucket b: hist[b][c] becomes the
//                           rows of b in chunks before c (exclusive scan over
//                           chunks); total[b] = rows of b
//   route_scatter  grid C, one wave: exclusive scan of total[] over buckets
//                           (the bucket bases; block 0 writes them as the
//                           expert offsets), then walks its chunk in order,
//                           64 entries at a time; a lane's rank among equal
//                           buckets of the batch comes from ballots, so every
//                           bucket keeps increasing f (a stable counting sort).
// The forward runs the histogram and the scan inside its fused prologue
// (prologue.hip) and then the same scatter.  All integer; integer atomics
// only in LDS, where order cannot matter.
#include "internal.hpp"
#include "steps.hpp"

namespace nvfp4 {

namespace {

constexpr int kHistThreads = kStepThreads;
constexpr int64_t kMinChunk = 256;
constexpr int64_t kMaxChunks = 1024;
constexpr int kScatterBatches = 4;   // 64-entry batches whose ids a lane loads at once

int64_t chunk_size(int64_t M) {
  int64_t ch = kMinChunk;
  if ((M + ch - 1) / ch > kMaxChunks) ch = ((M + kMaxChunks - 1) / kMaxChunks + 63) / 64 * 64;
  return ch;
}

__global__ __launch_bounds__(kHistThreads) void route_hist_kernel(
    const int32_t* __restrict__ ids, int64_t M, int64_t chunk, int64_t C, int E,
    int32_t* __restrict__ hist) {
  extern __shared__ int32_t cnt[];
  const int64_t lo = (int64_t)blockIdx.x * chunk;
  const int64_t hi = lo + chunk < M ? lo + chunk : M;
  chunk_hist(ids, lo, hi, E, cnt, hist, C, blockIdx.x);
}

__global__ __launch_bounds__(64) void route_scan_kernel(int32_t* __restrict__ hist, int64_t C,
                                                        int32_t* __restrict__ total) {
  scan_bucket(hist + (int64_t)blockIdx.x * C, C, total + blockIdx.x, threadIdx.x);
}

// Lanes of the wave whose bucket equals this lane's, among the lanes in
// `active`: one ballot per bit of the bucket index (nbits bits cover 0..E).
__device__ __forceinline__ uint64_t same_bucket_lanes(int e, bool active, int nbits) {
  uint64_t m = __ballot(active);
  for (int bit = 0; bit < nbits; ++bit) {
    const bool set = (e >> bit) & 1;
    const uint64_t ones = __ballot(active && set);
    m &= set ? ones : ~ones;
  }
  return m;
}

__global__ __launch_bounds__(64) void route_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t M, int64_t chunk, int64_t C, int E,
    const int32_t* __restrict__ hist, const int32_t* __restrict__ total,
    int32_t* __restrict__ offsets, int32_t* __restrict__ invalid_count,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm) {
  extern __shared__ int32_t cur[];
  const int nb = E + 1;
  const int lane = threadIdx.x;
  const int64_t lo = (int64_t)blockIdx.x * chunk;
  const int64_t hi = lo + chunk < M ? lo + chunk : M;
  // the first batches' ids, loaded while the bucket bases are computed
  int32_t pre[kScatterBatches];
#pragma unroll
  for (int i = 0; i < kScatterBatches; ++i) {
    const int64_t f = lo + 64 * i + lane;
    pre[i] = f < hi ? ids[f] : 0;
  }
  // bucket bases: each lane sums a contiguous segment of total[], then an
  // exclusive scan of the segment sums across the wave
  const int seg = (nb + 63) / 64;
  const int s0 = lane * seg;
  int32_t local = 0;
  for (int i = 0; i < seg; ++i)
    if (s0 + i < nb) local += total[s0 + i];
  int32_t run = wave_incl_scan(local, lane) - local;
  for (int i = 0; i < seg; ++i) {
    const int b = s0 + i;
    if (b < nb) {
      if (blockIdx.x == 0) offsets[b] = run;
      cur[b] = run + hist[(int64_t)b * C + blockIdx.x];
      run += total[b];
    }
  }
  if (blockIdx.x == 0 && invalid_count != nullptr && lane == (E / seg)) {
    // the lane owning bucket E: its rows are the invalid pairs
    invalid_count[0] = total[E];
  }
  __syncthreads();
  const int nbits = 32 - __builtin_clz((unsigned)E);   // bits of the largest bucket, E
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t base = lo, i = 0; base < hi; base += 64, ++i) {
    const int64_t f = base + lane;
    const bool active = f < hi;
    int32_t id;
    if (i < kScatterBatches) {
      id = pre[0];
#pragma unroll
      for (int j = 1; j < kScatterBatches; ++j)
        if (i == j) id = pre[j];
    } else {
      id = active ? ids[f] : 0;
    }
    const int e = bucket_of(id, E);
    const uint64_t m = same_bucket_lanes(e, active, nbits);
    const int rank = __popcll(m & below), cnt = __popcll(m);
    if (active) {
      const int32_t pos = cur[e] + rank;
      perm[pos] = (int32_t)f;
      inv_perm[f] = pos;
    }
    __syncthreads();
    if (active && rank == cnt - 1) cur[e] += cnt;
    __syncthreads();
  }
}

// Routing with a shared expert: slot k of every token is expert E with
// weight 1; routed ids outside [0, E) become -1 so that they stay invalid
// (and are never taken for the shared expert E).
__global__ __launch_bounds__(256) void route_add_shared_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ w, int64_t T, int k, int E,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
  const int64_t n = T * (k + 1);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / (k + 1);
    const int j = (int)(i - t * (k + 1));
    if (j < k) {
      const int32_t id = ids[t * k + j];
      ids_out[i] = (id >= 0 && id < E) ? id : -1;
      w_out[i] = w[t * k + j];
    } else {
      ids_out[i] = E;
      w_out[i] = 1.0f;
    }
  }
}

}  // namespace

hipError_t launch_route_add_shared(const int32_t* ids, const float* w, int64_t T, int k, int E,
                                   int32_t* ids_out, float* w_out, hipStream_t stream) {
  const int64_t n = T * (k + 1);
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  route_add_shared_kernel<<<(unsigned)blocks, 256, 0, stream>>>(ids, w, T, k, E, ids_out, w_out);
  return hipGetLastError();
}

int64_t route_chunks(int64_t T, int k) {
  const int64_t M = T * k;
  const int64_t ch = chunk_size(M);
  return (M + ch - 1) / ch;
}

size_t route_ws_bytes(int64_t T, int k, int E) {
  const int64_t C = route_chunks(T, k);
  const int64_t n = (C > 0 ? C : 1) * (int64_t)(E + 1) + (E + 1);   // hist, then total
  return (size_t)n * sizeof(int32_t);
}

int64_t route_chunk(int64_t M) { return chunk_size(M); }

hipError_t launch_route_scatter(const int32_t* topk_ids, int64_t M, int E, void* ws,
                                int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                                int32_t* invalid_count, hipStream_t stream) {
  const int64_t ch = chunk_size(M);
  const int64_t C = (M + ch - 1) / ch;
  const int32_t* hist = static_cast<const int32_t*>(ws);
  const int32_t* total = hist + C * (int64_t)(E + 1);
  route_scatter_kernel<<<(unsigned)C, 64, (size_t)(E + 1) * sizeof(int32_t), stream>>>(
      topk_ids, M, ch, C, E, hist, total, offsets, invalid_count, perm, inv_perm);
  return hipGetLastError();
}

hipError_t launch_route(const int32_t* topk_ids, int64_t T, int k, int E, int32_t* offsets,
                        int32_t* perm, int32_t* inv_perm, int32_t* invalid_count, void* ws,
                        hipStream_t stream) {
  const int64_t M = T * k;
  const int64_t ch = chunk_size(M);
  const int64_t C = (M + ch - 1) / ch;
  if (C == 0) {                    // no pairs: every offset and the invalid count are 0
    fill_i32(offsets, 0, E + 1, stream);
    if (invalid_count != nullptr) fill_i32(invalid_count, 0, 1, stream);
    return hipGetLastError();
  }
  int32_t* hist = static_cast<int32_t*>(ws);
  int32_t* total = hist + C * (int64_t)(E + 1);
  const size_t lds_hist = (size_t)(E + 1) * sizeof(int32_t);
  route_hist_kernel<<<(unsigned)C, kHistThreads, lds_hist, stream>>>(topk_ids, M, ch, C, E, hist);
  route_scan_kernel<<<(unsigned)(E + 1), 64, 0, stream>>>(hist, C, total);
  return launch_route_scatter(topk_ids, M, E, ws, offsets, perm, inv_perm, invalid_count, stream);
}

}  // namespace nvfp4
