// Weight layout: per-group transpose to K-major, with the optional gate/up
// interleave at granularity 8 (gfx950).
//
// README "NVFP4 MegaMoE Kernel", "What We Have" (bridge layer): the L1 weight
// is interleaved gate/up at granularity 8 along N and B is made K-major;
// "Fused SwiGLU — How It Works": the interleaved output alternates eight gate
// columns with the eight matching up columns; "The //2 Bug": the granularity
// is 8, not 4.
//
// dst[g][n][r] = src[g][r][col(n)], col(n) = n without interleave, else
//   8*(n/16) + n%8 (gate, n%16 < 8) or I + 8*(n/16) + n%8 - 8 (up), I = cols/2.
// 64x64 tiles through LDS: coalesced 16-bit reads along src rows and writes
// along dst rows.
#include "internal.hpp"

namespace nvfp4 {

namespace {

constexpr int kTile = 64;

__device__ __forceinline__ int64_t src_col(int64_t n, int64_t cols, int interleave) {
  if (!interleave) return n;
  const int64_t half = cols / 2, grp = n / 16, pos = n % 16;
  return pos < 8 ? grp * 8 + pos : half + grp * 8 + pos - 8;
}

// block (64, 4): tile of 64 src rows x 64 dst rows
__global__ __launch_bounds__(256) void weight_layout_kernel(
    const uint16_t* __restrict__ src, int64_t rows, int64_t cols, int interleave,
    uint16_t* __restrict__ dst) {
  __shared__ uint16_t tile[kTile][kTile + 2];
  const int64_t g = blockIdx.z;
  const int64_t r0 = (int64_t)blockIdx.y * kTile;   // src row / dst col
  const int64_t n0 = (int64_t)blockIdx.x * kTile;   // dst row
  const uint16_t* s = src + g * rows * cols;
  uint16_t* d = dst + g * rows * cols;
  const int tx = threadIdx.x, ty = threadIdx.y;
  // read: thread tx walks dst rows n0+tx (i.e. src column col(n0+tx))
  for (int i = ty; i < kTile; i += 4) {
    const int64_t r = r0 + i, n = n0 + tx;
    if (r < rows && n < cols) tile[i][tx] = s[r * cols + src_col(n, cols, interleave)];
  }
  __syncthreads();
  for (int i = ty; i < kTile; i += 4) {
    const int64_t n = n0 + i, r = r0 + tx;
    if (n < cols && r < rows) d[n * rows + r] = tile[tx][i];
  }
}

__global__ void fill_f32_kernel(float* p, float v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void fill_i32_kernel(int32_t* p, int32_t v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_weight_layout(const void* src, int64_t groups, int64_t rows, int64_t cols,
                                int interleave, void* dst, hipStream_t stream) {
  if (groups == 0) return hipSuccess;
  dim3 grid((unsigned)((cols + kTile - 1) / kTile), (unsigned)((rows + kTile - 1) / kTile),
            (unsigned)groups);
  weight_layout_kernel<<<grid, dim3(kTile, 4), 0, stream>>>(
      static_cast<const uint16_t*>(src), rows, cols, interleave, static_cast<uint16_t*>(dst));
  return hipGetLastError();
}

void fill_f32(float* p, float v, int64_t n, hipStream_t stream) {
  if (n <= 0) return;
  fill_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(p, v, n);
}

void fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t stream) {
  if (n <= 0) return;
  fill_i32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(p, v, n);
}

}  // namespace nvfp4
