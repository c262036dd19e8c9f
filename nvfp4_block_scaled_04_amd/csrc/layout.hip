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

// One thread per (expert, padded row, K stage): 64 code bytes and 8 scale
// bytes from the row-major weight to the stage-tiled layout (zeros for rows
// past N).
__global__ __launch_bounds__(256) void pack_weights_kernel(
    const uint4* __restrict__ q, const uint2* __restrict__ sf, int64_t N, int64_t Np, int64_t S,
    int64_t total, uint4* __restrict__ qp, uint2* __restrict__ sfp) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  // i enumerates the destination: ((e * T + t) * S + s) * ROWS + r
  const int64_t r = i % NVFP4_PACK_ROWS;
  const int64_t rest = i / NVFP4_PACK_ROWS;
  const int64_t s = rest % S;
  const int64_t et = rest / S;
  const int64_t tiles = Np / NVFP4_PACK_ROWS;
  const int64_t t = et % tiles, e = et / tiles;
  const int64_t n = t * NVFP4_PACK_ROWS + r;
  uint4 c0 = make_uint4(0, 0, 0, 0), c1 = c0, c2 = c0, c3 = c0;
  uint2 sc = make_uint2(0, 0);
  if (n < N) {
    const uint4* src = q + ((e * N + n) * S + s) * 4;       // 64 bytes = 4 x 16
    c0 = src[0]; c1 = src[1]; c2 = src[2]; c3 = src[3];
    sc = sf[(e * N + n) * S + s];
  }
  uint4* dst = qp + i * 4;
  dst[0] = c0; dst[1] = c1; dst[2] = c2; dst[3] = c3;
  sfp[i] = sc;
}

}  // namespace

int64_t packed_rows(int64_t N) { return (N + NVFP4_PACK_ROWS - 1) / NVFP4_PACK_ROWS * NVFP4_PACK_ROWS; }

hipError_t launch_pack_weights(const uint8_t* q, const uint8_t* sf, int64_t E, int64_t N, int64_t K,
                               uint8_t* qp, uint8_t* sfp, hipStream_t stream) {
  const int64_t Np = packed_rows(N), S = K / NVFP4_PACK_K;
  const int64_t total = E * Np * S;
  if (total == 0) return hipSuccess;
  pack_weights_kernel<<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(
      reinterpret_cast<const uint4*>(q), reinterpret_cast<const uint2*>(sf), N, Np, S, total,
      reinterpret_cast<uint4*>(qp), reinterpret_cast<uint2*>(sfp));
  return hipGetLastError();
}

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
