// Expert-grouped NVFP4 GEMM with a BF16 epilogue or a fused SwiGLU + NVFP4
// requantisation epilogue (gfx950).
//
// README "NVFP4 MegaMoE Kernel":
//   "What We Have", grouped GEMM: A(M,K) x B(E,K,N) -> C(M,N), per-16 FP8
//     scales on A and B, per-expert global scales;
//   "Fused SwiGLU — How It Works": weight columns interleaved gate/up at
//     granularity 8, gate and up paired explicitly in registers;
//   "Remaining Steps" 2: NVFP4 quantise in the epilogue (per-16 amax, FP8
//     scale, FP4 pack) so the L2 input never exists in BF16.
//
// Arithmetic.  An NVFP4 operand element is E2M1 (2 significant bits) times
// its E4M3 block scale (4 significant bits): at most 6 significant bits and
// a magnitude in [2^-10, 2688], so FP16 holds it exactly.  Codes are decoded
// with v_cvt_scalef32_pk_f16_fp4 at scale 1 (the instruction honours only the
// exponent of its scale) and multiplied by the block scale in packed FP16,
// which is exact; the products go through v_mfma_f32_32x32x16_f16 with fp32
// accumulation.  The global scales are applied once in the epilogue:
// acc * 1/(gs_a * gs_b[e]).
//
// Orientation.  The weight's N rows are the MFMA "A" (row) operand and the
// token rows the "B" (column) operand.  In the 32x32 accumulator a lane holds
// one token and 16 of the 32 N rows; rows 8 apart sit in the same lane, so
// with the tile's weight rows placed in LDS in a fixed permutation, a lane
// holds gate and up of the same 8 h columns: SwiGLU needs no data movement,
// and the 16-wide h block amax needs one exchange with lane l^32.
//
// K order.  The MFMA's 16-deep K step is fed, for lane half hf = lane/32,
// from elements [64*hf + 8*s, +8) of a 128-wide K stage (step s = 0..7).  A
// and B use the same map, so the dot products are unchanged; each lane reads
// 32 contiguous bytes of codes per row and stage.
//
// Scheduling.  The grid walks (m tile, n tile) pairs; a block finds its
// expert by scanning the device-side expert offsets (no host sync).  Rows
// past an expert's count read a clamped valid row and are not stored.
#include "internal.hpp"
#include "device.hpp"

namespace nvfp4 {

namespace {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int BK = 128;          // K elements per stage
constexpr int ROW_BYTES = BK / 2;  // 64 bytes of codes per row per stage
constexpr int ROW_STRIDE = 80;   // LDS row stride (64 + 16 pad: conflict-free b128 reads)
constexpr int SF_BYTES = BK / 16;  // 8 scale bytes per row per stage

struct Params {
  const uint8_t* a_q;
  const uint8_t* a_sf;
  const float* gs_a;
  const int32_t* a_row_src;
  int a_row_div;
  const int32_t* offsets;
  int E;
  int64_t M, N, K;
  const uint8_t* b_q;
  const uint8_t* b_sf;
  const float* gs_b;
  const float* gs_out;
  uint16_t* c_bf16;
  uint8_t* c_q;
  uint8_t* c_sf;
  float* c_debug;
  int n_tiles;
};

// decoded value pairs of 8 codes (one dword) times the block scale pair
__device__ __forceinline__ half8v decode8(uint32_t w, half2v sc) {
  half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sc;
  half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sc;
  half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sc;
  half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sc;
  half8v r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ half2v scale_pair(uint32_t bytes4, int sel) {
  float f;
  switch (sel) {
    case 0: f = __builtin_amdgcn_cvt_f32_fp8(bytes4, 0); break;
    case 1: f = __builtin_amdgcn_cvt_f32_fp8(bytes4, 1); break;
    case 2: f = __builtin_amdgcn_cvt_f32_fp8(bytes4, 2); break;
    default: f = __builtin_amdgcn_cvt_f32_fp8(bytes4, 3); break;
  }
  const _Float16 h = (_Float16)f;   // exact: every E4M3 value is an FP16 value
  half2v r;
  r[0] = h; r[1] = h;
  return r;
}

// LDS row of physical weight row q (0..31) of a 32-row group for SwiGLU:
// MFMA row 8a+4b+j (a in 0..3, b in 0..1, j in 0..3) reads physical row
// 16b + 4(a/2) + 8(a%2) + j, so lane half b holds gate/up of h columns
// 8b..8b+7 of the group's 16-column h block.
__device__ __forceinline__ int swiglu_lds_row(int q) {
  const int b = q >> 4, rem = q & 15;
  const int a = 2 * ((rem & 7) >> 2) + (rem >> 3);
  return 8 * a + 4 * b + (rem & 3);
}

// Block-wide search of the expert owning m tile `tile`: experts are split in
// contiguous ranges over the threads, range sums of ceil(count/BM) are
// scanned in LDS, and the owning thread walks its range.  Writes e = -1 when
// tile is past the last tile.
template <int NT, int BM>
__device__ __forceinline__ void find_tile(const int32_t* offsets, int E, int tile, int* scan,
                                          int& s_expert, int& s_row0, int& s_rows) {
  const int tid = threadIdx.x;
  const int per = (E + NT - 1) / NT;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int local = 0;
  for (int e = e0; e < e1; ++e) local += (offsets[e + 1] - offsets[e] + BM - 1) / BM;
  scan[tid] = local;
  if (tid == 0) s_expert = -1;
  __syncthreads();
  for (int off = 1; off < NT; off <<= 1) {
    const int v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  int acc = scan[tid] - local;
  if (tile >= acc && tile < acc + local) {
    for (int e = e0; e < e1; ++e) {
      const int c = offsets[e + 1] - offsets[e];
      const int t = (c + BM - 1) / BM;
      if (tile < acc + t) {
        s_expert = e;
        s_row0 = offsets[e] + (tile - acc) * BM;
        s_rows = min(BM, offsets[e + 1] - s_row0);
        break;
      }
      acc += t;
    }
  }
  __syncthreads();
}

template <int BN, int BM, int WN, int WM, int EPI>
__global__ __launch_bounds__(WN * WM * 64) void grouped_gemm_kernel(Params p) {
  constexpr int NT = WN * WM * 64;
  constexpr int TN = BN / WN, TM = BM / WM;    // wave tile
  constexpr int FN = TN / 32, FM = TM / 32;    // 32x32 MFMA blocks per wave
  constexpr int ROWS = BN + BM;                // LDS rows per stage (weights then tokens)
  constexpr int CODE_BYTES = ROWS * ROW_STRIDE;
  constexpr int STAGE_BYTES = CODE_BYTES + ROWS * SF_BYTES;
  constexpr int CHUNKS = ROWS * 4;             // 16-byte code chunks per stage
  constexpr int CPT = (CHUNKS + NT - 1) / NT;  // chunks per thread
  constexpr int SPT = (ROWS + NT - 1) / NT;    // scale rows per thread
  static_assert(TN % 32 == 0 && TM % 32 == 0, "wave tile must be a multiple of 32");

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_expert, s_row0, s_rows;
  __shared__ int s_scan[NT];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wn = wave % WN, wm = wave / WN;

  // ---- which expert / m tile is this block? (prefix of ceil(count/BM))
  const int tile = blockIdx.x / p.n_tiles;
  const int ntile = blockIdx.x % p.n_tiles;
  find_tile<NT, BM>(p.offsets, p.E, tile, s_scan, s_expert, s_row0, s_rows);
  const int e = s_expert;
  if (e < 0) return;
  const int row0 = s_row0, nrows = s_rows;
  const int64_t n0 = (int64_t)ntile * BN;
  const int64_t K = p.K;
  const int64_t kb = K / 2, ksf = K / 16;

  // ---- global source rows of this thread's chunks (weights, then tokens)
  const uint8_t* src_code[CPT];
  const uint8_t* src_sf[SPT];
  int lds_code[CPT], lds_sf[SPT];
  bool has_code[CPT], has_sf[SPT];
  auto row_ptrs = [&](int r, const uint8_t*& code, const uint8_t*& sf, int& lrow) {
    if (r < BN) {
      int64_t n = n0 + r;
      if (n >= p.N) n = p.N - 1;
      code = p.b_q + ((int64_t)e * p.N + n) * kb;
      sf = p.b_sf + ((int64_t)e * p.N + n) * ksf;
      lrow = (EPI == NVFP4_EPI_SWIGLU_NVFP4) ? ((r & ~31) | swiglu_lds_row(r & 31)) : r;
    } else {
      const int i = r - BN;
      int d = row0 + (i < nrows ? i : nrows - 1);
      int64_t arow = p.a_row_src ? (int64_t)(p.a_row_src[d] / p.a_row_div) : (int64_t)d;
      code = p.a_q + arow * kb;
      sf = p.a_sf + arow * ksf;
      lrow = r;
    }
  };
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int chunk = tid + c * NT;
    has_code[c] = chunk < CHUNKS;
    const int r = has_code[c] ? chunk >> 2 : 0;
    const uint8_t* sfp;
    int lrow;
    row_ptrs(r, src_code[c], sfp, lrow);
    src_code[c] += (chunk & 3) * 16;
    lds_code[c] = lrow * ROW_STRIDE + (chunk & 3) * 16;
  }
#pragma unroll
  for (int c = 0; c < SPT; ++c) {
    const int r0 = tid + c * NT;
    has_sf[c] = r0 < ROWS;
    const uint8_t* cp;
    int lrow;
    row_ptrs(has_sf[c] ? r0 : 0, cp, src_sf[c], lrow);
    lds_sf[c] = CODE_BYTES + lrow * SF_BYTES;
  }

  uint4 stage_code[CPT];
  uint2 stage_sf[SPT];
  auto gload = [&](int ks) {
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      if (has_code[c]) stage_code[c] = *reinterpret_cast<const uint4*>(src_code[c] + ks * ROW_BYTES);
#pragma unroll
    for (int c = 0; c < SPT; ++c)
      if (has_sf[c]) stage_sf[c] = *reinterpret_cast<const uint2*>(src_sf[c] + ks * SF_BYTES);
  };
  auto lstore = [&](int buf) {
    uint8_t* base = smem + buf * STAGE_BYTES;
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      if (has_code[c]) *reinterpret_cast<uint4*>(base + lds_code[c]) = stage_code[c];
#pragma unroll
    for (int c = 0; c < SPT; ++c)
      if (has_sf[c]) *reinterpret_cast<uint2*>(base + lds_sf[c]) = stage_sf[c];
  };

  float16v acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int hf = lane >> 5, l32 = lane & 31;
  const int nks = (int)(K / BK);
  gload(0);
  lstore(0);
  __syncthreads();

  for (int ks = 0; ks < nks; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nks) gload(ks + 1);
    const uint8_t* base = smem + buf * STAGE_BYTES;
    // fragments: 32 bytes of codes + 4 scale bytes per 32-row block per lane
    uint4 wa[FN][2], tb[FM][2];
    uint32_t wsf[FN], tsf[FM];
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const int r = wn * TN + i * 32 + l32;
      wa[i][0] = *reinterpret_cast<const uint4*>(base + r * ROW_STRIDE + hf * 32);
      wa[i][1] = *reinterpret_cast<const uint4*>(base + r * ROW_STRIDE + hf * 32 + 16);
      wsf[i] = *reinterpret_cast<const uint32_t*>(base + CODE_BYTES + r * SF_BYTES + hf * 4);
    }
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int r = BN + wm * TM + j * 32 + l32;
      tb[j][0] = *reinterpret_cast<const uint4*>(base + r * ROW_STRIDE + hf * 32);
      tb[j][1] = *reinterpret_cast<const uint4*>(base + r * ROW_STRIDE + hf * 32 + 16);
      tsf[j] = *reinterpret_cast<const uint32_t*>(base + CODE_BYTES + r * SF_BYTES + hf * 4);
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      half8v av[FN], bv[FM];
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const uint4& q = wa[i][s >> 2];
        const uint32_t w = (s & 3) == 0 ? q.x : (s & 3) == 1 ? q.y : (s & 3) == 2 ? q.z : q.w;
        av[i] = decode8(w, scale_pair(wsf[i], s >> 1));
      }
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const uint4& q = tb[j][s >> 2];
        const uint32_t w = (s & 3) == 0 ? q.x : (s & 3) == 1 ? q.y : (s & 3) == 2 ? q.z : q.w;
        bv[j] = decode8(w, scale_pair(tsf[j], s >> 1));
      }
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if (ks + 1 < nks) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  const float alpha = 1.0f / (p.gs_a[0] * p.gs_b[e]);
  if constexpr (EPI == NVFP4_EPI_BF16) {
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int tok = wm * TM + j * 32 + l32;
        if (tok >= nrows) continue;
        const int64_t d = row0 + tok;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t n = n0 + wn * TN + i * 32 + 8 * g + 4 * hf;
          if (n >= p.N) continue;
          uint2 o;
          o.x = f32_to_bf16_rne(acc[i][j][4 * g + 0] * alpha) |
                (f32_to_bf16_rne(acc[i][j][4 * g + 1] * alpha) << 16);
          o.y = f32_to_bf16_rne(acc[i][j][4 * g + 2] * alpha) |
                (f32_to_bf16_rne(acc[i][j][4 * g + 3] * alpha) << 16);
          *reinterpret_cast<uint2*>(p.c_bf16 + d * p.N + n) = o;
        }
      }
  } else {
    const float gs_h = p.gs_out[0];
    const int64_t I = p.N / 2;
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      // this 32-row N block is h block hb = (n0 + wn*TN + 32 i) / 32
      const int64_t nb = n0 + wn * TN + i * 32;
      const int64_t hb = nb / 32;
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int tok = wm * TM + j * 32 + l32;
        float h[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int gi = (q < 4) ? q : 8 + (q - 4);      // gate register
          const float g = acc[i][j][gi] * alpha;
          const float u = acc[i][j][gi + 4] * alpha;
          h[q] = (g / (1.0f + __expf(-g))) * u;
        }
        // block amax over 16 h columns: 8 here, 8 in lane l^32
        float m = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(h[q]));
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m),
                                                         false, false);
        const float amax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        if (tok >= nrows || nb >= p.N) continue;
        const int64_t d = row0 + tok;
        uint32_t codes = 0, sfb = 0;
        {
#pragma clang fp contract(off)
          const float a_s = amax * gs_h;
          if (!(amax == 0.0f || a_s < kUnderflow)) {
            const float t = fminf(a_s / 6.0f, kE4m3Max);
            sfb = e4m3_encode(t);
            const float r = gs_h / e4m3_decode(sfb);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const float v = fminf(fabsf(h[q] * r), 6.0f);
              const uint32_t c = e2m1_encode(v) | ((__float_as_uint(h[q]) >> 31) << 3);
              codes |= c << (4 * q);
            }
          }
        }
        *reinterpret_cast<uint32_t*>(p.c_q + d * (I / 2) + hb * 8 + hf * 4) = codes;
        if (hf == 0) p.c_sf[d * (I / 16) + hb] = (uint8_t)sfb;
        if (p.c_debug != nullptr) {
          float* dst = p.c_debug + d * I + hb * 16 + hf * 8;
#pragma unroll
          for (int q = 0; q < 8; ++q) dst[q] = h[q];
        }
      }
    }
  }
}

template <int BN, int BM, int WN, int WM, int EPI>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t stream) {
  Params p;
  p.a_q = a.a_q; p.a_sf = a.a_sf; p.gs_a = a.gs_a; p.a_row_src = a.a_row_src;
  p.a_row_div = a.a_row_div; p.offsets = a.offsets; p.E = a.E; p.M = a.M; p.N = a.N; p.K = a.K;
  p.b_q = a.b_q; p.b_sf = a.b_sf; p.gs_b = a.gs_b; p.gs_out = a.gs_out;
  p.c_bf16 = static_cast<uint16_t*>(a.c_bf16); p.c_q = a.c_q; p.c_sf = a.c_sf; p.c_debug = a.c_debug;
  p.n_tiles = (int)((a.N + BN - 1) / BN);
  const int64_t m_tiles = (a.M + BM - 1) / BM + a.E;   // upper bound on sum ceil(count/BM)
  const int64_t blocks = m_tiles * p.n_tiles;
  if (a.M == 0 || blocks == 0) return hipSuccess;
  constexpr int ROWS = BN + BM;
  constexpr size_t lds = 2 * (size_t)(ROWS * ROW_STRIDE + ROWS * SF_BYTES);
  auto kern = grouped_gemm_kernel<BN, BM, WN, WM, EPI>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  kern<<<(unsigned)blocks, WN * WM * 64, lds, stream>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t stream) {
  if (a.epilogue == NVFP4_EPI_SWIGLU_NVFP4) return launch_cfg<128, 128, 2, 2, NVFP4_EPI_SWIGLU_NVFP4>(a, stream);
  return launch_cfg<128, 128, 2, 2, NVFP4_EPI_BF16>(a, stream);
}

}  // namespace nvfp4
