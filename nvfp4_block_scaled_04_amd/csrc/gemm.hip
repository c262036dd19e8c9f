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
// Tiling.  A block is 4 waves stacked along N (wave tile 128 N x 128 tokens,
// 4x4 MFMA blocks, 256 fp32 accumulators per lane); decoding is done per wave
// from packed codes in LDS, so each decoded element feeds 4 MFMAs.  Stages of
// 128 K go from HBM straight into LDS (buffer loads with the lds flag), triple-buffered.  An
// expert's rows are cut into ceil(rows/128) m tiles with its 32-row blocks
// spread evenly over them; column blocks past a tile's rows are skipped.
// Launches whose experts average at most 32 rows (decode-sized batches) use
// 32-token tiles instead: smaller stages, four buffers, loads three stages
// ahead, weights loaded with the non-temporal cache policy.
//
// MX mode.  The same tiles, loads and epilogues run on MXFP4 operands (E2M1
// codes, one E8M0 scale per 32 elements stored once per 16-element block, as
// written by the NVFP4 -> MX re-encoding): the codes in LDS go straight into
// v_mfma_scale_f32_32x32x64_f8f6f4 with the scales as its per-lane scale
// operands, with no decode step.  Lane half hf holds K chunk 2hf + h (32
// elements) of each row for MFMA h of a stage, whose E8M0 scale is byte 2h
// of the lane's scale dword (bytes 4hf..4hf+3 of the row's 8 stage bytes).
//
// Split K.  When the tile list is too short to occupy every CU (a dense
// linear of few rows), each tile's K stages are split into ksplit equal
// ranges run as separate work items; they write fp32 partials (already
// scaled by the global scales) to a caller workspace and a reduction kernel
// sums them in split order and rounds to BF16.
//
// Scheduling.  A persistent grid (one block per CU, a multiple of 8).  The
// tile list runs expert by expert and, inside an expert, n tile by n tile
// with the expert's m tiles innermost (device offsets, no host sync); XCD x
// owns a contiguous eighth of it, so the tiles that share a weight n tile run
// side by side in one L2, and its blocks claim tiles from a per-XCD counter,
// stealing from other XCDs' ranges at the end.  A block finds a tile's expert
// by a two-round 64-way search of a per-expert m-tile prefix kept in LDS.
#include <atomic>

#include "internal.hpp"
#include "device.hpp"

namespace nvfp4 {

namespace {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef int int8v __attribute__((ext_vector_type(8)));

constexpr int kFmtNvfp4 = 0;   // E4M3 per 16: decode to FP16, FP16 MFMA
constexpr int kFmtMx = 1;      // E8M0 per 32: scaled FP4 MFMA

constexpr int BK = 128;            // K elements per stage
constexpr int ROW_BYTES = BK / 2;  // 64 bytes of codes per row per stage
constexpr int ROW_STRIDE = 80;     // LDS row stride (64 + 16 pad: conflict-free b128 reads)
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
  int* sched;       // per-XCD tile counters (8), zero at launch
  int n_tiles;
  int ksplit;       // K ranges per tile (1: no split)
  int nks_total;    // K / BK
  float* partial;   // split K: fp32 [ksplit][M][N]
};

// epilogue of a split-K work item: fp32 partial sums (internal value)
constexpr int kEpiPartial = 2;

// 8 codes (one dword) -> 8 FP16 values times the block scale
__device__ __forceinline__ half8v decode8(uint32_t w, _Float16 s) {
  half2v sc;
  sc[0] = s;
  sc[1] = s;
  const half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sc;
  const half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sc;
  const half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sc;
  const half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sc;
  half8v r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// four E4M3 scale bytes -> four FP16 values (exact: E4M3 is a subset of FP16)
struct Scales4 {
  half2v lo, hi;
};
__device__ __forceinline__ _Float16 sget(const Scales4& s, int i) {
  return i == 0 ? s.lo[0] : i == 1 ? s.lo[1] : i == 2 ? s.hi[0] : s.hi[1];
}
__device__ __forceinline__ Scales4 scales4(uint32_t b) {
  Scales4 s;
  s.lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, false);
  s.hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, true);
  return s;
}

__device__ __forceinline__ uint32_t pick(const uint4& q, int i) {
  return i == 0 ? q.x : i == 1 ? q.y : i == 2 ? q.z : q.w;
}

// SwiGLU row order inside a 32-row weight group: MFMA row x = 8a+4b+j
// (a in 0..3, b in 0..1, j in 0..3) reads physical row 16b + 4(a/2) +
// 8(a%2) + j, so lane half b holds gate and up of h columns 8b..8b+7 of the
// group's 16-column h block (gate in accumulator rows 8a'+.., up 8 rows on).
__device__ __forceinline__ int swiglu_phys_row(int x) {
  const int a = x >> 3, b = (x >> 2) & 1, j = x & 3;
  return 16 * b + 4 * (a >> 1) + 8 * (a & 1) + j;
}

// LDS layout of one stage: ROWS rows of 64 code bytes (four 16-byte chunks,
// chunk q of row r stored at position q ^ ((r >> 2) & 3): conflict-free
// 16-byte reads for 16 consecutive rows), then ROWS rows of 8 scale bytes.
template <int BN, int BM, int WN, int WM>
struct Cfg {
  static constexpr int NT = WN * WM * 64;
  static constexpr int NW = WN * WM;
  static constexpr int TN = BN / WN, TM = BM / WM;     // wave tile
  static constexpr int FN = TN / 32, FM = TM / 32;     // 32x32 MFMA blocks per wave
  static constexpr int ROWS = BN + BM;                 // LDS rows per stage: weights, tokens
  static constexpr int CODE_BYTES = ROWS * ROW_BYTES;
  static constexpr int STAGE_BYTES = CODE_BYTES + ROWS * SF_BYTES;
  // 32-token tiles (experts of a few rows): smaller stages, so four buffers
  // fit and loads run three stages ahead instead of two.  Every wave still
  // issues 12 loads per stage: its token code loads move 4 bytes per lane
  // (two loads fill a wave's 8 of the 32 rows), and its one token scale load
  // brings all 32 rows' scales (every wave writes the same 256 bytes)
  static constexpr bool SMALL = BM == 32;
  // tiles of fewer than 32 token rows per wave (32- and 64-token tiles): every
  // wave loads all of the tile's token scales, 32 rows per 4-byte load, and
  // the waves write the same LDS bytes
  static constexpr bool TSF_SHARED = BM < 32 * NW;
  static constexpr int MAX_E = SMALL ? 1024 : 4096;    // expert prefix kept in LDS
  static constexpr int NBUF = SMALL ? 4 : 3;           // LDS stage buffers
  static constexpr int AHEAD = NBUF - 1;               // stages loaded ahead of use
  static constexpr int LDS_BYTES = NBUF * STAGE_BYTES;
  // direct-to-LDS loads per wave and stage: a code load fills 16 rows; a
  // weight scale load (16 bytes per lane) 128 rows, a token scale load 32 rows
  static constexpr int CODE_LOADS_W = BN / 16 / NW;    // weight-row code loads
  static constexpr int CODE_LOADS = SMALL ? CODE_LOADS_W + 2 : ROWS / 16 / NW;
  static constexpr int SF_LOADS_W = BN / 128 / NW;
  static constexpr int SF_LOADS_T = TSF_SHARED ? BM / 32 : BM / 32 / NW;
  static constexpr int SF_LOADS = SF_LOADS_W + SF_LOADS_T;
  static constexpr int LOADS = CODE_LOADS + SF_LOADS;
  static_assert(TN % 32 == 0 && TM % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(BN % (16 * NW) == 0 && (SMALL ? NW == 4 : ROWS % (16 * NW) == 0),
                "code loads must divide evenly");
  static_assert(BN % (128 * NW) == 0 && (TSF_SHARED || BM % (32 * NW) == 0), "scale loads must divide evenly");
  static_assert(CODE_LOADS + SF_LOADS_W + SF_LOADS_T == 12, "the vmcnt bookkeeping assumes 12 loads per stage");
  static_assert(BN == NVFP4_PACK_ROWS && BK == NVFP4_PACK_K, "tiles follow the packed weight layout");
  static_assert(WM == 1, "column-block skipping assumes one wave row");
};

__device__ __forceinline__ int chunk_pos(int row, int q) { return q ^ ((row >> 2) & 3); }

// step (0..5) of the K loop that issues stage load L (0..11): two per step
__host__ __device__ constexpr int load_step(int L) { return L / 2; }
// loads issued in steps 0..3, still in flight at the mid-stage wait
constexpr int kLoadsBeforeBarrier = 8;

// Per-lane state of a tile's K loop; every member lives in registers once the
// stage functions below are inlined.
template <int BN, int BM, int WN, int WM, int JV>
struct KState {
  using C = Cfg<BN, BM, WN, WM>;
  int wn, wm, hf, l32;
  float16v acc[C::FN][C::FM];
  uint4 fa[C::FN], ta[C::FM], fb[C::FN], tb[C::FM];  // half-stage code fragments
  uint32_t wsr[C::FN], tsr[C::FM];                   // scale bytes of the next stage
  Scales4 wsc[C::FN], tsc[C::FM];                    // scales of the current stage
  half8v av0[C::FN], bv0[C::FM], av1[C::FN], bv1[C::FM];   // decoded operands: even, odd steps
};

// Workgroup barrier without a memory fence.  The waits a stage needs are its
// own s_waitcnt; the empty asm statements stop the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct-to-LDS loads of stage ks into `dst`: all of them (part < 0) or those
// of K step `part`.  wq/wsf: this tile's packed weight codes/scales; aq/asf:
// token codes/scales; coff/soff: per-lane byte offsets of the wave's loads.
// The load counts and sizes come from plain constexpr ints (NVFP4_LOAD_CONSTS):
// the host pass rejects the load builtin when its arguments involve members
// of the dependent tile configuration.  kWPol is the weight loads' cache
// policy: non-temporal (2) for 32-token tiles, whose expert weights are
// streamed once (decode: forward 6.5% faster), the default for 128-token
// tiles, whose weight stages are shared through L2 by the expert's m tiles.
#define NVFP4_LOAD_CONSTS                                                                       \
  constexpr int kNW = C::NW, kCodeLoads = C::CODE_LOADS, kCodeLoadsW = C::CODE_LOADS_W;         \
  constexpr int kSfLoads = C::SF_LOADS, kSfLoadsW = C::SF_LOADS_W, kCodeBytes = C::CODE_BYTES;  \
  constexpr bool kSmall = C::SMALL, kTsfShared = C::TSF_SHARED;                                \
  constexpr int kWPol = C::SMALL ? 2 : 0
// A direct load of `size` bytes per lane from base + voff (per lane, 32 bits)
// + soff (uniform) into LDS at dst, through a raw buffer resource: the base
// stays in scalar registers and the per-lane offset in one VGPR, so no
// 64-bit per-lane address is formed or kept per load.  The resource spans
// the whole 32-bit offset range (the offsets are validated on the host).
typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const uint8_t* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, -1, 0x00020000);
}
// LDS pointer from a generic pointer into LDS by its low 32 bits (the LDS
// offset in the shared aperture): a plain address-space cast of a pointer
// selected among the stage buffers makes the compiler emit an aperture check
// it then rejects
__device__ __forceinline__ lds_ptr_t lds_addr(const uint8_t* p) {
  return (lds_ptr_t)(uint32_t)(uintptr_t)p;
}
#define NVFP4_BLOAD(rs, voff, soff, dst, size, pol)                                             \
  __builtin_amdgcn_raw_ptr_buffer_load_lds((rs), lds_addr(dst), (size), (int)(voff),          \
                                           (int)(soff), 0, (pol))
#define NVFP4_ISSUE(ks, dst, part)                                                              \
  do {                                                                                          \
    uint8_t* sbw = (dst);                                                                       \
    const __amdgpu_buffer_rsrc_t rw_ = raw_rsrc(wq), rws_ = raw_rsrc(wsf);                      \
    const __amdgpu_buffer_rsrc_t ra_ = raw_rsrc(aq), ras_ = raw_rsrc(asf);                      \
    _Pragma("unroll") for (int c = 0; c < kCodeLoads; ++c) {                                    \
      if ((part) < 0 || load_step(c) == (part)) {                                               \
        if (c < kCodeLoadsW)                                                                    \
          NVFP4_BLOAD(rw_, coff[c], (uint32_t)(ks) * (BN * ROW_BYTES),                          \
                      sbw + (c * kNW + wave) * 1024, 16, kWPol);                                \
        else if (kSmall)                                                                        \
          NVFP4_BLOAD(ra_, coff[c], (uint32_t)(ks) * ROW_BYTES,                                 \
                      sbw + BN * ROW_BYTES + ((c - kCodeLoadsW) * kNW + wave) * 256, 4, 0);     \
        else                                                                                    \
          NVFP4_BLOAD(ra_, coff[c], (uint32_t)(ks) * ROW_BYTES, sbw + (c * kNW + wave) * 1024,  \
                      16, 0);                                                                   \
      }                                                                                         \
    }                                                                                           \
    _Pragma("unroll") for (int c = 0; c < kSfLoads; ++c) {                                      \
      if ((part) < 0 || load_step(kCodeLoads + c) == (part)) {                                  \
        if (c < kSfLoadsW)                                                                      \
          NVFP4_BLOAD(rws_, soff[c], (uint32_t)(ks) * (BN * SF_BYTES),                          \
                      sbw + kCodeBytes + (c * kNW + wave) * 1024, 16, kWPol);                   \
        else if (kTsfShared)                                                                    \
          NVFP4_BLOAD(ras_, soff[c], (uint32_t)(ks) * SF_BYTES,                                 \
                      sbw + kCodeBytes + BN * SF_BYTES + (c - kSfLoadsW) * 256, 4, 0);          \
        else                                                                                    \
          NVFP4_BLOAD(ras_, soff[c], (uint32_t)(ks) * SF_BYTES,                                 \
                      sbw + kCodeBytes + BN * SF_BYTES + ((c - kSfLoadsW) * kNW + wave) * 256, \
                      4, 0);                                                                    \
      }                                                                                         \
    }                                                                                           \
  } while (0)

// fragment reads: half h (0 or 1) of every A and B block of the stage held
// in `src`: 16 contiguous code bytes per lane and block
#define NVFP4_READ_HALF(src, h, WA, TB)                                                         \
  do {                                                                                          \
    const uint8_t* sbr = (src);                                                                 \
    _Pragma("unroll") for (int i = 0; i < FN; ++i) {                                            \
      const int r = st.wn * TN + i * 32 + st.l32;                                               \
      WA[i] = *reinterpret_cast<const uint4*>(sbr + r * ROW_BYTES + 16 * chunk_pos(r, 2 * st.hf + (h))); \
    }                                                                                           \
    _Pragma("unroll") for (int j = 0; j < JV; ++j) {                                            \
      const int r = BN + st.wm * TM + j * 32 + st.l32;                                          \
      TB[j] = *reinterpret_cast<const uint4*>(sbr + r * ROW_BYTES + 16 * chunk_pos(r, 2 * st.hf + (h))); \
    }                                                                                           \
  } while (0)

#define NVFP4_READ_SF(src, WS, TS)                                                              \
  do {                                                                                          \
    const uint8_t* sbr = (src) + C::CODE_BYTES;                                                 \
    _Pragma("unroll") for (int i = 0; i < FN; ++i)                                              \
      WS[i] = *reinterpret_cast<const uint32_t*>(sbr + (st.wn * TN + i * 32 + st.l32) * SF_BYTES + st.hf * 4); \
    _Pragma("unroll") for (int j = 0; j < JV; ++j)                                              \
      TS[j] = *reinterpret_cast<const uint32_t*>(sbr + (BN + st.wm * TM + j * 32 + st.l32) * SF_BYTES + st.hf * 4); \
  } while (0)

// decode of one 16-deep K step: dword (s & 3) of the half fragments with
// scale byte (s >> 1); and the FN x JV MFMAs of a decoded step
#define NVFP4_DECODE(s, WA, TB, WSC, TSC, AV, BV)                                               \
  do {                                                                                          \
    _Pragma("unroll") for (int i = 0; i < FN; ++i)                                              \
      AV[i] = decode8(pick(WA[i], (s) & 3), sget(WSC[i], (s) >> 1));                            \
    _Pragma("unroll") for (int j = 0; j < JV; ++j)                                              \
      BV[j] = decode8(pick(TB[j], (s) & 3), sget(TSC[j], (s) >> 1));                            \
  } while (0)
#define NVFP4_MFMAS(AV, BV)                                                                     \
  do {                                                                                          \
    _Pragma("unroll") for (int i = 0; i < FN; ++i)                                              \
      _Pragma("unroll") for (int j = 0; j < JV; ++j)                                            \
        st.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(AV[i], BV[j], st.acc[i][j], 0, 0, 0); \
  } while (0)
// interleave: one MFMA of this step, then VPM VALU of the next step's decode;
// the step's NL stage loads go right after MFMAs spread over the step, so a
// load that waits to issue leaves the matrix pipe busy
#define NVFP4_INTERLEAVE(NL)                                                                    \
  do {                                                                                          \
    constexpr int nl_ = (NL);                                                                   \
    constexpr int every_ = nl_ > 0 ? (FN * JV + nl_ - 1) / (nl_ > 0 ? nl_ : 1) : 1;             \
    _Pragma("unroll") for (int q = 0; q < FN * JV; ++q) {                                       \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                        \
      if (nl_ > 0 && q % every_ == 0 && q / every_ < nl_)                                       \
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                                      \
      __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);                                      \
    }                                                                                           \
  } while (0)

// Direct loads of a tile's first AHEAD stages into buffers b0, b1 (, b2).  The
// pointer parameters are __restrict__ here and in k_stage: LDS reads of one
// buffer are then known not to alias direct loads into another, so the
// compiler adds no wait on loads in flight; every wait those reads need is
// an explicit s_waitcnt + barrier.  (That holds within one function: k_begin
// below cannot tell its reads of b0 from these loads into b1 and b2.)
template <int BN, int BM, int WN, int WM>
__device__ __forceinline__ void k_issue_first(int nks, int wave, const uint32_t* coff,
                                              const uint32_t* soff,
                                              const uint8_t* __restrict__ wq,
                                              const uint8_t* __restrict__ wsf,
                                              const uint8_t* __restrict__ aq,
                                              const uint8_t* __restrict__ asf,
                                              uint8_t* __restrict__ b0, uint8_t* __restrict__ b1,
                                              uint8_t* __restrict__ b2) {
  using C = Cfg<BN, BM, WN, WM>;
  NVFP4_LOAD_CONSTS;
  NVFP4_ISSUE(0, b0, -1);
  if (nks > 1) NVFP4_ISSUE(1, b1, -1);
  if (C::AHEAD > 2 && nks > 2) NVFP4_ISSUE(2, b2, -1);
}

// Waits for stage 0 (in b0; the tile's first stages are the last loads
// issued, later vector memory operations are stores), synchronises the
// block and decodes step 0.  32-token tiles issue their first AHEAD stages
// here, from the same __restrict__ parameters as the reads: with the loads
// issued in k_issue_first the compiler cannot tell the reads of b0 from the
// loads into b1 and b2 and waits for all three stages before the first
// read.  Decode-sized launches run many short tiles and lost that time at
// every tile start (decode L2 -1.2%, forward -0.7%, A/B).  Larger tiles keep
// the issue in k_issue_first, after the epilogue: moving it into k_begin
// made their SwiGLU epilogue spill, and prefill L1 ran 1% slower.
template <int BN, int BM, int WN, int WM, int JV>
__device__ __forceinline__ void k_begin(KState<BN, BM, WN, WM, JV>& st, int nks, int wave,
                                        const uint32_t* coff, const uint32_t* soff,
                                        const uint8_t* __restrict__ wq,
                                        const uint8_t* __restrict__ wsf,
                                        const uint8_t* __restrict__ aq,
                                        const uint8_t* __restrict__ asf,
                                        uint8_t* __restrict__ b0, uint8_t* __restrict__ b1,
                                        uint8_t* __restrict__ b2) {
  using C = Cfg<BN, BM, WN, WM>;
  constexpr int FN = C::FN, TN = C::TN, TM = C::TM;
  static_assert(C::LOADS == 12 && kLoadsBeforeBarrier == 8, "vmcnt immediates assume 12 loads per stage");
  NVFP4_LOAD_CONSTS;
  if constexpr (C::SMALL) {
    NVFP4_ISSUE(0, b0, -1);
    if (nks > 1) NVFP4_ISSUE(1, b1, -1);
    if (nks > 2) NVFP4_ISSUE(2, b2, -1);
  }
  if (C::AHEAD > 2 && nks > 2) asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
  else if (nks > 1) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  stage_barrier();
  NVFP4_READ_HALF(b0, 0, st.fa, st.ta);
  NVFP4_READ_SF(b0, st.wsr, st.tsr);
#pragma unroll
  for (int i = 0; i < FN; ++i) st.wsc[i] = scales4(st.wsr[i]);
#pragma unroll
  for (int j = 0; j < JV; ++j) st.tsc[j] = scales4(st.tsr[j]);
  NVFP4_DECODE(0, st.fa, st.ta, st.wsc, st.tsc, st.av0, st.bv0);
}

// One stage ks, held in br; stage ks+1 is in bm; with LOADS (a literal 1 or
// 0: whether stage ks+AHEAD exists) its loads go into bw; PEND: whether the
// loads of stage ks+2 are in flight (with AHEAD 2 those issued here).  LOADS
// stages have no branches, so the loads and the MFMAs share one scheduling
// region.  With AHEAD 3 (four buffers) read "ks+3" for "ks+2" below where
// the loads issued by this stage are meant; stage ks+2 then stays in flight
// across the mid-stage wait.
//   steps 0-3: half A fragments (in registers); half B fragments of stage ks
//     are read from LDS;
//   after step 3: wait until stage ks+1 has landed (the loads of ks+2 issued
//     so far may stay in flight), synchronise the block, read the half A
//     fragments and scales of stage ks+1;
//   steps 4-7: half B;
//   the loads of stage ks+2 (ks+3 with four buffers) are spread over
//   steps 0-5, two per step.
// Every step runs its MFMAs on operands decoded during the previous step
// while it decodes the next step's operands, so decode and MFMA overlap;
// step 7 decodes step 0 of the next stage.  bw held stage ks-1, last read
// before the mid-stage barrier of ks-1.
template <int BN, int BM, int WN, int WM, int JV, int LOADS, int PEND = LOADS>
__device__ __forceinline__ void k_stage(KState<BN, BM, WN, WM, JV>& st, int ks, int nks, int wave,
                                        const uint32_t* coff, const uint32_t* soff,
                                        const uint8_t* __restrict__ wq,
                                        const uint8_t* __restrict__ wsf,
                                        const uint8_t* __restrict__ aq,
                                        const uint8_t* __restrict__ asf,
                                        const uint8_t* __restrict__ br,
                                        const uint8_t* __restrict__ bm,
                                        uint8_t* __restrict__ bw) {
  using C = Cfg<BN, BM, WN, WM>;
  constexpr int FN = C::FN, TN = C::TN, TM = C::TM;
  NVFP4_LOAD_CONSTS;
  // VALU of one step's decode per MFMA of a step
  constexpr int VPM = ((FN + JV) * 8 + FN * JV - 1) / (FN * JV);
  constexpr int NL = LOADS ? 2 : 0;
  constexpr int AH = C::AHEAD;
  static_assert(AH == 2 || AH == 3, "two or three stages ahead");
  static_assert(AH == 3 || PEND == LOADS, "with two stages ahead the pending loads are this stage's");
  NVFP4_READ_HALF(br, 1, st.fb, st.tb);
  const bool more1 = LOADS || PEND || ks + 1 < nks;
  // operands of even steps live in av0/bv0, of odd steps in av1/bv1
  if (LOADS) NVFP4_ISSUE(ks + AH, bw, 0);
  NVFP4_DECODE(1, st.fa, st.ta, st.wsc, st.tsc, st.av1, st.bv1); NVFP4_MFMAS(st.av0, st.bv0); NVFP4_INTERLEAVE(NL);
  if (LOADS) NVFP4_ISSUE(ks + AH, bw, 1);
  NVFP4_DECODE(2, st.fa, st.ta, st.wsc, st.tsc, st.av0, st.bv0); NVFP4_MFMAS(st.av1, st.bv1); NVFP4_INTERLEAVE(NL);
  if (LOADS) NVFP4_ISSUE(ks + AH, bw, 2);
  NVFP4_DECODE(3, st.fa, st.ta, st.wsc, st.tsc, st.av1, st.bv1); NVFP4_MFMAS(st.av0, st.bv0); NVFP4_INTERLEAVE(NL);
  if (LOADS) NVFP4_ISSUE(ks + AH, bw, 3);
  NVFP4_DECODE(4, st.fb, st.tb, st.wsc, st.tsc, st.av0, st.bv0); NVFP4_MFMAS(st.av1, st.bv1); NVFP4_INTERLEAVE(NL);
  // stage ks+1 must have landed; the loads of ks+AH issued so far, and with
  // AH 3 those of stage ks+2, may not have
  if (AH == 2 && LOADS) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");   // kLoadsBeforeBarrier
  else if (AH == 3 && LOADS) asm volatile("s_waitcnt vmcnt(20)" ::: "memory");  // 12 + 8
  else if (AH == 3 && PEND) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  stage_barrier();
  if (more1) {
    NVFP4_READ_HALF(bm, 0, st.fa, st.ta);
    NVFP4_READ_SF(bm, st.wsr, st.tsr);
  }
  // the reads go out here; their consumers stay in the last step (below),
  // so their latency hides behind steps 4-6 instead of stalling issue
  __builtin_amdgcn_sched_barrier(0);
  if (LOADS) NVFP4_ISSUE(ks + AH, bw, 4);
  NVFP4_DECODE(5, st.fb, st.tb, st.wsc, st.tsc, st.av1, st.bv1); NVFP4_MFMAS(st.av0, st.bv0); NVFP4_INTERLEAVE(NL);
  if (LOADS) NVFP4_ISSUE(ks + AH, bw, 5);
  NVFP4_DECODE(6, st.fb, st.tb, st.wsc, st.tsc, st.av0, st.bv0); NVFP4_MFMAS(st.av1, st.bv1); NVFP4_INTERLEAVE(NL);
  NVFP4_DECODE(7, st.fb, st.tb, st.wsc, st.tsc, st.av1, st.bv1); NVFP4_MFMAS(st.av0, st.bv0); NVFP4_INTERLEAVE(0);
  __builtin_amdgcn_sched_barrier(0);
  if (more1) {
#pragma unroll
    for (int i = 0; i < FN; ++i) st.wsc[i] = scales4(st.wsr[i]);
#pragma unroll
    for (int j = 0; j < JV; ++j) st.tsc[j] = scales4(st.tsr[j]);
    NVFP4_DECODE(0, st.fa, st.ta, st.wsc, st.tsc, st.av0, st.bv0);
  }
  NVFP4_MFMAS(st.av1, st.bv1); NVFP4_INTERLEAVE(0);
}
// ---- MX mode: no decode; each stage is two sets of FN x JV scaled FP4
// MFMAs (K chunks 2hf and 2hf + 1 of the lane's row)
__device__ __forceinline__ int8v widen(const uint4& q) {
  int8v v;
  v[0] = (int)q.x; v[1] = (int)q.y; v[2] = (int)q.z; v[3] = (int)q.w;
  v[4] = 0; v[5] = 0; v[6] = 0; v[7] = 0;
  return v;
}
// OPSEL picks the scale byte of the lane's dword: 0 for K chunk 2hf, 2 for 2hf + 1
#define NVFP4_MFMAS_MX(WA, TB, WS, TS, OPSEL)                                                   \
  do {                                                                                          \
    _Pragma("unroll") for (int i = 0; i < FN; ++i)                                              \
      _Pragma("unroll") for (int j = 0; j < JV; ++j)                                            \
        st.acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                         \
            widen(WA[i]), widen(TB[j]), st.acc[i][j], 4, 4, OPSEL, (int)WS[i], OPSEL, (int)TS[j]); \
  } while (0)

// Waits for stage 0, synchronises the block and reads half 0 of its
// fragments and its scales.
template <int BN, int BM, int WN, int WM, int JV>
__device__ __forceinline__ void k_begin_mx(KState<BN, BM, WN, WM, JV>& st, int nks,
                                           const uint8_t* __restrict__ b0) {
  using C = Cfg<BN, BM, WN, WM>;
  constexpr int FN = C::FN, TN = C::TN, TM = C::TM;
  static_assert(C::LOADS == 12, "vmcnt immediates assume 12 loads per stage");
  if (nks > 1) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  stage_barrier();
  NVFP4_READ_HALF(b0, 0, st.fa, st.ta);
  NVFP4_READ_SF(b0, st.wsr, st.tsr);
}

// One MX stage ks (buffers as in k_stage):
//   issue all loads of stage ks+2 into bw (its last reader, stage ks-1,
//     finished before the mid-stage barrier of ks-1);
//   read half 1 of stage ks; MFMAs on half 0;
//   wait until stage ks+1 has landed and this wave's LDS reads are done,
//     synchronise the block;
//   read half 0 and the scales of stage ks+1 while the MFMAs on half 1 run.
template <int BN, int BM, int WN, int WM, int JV, int LOADS>
__device__ __forceinline__ void k_stage_mx(KState<BN, BM, WN, WM, JV>& st, int ks, int nks,
                                           int wave, const uint32_t* coff, const uint32_t* soff,
                                           const uint8_t* __restrict__ wq,
                                           const uint8_t* __restrict__ wsf,
                                           const uint8_t* __restrict__ aq,
                                           const uint8_t* __restrict__ asf,
                                           const uint8_t* __restrict__ br,
                                           const uint8_t* __restrict__ bm,
                                           uint8_t* __restrict__ bw) {
  using C = Cfg<BN, BM, WN, WM>;
  constexpr int FN = C::FN, TN = C::TN, TM = C::TM;
  NVFP4_LOAD_CONSTS;
  const bool more1 = LOADS || ks + 1 < nks;
  if (LOADS) NVFP4_ISSUE(ks + 2, bw, -1);
  NVFP4_READ_HALF(br, 1, st.fb, st.tb);
  NVFP4_MFMAS_MX(st.fa, st.ta, st.wsr, st.tsr, 0);
  if (LOADS) asm volatile("s_waitcnt vmcnt(12) lgkmcnt(0)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  stage_barrier();
  uint32_t wsn[C::FN], tsn[C::FM];
  if (more1) {
    NVFP4_READ_HALF(bm, 0, st.fa, st.ta);
    NVFP4_READ_SF(bm, wsn, tsn);
  }
  NVFP4_MFMAS_MX(st.fb, st.tb, st.wsr, st.tsr, 2);
  if (more1) {
#pragma unroll
    for (int i = 0; i < FN; ++i) st.wsr[i] = wsn[i];
#pragma unroll
    for (int j = 0; j < JV; ++j) st.tsr[j] = tsn[j];
  }
}
#undef NVFP4_MFMAS_MX

#undef NVFP4_ISSUE
#undef NVFP4_LOAD_CONSTS
#undef NVFP4_READ_HALF
#undef NVFP4_READ_SF
#undef NVFP4_DECODE
#undef NVFP4_MFMAS
#undef NVFP4_INTERLEAVE

// A tile: expert e, rows [row0, row0 + nrows) of the expert-ordered M
// dimension, weight rows [n0, n0 + BN), jv occupied 32-token column blocks.
struct Tile {
  int e, row0, nrows, jv;
  int64_t n0;
  int split, ks_lo, nks;   // K range [ks_lo, ks_lo + nks) in stages
};

// Lane index within the wave (0..63), recomputed wherever it is called: an
// asm statement with side effects is not hoisted out of a loop or merged
// with another call.
__device__ __forceinline__ int lane_index() {
  int lane;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  return lane;
}

// Wave-uniform read of a device array through the constant address space: a
// scalar load, counted by lgkmcnt.  A vector load here would be counted by
// vmcnt, which completes in order, so the compiler's wait for it would also
// wait for every direct load issued before it (the next tile's first
// stages).  Only for arrays the kernel never writes.
__device__ __forceinline__ float uniform_load(const float* p, int i) {
  return ((const __attribute__((address_space(4))) float*)p)[i];
}
__device__ __forceinline__ int uniform_load(const int32_t* p, int i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

// Tile number `logical` (< number of tiles) of the expert-ordered tile list
// (per expert: n tiles, and inside each n tile the expert's m tiles of BM
// rows, so the tiles that read one weight n tile are neighbours in the list
// and run side by side; split-K parts innermost).  tprefix: per-expert
// m-tile prefix (E <= 4096).  The fields are wave-uniform: readfirstlane
// keeps them in scalar registers.
template <int BN, int BM, bool LANE_ASM = false>
__device__ __forceinline__ void tile_at(const Params& p, const int* tprefix, int logical, Tile& t) {
  const int tix = logical / p.ksplit;
  const int split = logical - tix * p.ksplit;
  // expert e owns tiles [tprefix[e] * n_tiles, tprefix[e + 1] * n_tiles):
  // the largest e with tprefix[e] <= tix / n_tiles (fixed steps, no loop:
  // tprefix is non-decreasing and tprefix[0] = 0)
  const int mg = tix / p.n_tiles;
  // two wave-wide rounds of 64 tests (E <= 4096): lane l tests expert l*S
  // (S = ceil(E / 64)), then expert e0 + l; the lanes that pass form a prefix
  // (tprefix is non-decreasing), and lane 0 always passes
  int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  if constexpr (LANE_ASM) lane = lane_index();   // see run_tile
  const int S = (p.E + 63) >> 6;
  int c = lane * S;
  const int e0 = (__popcll(__ballot(c < p.E && tprefix[c] <= mg)) - 1) * S;
  c = e0 + lane;
  const int e = e0 + __popcll(__ballot(lane < S && c < p.E && tprefix[c] <= mg)) - 1;
  t.e = __builtin_amdgcn_readfirstlane(e);
  const int mcount = tprefix[t.e + 1] - tprefix[t.e];
  const int local = tix - tprefix[t.e] * p.n_tiles;
  const int nt = local / mcount;
  const int mt = local - nt * mcount;
  // The expert's 32-row blocks are spread evenly over its m tiles (at most
  // BM/32 each, the larger shares first): with 9 blocks the tiles take 3, 3, 3
  // rather than 4, 4, 1, since a one-block tile decodes the whole weight
  // tile for a quarter of the MFMAs and is VALU-bound.
  const int off_e = uniform_load(p.offsets, t.e), off_e1 = uniform_load(p.offsets, t.e + 1);
  const int rows_e = off_e1 - off_e;
  const int nblk = (rows_e + 31) / 32;
  const int per = nblk / mcount, rem = nblk - per * mcount;
  const int blk0 = mt * per + min(mt, rem);
  const int nblk_t = per + (mt < rem ? 1 : 0);
  t.row0 = __builtin_amdgcn_readfirstlane(off_e + 32 * blk0);
  t.nrows = __builtin_amdgcn_readfirstlane(min(32 * nblk_t, off_e1 - t.row0));
  t.n0 = (int64_t)__builtin_amdgcn_readfirstlane(nt) * BN;
  t.jv = (t.nrows + 31) / 32;
  t.split = __builtin_amdgcn_readfirstlane(split);
  t.ks_lo = __builtin_amdgcn_readfirstlane(split * p.nks_total / p.ksplit);
  t.nks = __builtin_amdgcn_readfirstlane((split + 1) * p.nks_total / p.ksplit) - t.ks_lo;
}

// Tile scheduling.  XCD x (blocks b with b % 8 == x) owns tiles
// [total*x/8, total*(x+1)/8), an eighth of the list, contiguous so that an
// expert's tiles share one L2; its blocks claim tiles dynamically from
// counter x.  The XCDs do not run at one clock, so a block whose range is
// exhausted steals from the other XCDs' counters.  Thread 0 of a block
// claims its next tile when the current tile enters its last two K stages
// (after the tile's last load is issued, so the claim only makes the
// remaining vmcnt waits stricter); the claim is published through LDS at the
// post-K-loop barrier, when every load has completed.  A tile therefore
// starts within about two stages and an epilogue of its claim, and the m
// tiles of one weight n tile, claimed one after another, stream that n tile
// nearly in step and share it through L2.
struct Sched {
  int64_t total;    // tiles in the list
  int* counters;    // eight per-XCD claim counters, zero at launch
  int* s_claim;     // LDS: [0] pending claim, [2] stolen tile, [3] its counter
  int cx;           // counter this block claims from (its XCD's first)
};

__device__ __forceinline__ int range_lo(int64_t total, int c) { return (int)((total * c) >> 3); }

// Tile index of claim k made on counter sc.cx, or -1 when every range is
// exhausted.  Every thread calls it with the same k; when sc.cx's range is
// exhausted wave 0 looks for another range with tiles left and the result
// is broadcast through LDS (one extra barrier, only at the end of a range).
// Lanes 1-7 read the other counters at once (agent-scope atomic loads; a
// counter only grows, so a stale value that shows its range exhausted is
// right), and thread 0 then claims, in order, only from ranges that looked
// open.  Claiming on every counter in turn took seven dependent atomics,
// about 15 us, at the end of every block's work (12% of a dense linear).
__device__ __forceinline__ int resolve_claim(Sched& sc, int k) {
  if (range_lo(sc.total, sc.cx) + k < range_lo(sc.total, sc.cx + 1))
    return range_lo(sc.total, sc.cx) + k;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int c = (sc.cx + lane) & 7;
    bool open = false;
    if (lane >= 1 && lane < 8) {
      const int cnt = __hip_atomic_load(sc.counters + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      open = range_lo(sc.total, c) + cnt < range_lo(sc.total, c + 1);
    }
    uint64_t cand = __ballot(open);
    if (lane == 0) {
      int t = -1, cc = sc.cx;
      while (cand != 0 && t < 0) {
        const int d = __builtin_ctzll(cand);   // next open range, in order from sc.cx
        cand &= cand - 1;
        cc = (sc.cx + d) & 7;
        const int kk = atomicAdd(sc.counters + cc, 1);
        if (range_lo(sc.total, cc) + kk < range_lo(sc.total, cc + 1)) t = range_lo(sc.total, cc) + kk;
      }
      sc.s_claim[2] = t;
      sc.s_claim[3] = cc;
    }
  }
  __syncthreads();
  sc.cx = __builtin_amdgcn_readfirstlane(sc.s_claim[3]);
  return __builtin_amdgcn_readfirstlane(sc.s_claim[2]);
}

// packed weights: tile (e, n0 / BN) is K/BK stages of BN rows (64 code bytes
// and 8 scale bytes per row), rows zero-padded to a multiple of BN; the
// pointers returned start at the tile's first K stage
template <int BN>
__device__ __forceinline__ const uint8_t* tile_wq(const Params& p, const Tile& t) {
  const int64_t Np = (p.N + BN - 1) / BN * BN;
  return p.b_q + ((int64_t)t.e * Np + t.n0) * (p.K / 2) + (int64_t)t.ks_lo * (BN * ROW_BYTES);
}
template <int BN>
__device__ __forceinline__ const uint8_t* tile_wsf(const Params& p, const Tile& t) {
  const int64_t Np = (p.N + BN - 1) / BN * BN;
  return p.b_sf + ((int64_t)t.e * Np + t.n0) * (p.K / 16) + (int64_t)t.ks_lo * (BN * SF_BYTES);
}
// token codes/scales from the tile's first K stage on (rows are added by the
// per-lane load offsets)
__device__ __forceinline__ const uint8_t* tile_aq(const Params& p, const Tile& t) {
  return p.a_q + (int64_t)t.ks_lo * ROW_BYTES;
}
__device__ __forceinline__ const uint8_t* tile_asf(const Params& p, const Tile& t) {
  return p.a_sf + (int64_t)t.ks_lo * SF_BYTES;
}

// Per-lane byte offsets (stage 0) of this wave's direct loads for tile t.
template <int BN, int BM, int WN, int WM, int EPI>
__device__ __forceinline__ void tile_offsets(const Params& p, const Tile& t, int wave, int lane,
                                             uint32_t* coff, uint32_t* soff) {
  using C = Cfg<BN, BM, WN, WM>;
  const uint32_t kb = (uint32_t)(p.K / 2), ksf = (uint32_t)(p.K / 16);
  // physical weight row (within the tile) held by LDS row r
  auto wrow = [&](int r) -> int {
    return (EPI == NVFP4_EPI_SWIGLU_NVFP4) ? ((r & ~31) | swiglu_phys_row(r & 31)) : r;
  };
  // token row of LDS row BN + i: clamped to the tile's last row, gathered.
  // SwiGLU launches (the ones that gather) read the gather index through a
  // buffer resource over the tile's own entries (based at row0, nrows
  // records; none when there is no gather, and an out-of-range buffer load
  // returns 0 and touches no memory), so the loads need no branch and go out
  // together: with a branch per row the compiler waited for each load in
  // turn.  Offsets stay below 512 bytes whatever M is.
  const bool gather = p.a_row_src != nullptr;
  const __amdgpu_buffer_rsrc_t grs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(gather ? p.a_row_src + t.row0 : nullptr), (short)0,
      EPI == NVFP4_EPI_SWIGLU_NVFP4 && gather ? t.nrows * 4 : 0, 0x00020000);
  auto trow = [&](int i) -> uint32_t {
    const int li = i < t.nrows ? i : t.nrows - 1;
    const int d = t.row0 + li;
    if constexpr (EPI == NVFP4_EPI_SWIGLU_NVFP4) {
      const int g = __builtin_amdgcn_raw_buffer_load_b32(grs, li * 4, 0, 0);
      // one select and one division for both cases, so no branch sinks the load
      return (uint32_t)((gather ? g : d) / (gather ? p.a_row_div : 1));
    } else {
      return (uint32_t)(gather ? p.a_row_src[d] / p.a_row_div : d);
    }
  };
#pragma unroll
  for (int c = 0; c < C::CODE_LOADS; ++c) {
    const int g = c * C::NW + wave;                // 16-row group
    const int r = 16 * g + (lane >> 2);
    const int q = chunk_pos(r, lane & 3);          // logical chunk stored at this lane's position
    if constexpr (C::SMALL) {
      if (c < C::CODE_LOADS_W) {
        coff[c] = (uint32_t)(wrow(r) * ROW_BYTES + 16 * q);
      } else {
        // 4 bytes per lane: token row i = 4 g' + lane / 16 (g' = the wave's
        // token load number), byte 4 (lane % 16) of its LDS row, i.e. byte
        // 4 (lane % 4) of the chunk at position (lane % 16) / 4
        const int i = 4 * ((c - C::CODE_LOADS_W) * C::NW + wave) + (lane >> 4);
        const int qs = chunk_pos(BN + i, (lane >> 2) & 3);
        coff[c] = trow(i) * kb + 16 * qs + 4 * (lane & 3);
      }
    } else {
      coff[c] = (c < C::CODE_LOADS_W) ? (uint32_t)(wrow(r) * ROW_BYTES + 16 * q)
                                      : trow(r - BN) * kb + 16 * q;
    }
  }
#pragma unroll
  for (int c = 0; c < C::SF_LOADS_W; ++c) {      // 2 consecutive rows per lane
    const int r = 128 * (c * C::NW + wave) + 2 * lane;
    soff[c] = (uint32_t)(wrow(r) * SF_BYTES);      // wrow(r + 1) == wrow(r) + 1 (r even)
  }
#pragma unroll
  for (int c = 0; c < C::SF_LOADS_T; ++c) {      // one 4-byte half row per lane
    const int i = C::TSF_SHARED ? 32 * c + (lane >> 1) : 32 * (c * C::NW + wave) + (lane >> 1);
    soff[C::SF_LOADS_W + c] = trow(i) * ksf + 4 * (lane & 1);
  }
}

// BF16 epilogue through LDS.  In the accumulator layout a lane holds one
// token row (l32) and 16 of the wave's N columns in four 8-byte pieces, so a
// direct store instruction writes 8-byte pieces of 32 different rows: 32
// partially written cache lines per instruction, and the address unit's time
// per line made these stores a tenth of the L2 GEMM.  Instead each 32-token
// column block is scaled, converted and written to a wave-private LDS region
// as 32 rows of the wave's TN columns, read back 16 bytes per lane along the
// rows and stored as whole row segments (a store instruction covers 4 rows of
// 2*TN contiguous bytes).  The region lies in the last stage buffer, which no
// load of the next tile targets before that tile's first stage barrier, so
// no block synchronisation is needed; rows past the tile's rows and columns
// past N are written to LDS but never stored.
constexpr int kEpiStride = 2 * 128 + 8;          // LDS bytes per staged row (TN = 128, 8 bytes pad)
constexpr int kEpiWaveBytes = 32 * kEpiStride;   // one 32-token column block of a wave

template <int TN, int FN, int FM, int JV>
__device__ __forceinline__ void epilogue_bf16(const Params& p, float16v (&acc)[FN][FM],
                                              float alpha, int row0, int nrows, int64_t nw0,
                                              int lane, uint8_t* __restrict__ ep) {
  static_assert(TN == 128 && FN == 4, "staging layout assumes a 128-column wave tile");
  const int hf = lane >> 5, l32 = lane & 31;
  const int64_t N = p.N;
  const int rr = lane >> 4, ch = lane & 15;      // read-back: row (of 4) and 16-byte chunk
  const bool col_ok = nw0 + 8 * ch < N;
#pragma unroll
  for (int j = 0; j < JV; ++j) {
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      // one 32 x 32 block at a time: the scheduler would otherwise copy all
      // accumulators out of the AGPRs at once and spill
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 o;
        o.x = pack_bf16x2(acc[i][j][4 * g + 0] * alpha, acc[i][j][4 * g + 1] * alpha);
        o.y = pack_bf16x2(acc[i][j][4 * g + 2] * alpha, acc[i][j][4 * g + 3] * alpha);
        *reinterpret_cast<uint2*>(ep + l32 * kEpiStride + 2 * (i * 32 + 8 * g + 4 * hf)) = o;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int tok = j * 32 + 4 * it + rr;
      const uint4 v = *reinterpret_cast<const uint4*>(ep + (4 * it + rr) * kEpiStride + 16 * ch);
      if (tok < nrows && col_ok)
        *reinterpret_cast<uint4*>(p.c_bf16 + (int64_t)(row0 + tok) * N + nw0 + 8 * ch) = v;
    }
  }
}

// One tile: the K loop and the epilogue.  JV = number of 32-token column
// blocks that hold rows (1..FM); the rest are skipped.  The tile's first
// AHEAD stages (0 and 1) were issued by the caller with the load offsets
// coff/soff; after the epilogue those of the next tile (if any) are issued,
// with coff/soff rewritten for it.  Issuing them before the epilogue would
// overlap their latency with it, but keeps the offsets and the next tile's
// bases live through the epilogue, whose spill reloads (vector loads,
// completing in order) then wait for those loads anyway; the later issue
// measured faster (prefill L1 -1.8%).  32-token tiles compute coff/soff and
// issue their first three stages at the start of the tile, in k_begin.
template <int BN, int BM, int WN, int WM, int EPI, int FMT, int JV>
__device__ __forceinline__ bool run_tile(const Params& p, uint8_t* smem, const int* tprefix,
                                         const float* rtab,
                                         Sched& sc, const Tile& cur, uint32_t* coff,
                                         uint32_t* soff, int& claim, Tile& nxt) {
  using C = Cfg<BN, BM, WN, WM>;
  constexpr int FN = C::FN, FM = C::FM, TN = C::TN, TM = C::TM;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // The BF16 128-token tiles take the lane index from an asm statement the
  // compiler cannot hoist out of the tile loop.  Derived from threadIdx.x,
  // it and the lane's LDS fragment addresses are computed once before the
  // loop, kept across every epilogue, spilled there and reloaded behind its
  // stores (L2 GEMM: 41 -> 8 scratch instructions, prefill L2 -1.2%).  The
  // SwiGLU tiles keep the plain index: there the change measured no gain.
  int lane = tid & 63;
  if constexpr (EPI == NVFP4_EPI_BF16 && BM == 128) lane = lane_index();
  const int wn = wave % WN, wm = wave / WN;
  const int hf = lane >> 5, l32 = lane & 31;
  const int64_t N = p.N, K = p.K;
  const int e = cur.e, row0 = cur.row0, nrows = cur.nrows;
  const int64_t n0 = cur.n0;
  const uint8_t* wbase = tile_wq<BN>(p, cur);
  const uint8_t* wsbase = tile_wsf<BN>(p, cur);
  const uint8_t* abase = tile_aq(p, cur);
  const uint8_t* asbase = tile_asf(p, cur);
  if constexpr (C::SMALL) tile_offsets<BN, BM, WN, WM, EPI>(p, cur, wave, lane, coff, soff);

  KState<BN, BM, WN, WM, JV> st;
  st.wn = wn; st.wm = wm; st.hf = hf; st.l32 = l32;
  {
    // zero accumulators from the matrix pipe, idle until the first stage has
    // landed: one MFMA of zero operands per block (0 * 0 + 0 = +0) instead of
    // 16 v_accvgpr_write each.  The zero operands come from asm, so the
    // compiler neither folds the products nor merges the 16 MFMAs into one
    half8v za[FN], zb[FM];
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      int z;
      asm volatile("v_mov_b32 %0, 0" : "=v"(z));
      za[i] = __builtin_bit_cast(half8v, make_int4(z, z, z, z));
    }
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      int z;
      asm volatile("v_mov_b32 %0, 0" : "=v"(z));
      zb[j] = __builtin_bit_cast(half8v, make_int4(z, z, z, z));
    }
    const float16v c0 = {};
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j)
        st.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(za[i], zb[j], c0, 0, 0, 0);
  }

  // three LDS stage buffers, stage ks in buffer ks % 3 (four with AHEAD 3)
  const int nks = cur.nks;
  if constexpr (FMT == kFmtMx) {
    k_begin_mx(st, nks, smem);
    int buf = 0;
    int ks = 0;
    for (; ks + 2 < nks; ++ks) {
      const int buf1 = buf == 2 ? 0 : buf + 1, buf2 = buf == 0 ? 2 : buf - 1;
      k_stage_mx<BN, BM, WN, WM, JV, 1>(st, ks, nks, wave, coff, soff, wbase, wsbase, abase,
                                        asbase, smem + buf * C::STAGE_BYTES,
                                        smem + buf1 * C::STAGE_BYTES, smem + buf2 * C::STAGE_BYTES);
      buf = buf1;
    }
    if (tid == 0) claim = atomicAdd(sc.counters + sc.cx, 1);
    for (; ks < nks; ++ks) {
      const int buf1 = buf == 2 ? 0 : buf + 1, buf2 = buf == 0 ? 2 : buf - 1;
      k_stage_mx<BN, BM, WN, WM, JV, 0>(st, ks, nks, wave, coff, soff, wbase, wsbase, abase,
                                        asbase, smem + buf * C::STAGE_BYTES,
                                        smem + buf1 * C::STAGE_BYTES, smem + buf2 * C::STAGE_BYTES);
      buf = buf1;
    }
  } else if constexpr (C::AHEAD == 3) {
    // four LDS stage buffers, stage ks in buffer ks % 4
    constexpr int SB = C::STAGE_BYTES;
    k_begin(st, nks, wave, coff, soff, wbase, wsbase, abase, asbase, smem, smem + SB, smem + 2 * SB);
    int ks = 0;
    for (; ks + 3 < nks; ++ks)
      k_stage<BN, BM, WN, WM, JV, 1, 1>(st, ks, nks, wave, coff, soff, wbase, wsbase, abase, asbase,
                                        smem + (ks & 3) * SB, smem + ((ks + 1) & 3) * SB,
                                        smem + ((ks + 3) & 3) * SB);
    if (ks + 2 < nks) {
      k_stage<BN, BM, WN, WM, JV, 0, 1>(st, ks, nks, wave, coff, soff, wbase, wsbase, abase, asbase,
                                        smem + (ks & 3) * SB, smem + ((ks + 1) & 3) * SB,
                                        smem + ((ks + 3) & 3) * SB);
      ++ks;
    }
    if (tid == 0) claim = atomicAdd(sc.counters + sc.cx, 1);
    for (; ks < nks; ++ks)
      k_stage<BN, BM, WN, WM, JV, 0, 0>(st, ks, nks, wave, coff, soff, wbase, wsbase, abase, asbase,
                                        smem + (ks & 3) * SB, smem + ((ks + 1) & 3) * SB,
                                        smem + ((ks + 3) & 3) * SB);
  } else {
    k_begin(st, nks, wave, coff, soff, wbase, wsbase, abase, asbase, smem,
            smem + C::STAGE_BYTES, smem + 2 * C::STAGE_BYTES);
    int buf = 0;
    int ks = 0;
    for (; ks + 2 < nks; ++ks) {
      const int buf1 = buf == 2 ? 0 : buf + 1, buf2 = buf == 0 ? 2 : buf - 1;
      k_stage<BN, BM, WN, WM, JV, 1>(st, ks, nks, wave, coff, soff, wbase, wsbase, abase, asbase,
                                     smem + buf * C::STAGE_BYTES, smem + buf1 * C::STAGE_BYTES,
                                     smem + buf2 * C::STAGE_BYTES);
      buf = buf1;
    }
    if (tid == 0) claim = atomicAdd(sc.counters + sc.cx, 1);
    for (; ks < nks; ++ks) {
      const int buf1 = buf == 2 ? 0 : buf + 1, buf2 = buf == 0 ? 2 : buf - 1;
      k_stage<BN, BM, WN, WM, JV, 0>(st, ks, nks, wave, coff, soff, wbase, wsbase, abase, asbase,
                                     smem + buf * C::STAGE_BYTES, smem + buf1 * C::STAGE_BYTES,
                                     smem + buf2 * C::STAGE_BYTES);
      buf = buf1;
    }
  }
  float16v (&acc)[FN][FM] = st.acc;
  // the last stage waited for every load, the pending claim included
  if (tid == 0) *sc.s_claim = claim;
  __syncthreads();   // every wave is done with the stage buffers
  // Lane index values for the code after the K loop, from an opaque copy:
  // the compiler cannot compute them (and their addresses) before the loop
  // and keep them live across it, which would spill.
  int lane_x = lane;
  asm volatile("" : "+v"(lane_x));
  const int t_next = resolve_claim(sc, __builtin_amdgcn_readfirstlane(*sc.s_claim));
  const bool has_next = t_next >= 0;
  if (has_next) tile_at<BN, BM, EPI == NVFP4_EPI_BF16 && BM == 128>(p, tprefix, t_next, nxt);
  {
  const int lane = lane_x, hf = lane_x >> 5, l32 = lane_x & 31;

  // ---- epilogue
  const float alpha = 1.0f / (uniform_load(p.gs_a, 0) *
                               uniform_load(p.gs_b, __builtin_amdgcn_readfirstlane(e)));
  if constexpr (EPI == kEpiPartial) {
    // fp32 partial sums of this K range: the lane's 4 contiguous columns of
    // each (i, g) as one 16-byte store; summed by splitk_reduce_kernel
    const int64_t nw0 = n0 + wn * TN;
#pragma unroll
    for (int j = 0; j < JV; ++j) {
      const int tok = j * 32 + l32;
      float* prow = p.partial + ((int64_t)cur.split * p.M + row0 + tok) * N + nw0 + 4 * hf;
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (tok >= nrows || nw0 + i * 32 >= N) continue;
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<float4*>(prow + i * 32 + 8 * g) =
              make_float4(acc[i][j][4 * g + 0] * alpha, acc[i][j][4 * g + 1] * alpha,
                          acc[i][j][4 * g + 2] * alpha, acc[i][j][4 * g + 3] * alpha);
      }
    }
  } else if constexpr (EPI == NVFP4_EPI_BF16) {
    static_assert(C::NW * kEpiWaveBytes <= C::STAGE_BYTES, "staged epilogue must fit a stage buffer");
    epilogue_bf16<C::TN, FN, FM, JV>(p, acc, alpha, row0, nrows, n0 + wn * TN, lane,
                                 smem + (C::NBUF - 1) * C::STAGE_BYTES + wave * kEpiWaveBytes);
  } else {
    const float gs_h = uniform_load(p.gs_out, 0);
    const int64_t I = N / 2;
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      // this 32-row N block is h block hb (16 h columns)
      const int64_t nb = n0 + wn * TN + i * 32;
      const int64_t hb = nb / 32;
#pragma unroll
      for (int j = 0; j < JV; ++j) {
        // one 32 x 32 block at a time (see the BF16 epilogue)
        __builtin_amdgcn_sched_barrier(0);
        const int tok = wm * TM + j * 32 + l32;
        float h[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int gi = (q < 4) ? q : 8 + (q - 4);      // gate register; up is gi + 4
          const float g = acc[i][j][gi] * alpha;
          const float u = acc[i][j][gi + 4] * alpha;
          // silu(g) * u; v_rcp_f32 (1 ulp) in place of an IEEE division
          h[q] = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
        }
        // block amax over 16 h columns: 8 in this lane, 8 in lane l^32
        float m = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(h[q]));
        const auto swp = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m),
                                                          false, false);
        const float amax = fmaxf(__uint_as_float(swp[0]), __uint_as_float(swp[1]));
        uint32_t codes, sfb;
        {
#pragma clang fp contract(off)
          const float a_s = amax * gs_h;
          const bool zero = amax == 0.0f || a_s < kUnderflow;
          // every lane encodes (a zeroed block gives r = inf and is replaced):
          // no branch inside the block's chain
          const float t = fminf(div6_rn(a_s), kE4m3Max);   // a_s < 6 * 2^-9 is zeroed below
          const uint32_t sb = e4m3_encode(t);
          const float r = rtab[sb];                       // gs_h / e4m3_decode(sb)
          // sign | E2M1(min(|h*r|, 6)); r > 0, so h*r has the sign of h
          const uint32_t c = e2m1_pack8(h[0] * r, h[1] * r, h[2] * r, h[3] * r, h[4] * r,
                                        h[5] * r, h[6] * r, h[7] * r);
          codes = zero ? 0u : c;
          sfb = zero ? 0u : sb;
        }
        if (tok >= nrows || nb >= N) continue;
        const int64_t d = row0 + tok;
        *reinterpret_cast<uint32_t*>(p.c_q + d * (I / 2) + hb * 8 + hf * 4) = codes;
        if (hf == 0) p.c_sf[d * (I / 16) + hb] = (uint8_t)sfb;
        if (p.c_debug != nullptr) {
          float4* dst = reinterpret_cast<float4*>(p.c_debug + d * I + hb * 16 + hf * 8);
          dst[0] = make_float4(h[0], h[1], h[2], h[3]);
          dst[1] = make_float4(h[4], h[5], h[6], h[7]);
        }
      }
    }
  }
  if (!C::SMALL && has_next) {
    tile_offsets<BN, BM, WN, WM, EPI>(p, nxt, wave, lane, coff, soff);
    k_issue_first<BN, BM, WN, WM>(nxt.nks, wave, coff, soff, tile_wq<BN>(p, nxt), tile_wsf<BN>(p, nxt),
                                  tile_aq(p, nxt), tile_asf(p, nxt), smem, smem + C::STAGE_BYTES,
                                  smem + 2 * C::STAGE_BYTES);
  }
  }
  return has_next;
}

template <int BN, int BM, int WN, int WM, int EPI, int FMT>
__global__ __launch_bounds__(WN * WM * 64, 1) void grouped_gemm_kernel(Params p) {
  using C = Cfg<BN, BM, WN, WM>;
  static_assert(!C::SMALL || FMT == kFmtNvfp4, "the MX stage assumes two stages ahead");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int* tprefix = reinterpret_cast<int*>(smem + C::LDS_BYTES);   // [E + 1]
  __shared__ int s_scan[C::NT];
  const int tid = threadIdx.x;

  // per-expert m-tile prefix (tiles of BM rows), once per block
  {
    const int E = p.E;
    const int per = (E + C::NT - 1) / C::NT;
    const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
    int local = 0;
    for (int e = e0; e < e1; ++e) local += (p.offsets[e + 1] - p.offsets[e] + BM - 1) / BM;
    s_scan[tid] = local;
    __syncthreads();
    for (int off = 1; off < C::NT; off <<= 1) {
      const int v = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += v;
      __syncthreads();
    }
    int acc = s_scan[tid] - local;
    for (int e = e0; e < e1; ++e) {
      tprefix[e] = acc;
      acc += (p.offsets[e + 1] - p.offsets[e] + BM - 1) / BM;
    }
    if (tid == C::NT - 1) tprefix[E] = s_scan[C::NT - 1];
    __syncthreads();
  }
  __shared__ int s_claim[4];
  // SwiGLU epilogue: gs_h / E4M3 value of every scale byte the requant can
  // produce (0..0x7E; 0 gives inf, selected away), one IEEE division each per
  // block instead of one per 16-column block and lane
  __shared__ float rtab[EPI == NVFP4_EPI_SWIGLU_NVFP4 ? 128 : 1];
  if constexpr (EPI == NVFP4_EPI_SWIGLU_NVFP4) {
    if (tid < 128) rtab[tid] = uniform_load(p.gs_out, 0) / e4m3_decode((uint32_t)tid);
  }
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  Sched sc;
  sc.total = (int64_t)tprefix[p.E] * p.n_tiles * p.ksplit;
  sc.counters = p.sched;
  sc.s_claim = s_claim;
  sc.cx = blockIdx.x & 7;                  // own XCD (blocks are dispatched round-robin)
  if (tid == 0) s_claim[0] = atomicAdd(sc.counters + sc.cx, 1);
  __syncthreads();
  const int t0 = resolve_claim(sc, __builtin_amdgcn_readfirstlane(s_claim[0]));
  bool have = t0 >= 0;
  int claim = 0;                           // pending claim, meaningful in thread 0 only
  Tile cur;
  uint32_t coff[C::CODE_LOADS], soff[C::SF_LOADS];
  if (have) {
    tile_at<BN, BM>(p, tprefix, t0, cur);
  }
  if (!C::SMALL && have) {
    tile_offsets<BN, BM, WN, WM, EPI>(p, cur, wave, lane, coff, soff);
    k_issue_first<BN, BM, WN, WM>(cur.nks, wave, coff, soff, tile_wq<BN>(p, cur), tile_wsf<BN>(p, cur),
                                  tile_aq(p, cur), tile_asf(p, cur), smem, smem + C::STAGE_BYTES,
                                  smem + 2 * C::STAGE_BYTES);
  }
  while (have) {
    Tile nxt;
    bool more = false;
    if (cur.jv >= C::FM) {
      more = run_tile<BN, BM, WN, WM, EPI, FMT, C::FM>(p, smem, tprefix, rtab, sc, cur, coff, soff, claim, nxt);
    } else if constexpr (C::FM > 1) {
      if (cur.jv == 1) more = run_tile<BN, BM, WN, WM, EPI, FMT, 1>(p, smem, tprefix, rtab, sc, cur, coff, soff, claim, nxt);
      else if constexpr (C::FM > 2) {
        if (cur.jv == 2) more = run_tile<BN, BM, WN, WM, EPI, FMT, 2>(p, smem, tprefix, rtab, sc, cur, coff, soff, claim, nxt);
        else if constexpr (C::FM > 3) more = run_tile<BN, BM, WN, WM, EPI, FMT, 3>(p, smem, tprefix, rtab, sc, cur, coff, soff, claim, nxt);
      }
    }
    cur = nxt;
    have = more;
  }
}

__global__ void zero_ints_kernel(int* p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0;
}

// c[d][n] = bf16_rne(sum over s in order of partial[s][d][n]) for the rows
// d < offsets[E] (the rows the GEMM defines); 8 columns per thread
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial,
                                                            int ksplit, int64_t M, int64_t N,
                                                            const int32_t* __restrict__ offsets,
                                                            int E, uint16_t* __restrict__ c) {
  const int64_t rows = offsets[E];
  const int64_t per_row = N / 8;
  const int64_t total = rows * per_row;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < total;
       v += (int64_t)gridDim.x * blockDim.x) {
    const int64_t off = v * 8;
    float4 lo = *reinterpret_cast<const float4*>(partial + off);
    float4 hi = *reinterpret_cast<const float4*>(partial + off + 4);
    for (int s = 1; s < ksplit; ++s) {
      const float4 a = *reinterpret_cast<const float4*>(partial + s * M * N + off);
      const float4 b = *reinterpret_cast<const float4*>(partial + s * M * N + off + 4);
      lo.x += a.x; lo.y += a.y; lo.z += a.z; lo.w += a.w;
      hi.x += b.x; hi.y += b.y; hi.z += b.z; hi.w += b.w;
    }
    uint4 o;
    o.x = pack_bf16x2(lo.x, lo.y);
    o.y = pack_bf16x2(lo.z, lo.w);
    o.z = pack_bf16x2(hi.x, hi.y);
    o.w = pack_bf16x2(hi.z, hi.w);
    *reinterpret_cast<uint4*>(c + off) = o;
  }
}

// Per-device launch facts, cached on first use with that device current:
// the CU count (grid size, split-K choice) and, per kernel instantiation,
// whether its dynamic LDS limit has been raised.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

hipError_t current_device(int& dev) {
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  return (dev >= 0 && dev < kMaxDevices) ? hipSuccess : hipErrorInvalidDevice;
}

hipError_t device_cus(int& cus) {
  int dev = 0;
  hipError_t err = current_device(dev);
  if (err != hipSuccess) return err;
  cus = g_cus[dev].load(std::memory_order_relaxed);
  if (cus > 0) return hipSuccess;
  err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  g_cus[dev].store(cus, std::memory_order_relaxed);
  return hipSuccess;
}

constexpr int kBN = 512, kBM = 128;   // the tile of every launch but small experts
constexpr int kBMSmall = 32;          // experts of at most 32 rows on average
constexpr int kBMMid = 64;            // BF16 launches whose 128-token tiles leave CUs idle

// upper bound on the tile count: sum over experts of ceil(rows_e / BM)
// <= (M + E * (BM - 1)) / BM m tiles, times the n tiles
int64_t tile_bound(int64_t M, int64_t N, int E, int bm = kBM) {
  return (M + (int64_t)E * (bm - 1)) / bm * ((N + kBN - 1) / kBN);
}

// K ranges per tile: 1, unless a BF16-epilogue launch has at most half as
// many tiles as the device has CUs; then enough ranges to cover the CUs, at
// most 4 and at least 4 K stages each
int splitk_factor(int epilogue, int64_t M, int64_t N, int64_t K, int E, int cus) {
  if (epilogue != NVFP4_EPI_BF16 || M == 0 || cus <= 0) return 1;
  // 64-token tiles come first: split only when even they leave half the
  // device idle
  if (2 * tile_bound(M, N, E, kBMMid) > cus) return 1;
  const int64_t tiles = tile_bound(M, N, E);
  if (2 * tiles > cus) return 1;
  int64_t f = cus / tiles;
  if (f > 4) f = 4;
  while (f > 1 && K / BK / f < 4) --f;
  return (int)f;
}

// fp32 partials follow the scheduler counters, 256-byte aligned
float* splitk_partial(void* ws) {
  const uintptr_t b = reinterpret_cast<uintptr_t>(ws) + kGemmWorkspaceBytes;
  return reinterpret_cast<float*>((b + 255) & ~uintptr_t(255));
}

template <int BN, int BM, int WN, int WM, int EPI, int FMT>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t stream) {
  using C = Cfg<BN, BM, WN, WM>;
  Params p;
  p.a_q = a.a_q; p.a_sf = a.a_sf; p.gs_a = a.gs_a; p.a_row_src = a.a_row_src;
  p.a_row_div = a.a_row_div; p.offsets = a.offsets; p.E = a.E; p.M = a.M; p.N = a.N; p.K = a.K;
  p.b_q = a.b_q; p.b_sf = a.b_sf; p.gs_b = a.gs_b; p.gs_out = a.gs_out;
  p.c_bf16 = static_cast<uint16_t*>(a.c_bf16); p.c_q = a.c_q; p.c_sf = a.c_sf; p.c_debug = a.c_debug;
  p.sched = static_cast<int*>(a.ws);
  p.n_tiles = (int)((a.N + BN - 1) / BN);
  p.nks_total = (int)(a.K / BK);
  p.ksplit = 1;
  p.partial = nullptr;
  if (a.M == 0) return hipSuccess;
  int dev = 0, cus = 0;
  hipError_t err = current_device(dev);
  if (err != hipSuccess) return err;
  err = device_cus(cus);
  if (err != hipSuccess) return err;
  if (EPI == kEpiPartial) {
    p.ksplit = splitk_factor(a.epilogue, a.M, a.N, a.K, a.E, cus);
    p.partial = splitk_partial(a.ws);
  }
  if (a.E > C::MAX_E) return hipErrorInvalidValue;
  const int64_t tiles = tile_bound(a.M, a.N, a.E, BM) * p.ksplit;
  int64_t grid = cus;                                     // one block per CU (LDS-limited)
  if (grid > tiles) grid = tiles;
  grid = (grid + 7) / 8 * 8;
  const size_t lds = (size_t)C::LDS_BYTES + sizeof(int) * (size_t)(a.E + 1);
  auto kern = grouped_gemm_kernel<BN, BM, WN, WM, EPI, FMT>;
  static std::atomic<bool> attr_set[kMaxDevices];
  if (!attr_set[dev].load(std::memory_order_relaxed)) {
    err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)(C::LDS_BYTES + sizeof(int) * (C::MAX_E + 1)));
    if (err != hipSuccess) return err;
    attr_set[dev].store(true, std::memory_order_relaxed);
  }
  if (a.clear_sched)
    zero_ints_kernel<<<1, 64, 0, stream>>>(p.sched, 8);   // a kernel, not a memset: graph-safe
  kern<<<(unsigned)grid, C::NT, lds, stream>>>(p);
  if (EPI == kEpiPartial) {
    const int64_t vecs = a.M * a.N / 8;
    int64_t blocks = (vecs + 255) / 256;
    if (blocks > 8 * (int64_t)cus) blocks = 8 * (int64_t)cus;
    splitk_reduce_kernel<<<(unsigned)blocks, 256, 0, stream>>>(
        p.partial, p.ksplit, a.M, a.N, a.offsets, a.E, static_cast<uint16_t*>(a.c_bf16));
  }
  return hipGetLastError();
}

}  // namespace

size_t gemm_splitk_ws_bytes(int epilogue, int64_t M, int64_t N, int64_t K, int E) {
  int cus = 0;
  if (device_cus(cus) != hipSuccess) return kGemmWorkspaceBytes;
  const int f = splitk_factor(epilogue, M, N, K, E, cus);
  if (f <= 1) return kGemmWorkspaceBytes;
  return kGemmWorkspaceBytes + 255 + (size_t)f * (size_t)M * (size_t)N * sizeof(float);
}

// 32-token tiles for NVFP4 launches whose experts hold at most 32 rows on
// average (decode-sized batches)
bool small_experts(int fmt, int64_t M, int E) {
  return fmt == kFmtNvfp4 && E <= Cfg<kBN, kBMSmall, 4, 1>::MAX_E && M <= (int64_t)kBMSmall * E;
}

template <int FMT>
hipError_t launch_fmt(const GemmArgs& a, hipStream_t stream) {
  constexpr int FS = FMT == kFmtNvfp4 ? kBMSmall : kBM;   // MX keeps the large tile
  const bool small = small_experts(FMT, a.M, a.E);
  if (a.epilogue == NVFP4_EPI_SWIGLU_NVFP4)
    return small ? launch_cfg<kBN, FS, 4, 1, NVFP4_EPI_SWIGLU_NVFP4, FMT>(a, stream)
                 : launch_cfg<kBN, kBM, 4, 1, NVFP4_EPI_SWIGLU_NVFP4, FMT>(a, stream);
  // split K only when the caller's workspace holds the partials
  if (a.M > 0 && a.ws_bytes > kGemmWorkspaceBytes &&
      gemm_splitk_ws_bytes(a.epilogue, a.M, a.N, a.K, a.E) > kGemmWorkspaceBytes &&
      a.ws_bytes >= gemm_splitk_ws_bytes(a.epilogue, a.M, a.N, a.K, a.E))
    return launch_cfg<kBN, kBM, 4, 1, kEpiPartial, FMT>(a, stream);
  if (small) return launch_cfg<kBN, FS, 4, 1, NVFP4_EPI_BF16, FMT>(a, stream);
  // 64-token tiles when the 128-token tile list would leave half the CUs idle
  // (a dense linear of a few thousand rows: 4096 x 2048 gives 128 tiles of
  // 128 x 512, 256 of 64 x 512)
  int cus = 0;
  const hipError_t err = device_cus(cus);
  if (err != hipSuccess) return err;
  if (a.M > 0 && 2 * tile_bound(a.M, a.N, a.E, kBM) <= cus)
    return launch_cfg<kBN, kBMMid, 4, 1, NVFP4_EPI_BF16, FMT>(a, stream);
  return launch_cfg<kBN, kBM, 4, 1, NVFP4_EPI_BF16, FMT>(a, stream);
}

hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t stream) {
  return a.mx ? launch_fmt<kFmtMx>(a, stream) : launch_fmt<kFmtNvfp4>(a, stream);
}

}  // namespace nvfp4
