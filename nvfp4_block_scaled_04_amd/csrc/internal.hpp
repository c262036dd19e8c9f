// Internal launch interface between the C ABI (api.hip) and the kernels.
// Every launch_* enqueues on `stream`, allocates nothing and assumes its
// arguments were validated by the caller.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "nvfp4moe.h"

namespace nvfp4 {

// small utility kernels (layout.hip); fills instead of hipMemsetAsync so the
// sequence stays correct under hipGraph replay
void fill_f32(float* p, float v, int64_t n, hipStream_t stream);
void fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t stream);

// quantize.hip
int quantize_parts(int64_t groups, int64_t rows_per_group, int64_t cols);
// x rows are ld_x bf16 elements apart (ld_x >= cols, ld_x % 8 == 0)
hipError_t launch_quantize(const void* x, int64_t groups, int64_t rows_per_group, int64_t cols,
                           int64_t ld_x, const float* gs_in, uint8_t* q, uint8_t* sf,
                           float* gs_out, float* ws, hipStream_t stream);

// x (T, H) -> NVFP4 with a per-call global scale, each token row written to
// its k expert-order rows (inv_perm), rows >= offsets[E] skipped
hipError_t launch_quantize_scatter(const void* x, int64_t T, int64_t H, int k,
                                   const int32_t* inv_perm, const int32_t* offsets, int E,
                                   uint8_t* q, uint8_t* sf, float* gs_out, float* ws,
                                   hipStream_t stream);

// route.hip
int64_t route_chunks(int64_t T, int k);
int64_t route_chunk(int64_t M);   // entries per chunk for M routed pairs
size_t route_ws_bytes(int64_t T, int k, int E);
hipError_t launch_route(const int32_t* topk_ids, int64_t T, int k, int E, int32_t* offsets,
                        int32_t* perm, int32_t* inv_perm, int32_t* invalid_count, void* ws,
                        hipStream_t stream);
// the last routing launch alone: ws holds the scanned histogram and the
// bucket totals (route_ws_bytes layout); M > 0
hipError_t launch_route_scatter(const int32_t* topk_ids, int64_t M, int E, void* ws,
                                int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                                int32_t* invalid_count, hipStream_t stream);

// prologue.hip: quantize x (one group, per-call global scale) and route,
// in the same bytes as launch_quantize + launch_route, and clear sched_ints
// ints at sched (the GEMMs' scheduler counters); T > 0, qws and rws sized
// as for launch_quantize and launch_route
hipError_t launch_forward_prologue(const void* x, int64_t T, int64_t H, const int32_t* topk_ids,
                                   int k, int E, uint8_t* a_q, uint8_t* a_sf, float* gs_a,
                                   float* qws, void* rws, int32_t* offsets, int32_t* perm,
                                   int32_t* inv_perm, int32_t* invalid_count, int* sched,
                                   int sched_ints, hipStream_t stream);

// slot k of every token -> expert E with weight 1 (ids [T][k+1], w [T][k+1])
hipError_t launch_route_add_shared(const int32_t* ids, const float* w, int64_t T, int k, int E,
                                   int32_t* ids_out, float* w_out, hipStream_t stream);

// layout.hip
int64_t packed_rows(int64_t N);
hipError_t launch_pack_weights(const uint8_t* q, const uint8_t* sf, int64_t E, int64_t N, int64_t K,
                               uint8_t* qp, uint8_t* sfp, hipStream_t stream);
hipError_t launch_weight_layout(const void* src, int64_t groups, int64_t rows, int64_t cols,
                                int interleave, void* dst, hipStream_t stream);

// gemm.hip
struct GemmArgs {
  int epilogue;
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
  void* c_bf16;
  uint8_t* c_q;
  uint8_t* c_sf;
  float* c_debug;
  void* ws;         // the tile scheduler's counters (kGemmWorkspaceBytes), then
                    // room for split-K partials if ws_bytes allows
  size_t ws_bytes;
  int mx = 0;       // operands are MXFP4 (nvfp4 -> mx re-encoding), not NVFP4
  bool clear_sched = true;   // false: an earlier launch on the stream zeroed the counters
};
constexpr size_t kGemmWorkspaceBytes = 256;
// workspace with which a launch of this shape splits K (kGemmWorkspaceBytes
// when it would not split)
size_t gemm_splitk_ws_bytes(int epilogue, int64_t M, int64_t N, int64_t K, int E);
hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t stream);

// mx.hip: NVFP4 (q [rows][cols/2], E4M3 sf [rows][cols/16]) -> MXFP4 codes
// and E8M0 scales in the same shapes (each scale byte stored twice);
// cols % 32 == 0; in place allowed
hipError_t launch_mx_reencode(const uint8_t* q, const uint8_t* sf, int64_t rows, int64_t cols,
                              uint8_t* q_mx, uint8_t* sc_mx, hipStream_t stream);
constexpr int kRouterMaxExperts = 1024;
hipError_t launch_router_topk(const float* logits, int64_t T, int E, int k, int32_t* topk_ids,
                              float* topk_w, hipStream_t stream);

// combine.hip
hipError_t launch_combine(const void* y, const int32_t* inv_perm, const float* topk_w,
                          const int32_t* offsets, int64_t T, int k, int E, int64_t H, void* out,
                          hipStream_t stream);

}  // namespace nvfp4
