// C ABI of the NVFP4 MoE expert forward: argument validation, workspace
// carving and kernel launches.  Declarations and the contract of every entry
// point are in include/nvfp4moe.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "nvfp4moe.h"
#include "internal.hpp"

namespace {

thread_local std::string g_last_error;

nvfp4_status fail(nvfp4_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

nvfp4_status hip_fail(hipError_t err, const char* what) {
  return fail(NVFP4_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// per-device cache of the architecture check: 0 unknown, 1 gfx950, 2 other
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

nvfp4_status check_arch() {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return hip_fail(err, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(NVFP4_ERR_ARCH, "device index %d out of range", dev);
  int state = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    err = hipGetDeviceProperties(&prop, dev);
    if (err != hipSuccess) return hip_fail(err, "hipGetDeviceProperties");
    state = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch_ok[dev].store(state, std::memory_order_relaxed);
    if (state == 2) return fail(NVFP4_ERR_ARCH, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  }
  if (state == 2) return fail(NVFP4_ERR_ARCH, "device %d is not gfx950", dev);
  return NVFP4_OK;
}

nvfp4_status finish(hipError_t err, const char* what) {
  if (err != hipSuccess) return hip_fail(err, what);
  g_last_error.clear();
  return NVFP4_OK;
}

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// ---------------------------------------------------------------- checks

nvfp4_status check_quantize(const void* x, int64_t groups, int64_t rpg, int64_t cols, int64_t ld_x,
                            uint8_t* q, uint8_t* sf, float* gs_out) {
  if (groups < 0 || rpg < 0) return fail(NVFP4_ERR_SHAPE, "groups and rows_per_group must be >= 0");
  if (groups > 65535) return fail(NVFP4_ERR_SHAPE, "groups must be <= 65535");
  if (cols < 16 || cols % 16) return fail(NVFP4_ERR_SHAPE, "cols must be a positive multiple of 16 (got %lld)", (long long)cols);
  if (ld_x < cols || ld_x % 8)
    return fail(NVFP4_ERR_SHAPE, "ld_x must be >= cols and a multiple of 8 (got %lld)", (long long)ld_x);
  if (groups == 0) return NVFP4_OK;
  if (!gs_out) return fail(NVFP4_ERR_INVALID_ARG, "gs_out is NULL");
  if (rpg == 0) return NVFP4_OK;
  if (!x || !q || !sf) return fail(NVFP4_ERR_INVALID_ARG, "x, q and sf must be non-NULL");
  if (!aligned(x, 16) || !aligned(q, 8)) return fail(NVFP4_ERR_INVALID_ARG, "x must be 16-byte and q 8-byte aligned");
  if ((groups * rpg * cols / 16) >= (int64_t(1) << 40) || groups * rpg * (ld_x / 8) >= (int64_t(1) << 40))
    return fail(NVFP4_ERR_SHAPE, "tensor too large");
  return NVFP4_OK;
}

nvfp4_status check_route(const int32_t* ids, int64_t T, int k, int E, int32_t* off, int32_t* perm,
                         int32_t* inv) {
  if (T < 0) return fail(NVFP4_ERR_SHAPE, "T must be >= 0");
  if (k < 1 || k > 64) return fail(NVFP4_ERR_SHAPE, "k must be in [1, 64] (got %d)", k);
  if (E < 1 || E > 4096) return fail(NVFP4_ERR_SHAPE, "E must be in [1, 4096] (got %d)", E);
  if (T * k >= (int64_t(1) << 31)) return fail(NVFP4_ERR_SHAPE, "T*k must be < 2^31");
  if (!off) return fail(NVFP4_ERR_INVALID_ARG, "expert_offsets is NULL");
  if (T > 0 && (!ids || !perm || !inv)) return fail(NVFP4_ERR_INVALID_ARG, "topk_ids, perm and inv_perm must be non-NULL");
  return NVFP4_OK;
}

nvfp4_status check_gemm(const nvfp4::GemmArgs& a) {
  if (a.epilogue != NVFP4_EPI_BF16 && a.epilogue != NVFP4_EPI_SWIGLU_NVFP4)
    return fail(NVFP4_ERR_INVALID_ARG, "unknown epilogue %d", a.epilogue);
  if (a.E < 1 || a.E > 4096) return fail(NVFP4_ERR_SHAPE, "E must be in [1, 4096] (got %d)", a.E);
  if (a.M < 0 || a.M >= (int64_t(1) << 31)) return fail(NVFP4_ERR_SHAPE, "M must be in [0, 2^31)");
  if (a.K < 128 || a.K % 128) return fail(NVFP4_ERR_SHAPE, "K must be a positive multiple of 128 (got %lld)", (long long)a.K);
  if (a.N < 32 || a.N % 32) return fail(NVFP4_ERR_SHAPE, "N must be a positive multiple of 32 (got %lld)", (long long)a.N);
  if (a.N >= (int64_t(1) << 30)) return fail(NVFP4_ERR_SHAPE, "N must be < 2^30");
  // the kernels address a K stage of a weight tile (512 rows x 64 bytes) and
  // an A row (K/2 bytes) with 32-bit byte offsets
  if (a.K >= (int64_t(1) << 24)) return fail(NVFP4_ERR_SHAPE, "K must be < 2^24");
  if (!a.a_row_src && a.M * (a.K / 2) >= (int64_t(1) << 32))
    return fail(NVFP4_ERR_SHAPE, "A codes must be below 4 GiB (M*K/2 = %lld bytes)",
                (long long)(a.M * (a.K / 2)));
  if (a.a_row_src && a.a_row_div < 1) return fail(NVFP4_ERR_SHAPE, "a_row_div must be >= 1");
  // tile indices are 32-bit: (M/128 + E) m tiles times N/512 n tiles
  if (((a.M + 127) / 128 + a.E) * ((a.N + 511) / 512) >= (int64_t(1) << 31))
    return fail(NVFP4_ERR_SHAPE, "too many GEMM tiles (M, N too large)");
  if (!a.offsets) return fail(NVFP4_ERR_INVALID_ARG, "expert_offsets is NULL");
  if (a.M == 0) return NVFP4_OK;
  if (!a.a_q || !a.a_sf || !a.gs_a || !a.b_q || !a.b_sf || !a.gs_b)
    return fail(NVFP4_ERR_INVALID_ARG, "A and B operands and their scales must be non-NULL");
  if (!aligned(a.a_q, 16) || !aligned(a.b_q, 16) || !aligned(a.a_sf, 8) || !aligned(a.b_sf, 8))
    return fail(NVFP4_ERR_INVALID_ARG, "codes must be 16-byte and scales 8-byte aligned");
  if (a.epilogue == NVFP4_EPI_BF16) {
    if (!a.c_bf16) return fail(NVFP4_ERR_INVALID_ARG, "c_bf16 is NULL");
    if (!aligned(a.c_bf16, 8)) return fail(NVFP4_ERR_INVALID_ARG, "c_bf16 must be 8-byte aligned");
  } else {
    if (!a.c_q || !a.c_sf || !a.gs_out) return fail(NVFP4_ERR_INVALID_ARG, "c_q, c_sf and gs_out must be non-NULL");
    if (!aligned(a.c_q, 4)) return fail(NVFP4_ERR_INVALID_ARG, "c_q must be 4-byte aligned");
  }
  return NVFP4_OK;
}

nvfp4_status check_combine(const void* y, const int32_t* inv, const float* w, const int32_t* off,
                           int64_t T, int k, int E, int64_t H, void* out) {
  if (T < 0) return fail(NVFP4_ERR_SHAPE, "T must be >= 0");
  if (k < 1 || k > 64) return fail(NVFP4_ERR_SHAPE, "k must be in [1, 64] (got %d)", k);
  if (E < 1 || E > 4096) return fail(NVFP4_ERR_SHAPE, "E must be in [1, 4096] (got %d)", E);
  if (H < 8 || H % 8) return fail(NVFP4_ERR_SHAPE, "H must be a positive multiple of 8 (got %lld)", (long long)H);
  if (T == 0) return NVFP4_OK;
  if (!y || !inv || !w || !off || !out) return fail(NVFP4_ERR_INVALID_ARG, "y, inv_perm, topk_w, expert_offsets and out must be non-NULL");
  if (!aligned(y, 16) || !aligned(out, 16)) return fail(NVFP4_ERR_INVALID_ARG, "y and out must be 16-byte aligned");
  return NVFP4_OK;
}

struct FwdLayout {
  size_t a_q, a_sf, gs_a, qws, off, perm, inv, bad, rws, gws, h_q, h_sf, y, total;
};

FwdLayout fwd_layout(int64_t T, int64_t H, int64_t I, int E, int k) {
  FwdLayout L;
  const int64_t M = T * k;
  size_t o = 0;
  auto take = [&](size_t n) { size_t at = o; o += align256(n); return at; };
  L.a_q = take((size_t)(T * H / 2));
  L.a_sf = take((size_t)(T * H / 16));
  L.gs_a = take(sizeof(float));
  L.qws = take(sizeof(float) * (size_t)nvfp4::quantize_parts(1, T, H));
  L.off = take(sizeof(int32_t) * (size_t)(E + 1));
  L.perm = take(sizeof(int32_t) * (size_t)M);
  L.inv = take(sizeof(int32_t) * (size_t)M);
  L.bad = take(sizeof(int32_t));
  L.rws = take(nvfp4::route_ws_bytes(T, k, E));
  L.gws = take(2 * nvfp4::kGemmWorkspaceBytes);   // L1's scheduler counters, then L2's
  L.h_q = take((size_t)(M * I / 2));
  L.h_sf = take((size_t)(M * I / 16));
  L.y = take((size_t)(M * H * 2));
  L.total = o;
  return L;
}

}  // namespace

extern "C" {

const char* nvfp4_status_string(nvfp4_status s) {
  switch (s) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_INVALID_ARG: return "invalid argument";
    case NVFP4_ERR_SHAPE: return "unsupported shape";
    case NVFP4_ERR_WORKSPACE: return "workspace missing or too small";
    case NVFP4_ERR_ARCH: return "device is not gfx950";
    case NVFP4_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* nvfp4_last_error(void) { return g_last_error.c_str(); }

int nvfp4_version(void) { return 100; }

nvfp4_status nvfp4_weight_layout(const void* src, int64_t groups, int64_t rows, int64_t cols,
                                 int interleave, void* dst, void* stream) {
  if (groups < 0 || groups > 65535) return fail(NVFP4_ERR_SHAPE, "groups must be in [0, 65535]");
  if (rows < 1 || cols < 1) return fail(NVFP4_ERR_SHAPE, "rows and cols must be >= 1");
  if (interleave && cols % 16) return fail(NVFP4_ERR_SHAPE, "interleave needs cols % 16 == 0");
  if (groups > 0 && (!src || !dst)) return fail(NVFP4_ERR_INVALID_ARG, "src and dst must be non-NULL");
  if (groups > 0 && src == dst) return fail(NVFP4_ERR_INVALID_ARG, "src and dst must not overlap");
  nvfp4_status st = check_arch();
  if (st != NVFP4_OK) return st;
  return finish(nvfp4::launch_weight_layout(src, groups, rows, cols, interleave, dst,
                                            static_cast<hipStream_t>(stream)),
                "nvfp4_weight_layout launch");
}

size_t nvfp4_packed_weight_bytes(int64_t E, int64_t N, int64_t K, size_t* sf_bytes) {
  if (E < 1 || N < 1 || K < NVFP4_PACK_K || K % NVFP4_PACK_K) {
    if (sf_bytes) *sf_bytes = 0;
    return 0;
  }
  const int64_t Np = nvfp4::packed_rows(N);
  if (sf_bytes) *sf_bytes = (size_t)(E * Np * (K / 16));
  return (size_t)(E * Np * (K / 2));
}

nvfp4_status nvfp4_pack_weights(const uint8_t* q, const uint8_t* sf, int64_t E, int64_t N,
                                int64_t K, uint8_t* q_packed, uint8_t* sf_packed, void* stream) {
  if (E < 1 || E > 65535 || N < 1) return fail(NVFP4_ERR_SHAPE, "E must be in [1, 65535] and N >= 1");
  if (K < NVFP4_PACK_K || K % NVFP4_PACK_K)
    return fail(NVFP4_ERR_SHAPE, "K must be a positive multiple of %d (got %lld)", NVFP4_PACK_K, (long long)K);
  if (!q || !sf || !q_packed || !sf_packed) return fail(NVFP4_ERR_INVALID_ARG, "all pointers must be non-NULL");
  if (!aligned(q, 16) || !aligned(q_packed, 16) || !aligned(sf, 8) || !aligned(sf_packed, 8))
    return fail(NVFP4_ERR_INVALID_ARG, "codes must be 16-byte and scales 8-byte aligned");
  if (q == q_packed || sf == sf_packed) return fail(NVFP4_ERR_INVALID_ARG, "in and out must not overlap");
  nvfp4_status st = check_arch();
  if (st != NVFP4_OK) return st;
  return finish(nvfp4::launch_pack_weights(q, sf, E, N, K, q_packed, sf_packed,
                                           static_cast<hipStream_t>(stream)),
                "nvfp4_pack_weights launch");
}

size_t nvfp4_quantize_workspace_size(int64_t groups, int64_t rows_per_group, int64_t cols) {
  if (groups <= 0 || rows_per_group <= 0 || cols <= 0) return 0;
  return sizeof(float) * (size_t)groups * (size_t)nvfp4::quantize_parts(groups, rows_per_group, cols);
}

nvfp4_status nvfp4_quantize(const void* x, int64_t groups, int64_t rows_per_group, int64_t cols,
                            int64_t ld_x, const float* gs_in, uint8_t* q, uint8_t* sf,
                            float* gs_out, void* ws, size_t ws_bytes, void* stream) {
  nvfp4_status st = check_quantize(x, groups, rows_per_group, cols, ld_x, q, sf, gs_out);
  if (st != NVFP4_OK) return st;
  if (gs_in == nullptr) {
    const size_t need = nvfp4_quantize_workspace_size(groups, rows_per_group, cols);
    if (need > 0 && (ws == nullptr || ws_bytes < need))
      return fail(NVFP4_ERR_WORKSPACE, "quantize needs %zu workspace bytes (got %zu)", need, ws_bytes);
    if (ws && !aligned(ws, 4)) return fail(NVFP4_ERR_WORKSPACE, "workspace must be 4-byte aligned");
  }
  if (groups == 0) return NVFP4_OK;
  st = check_arch();
  if (st != NVFP4_OK) return st;
  return finish(nvfp4::launch_quantize(x, groups, rows_per_group, cols, ld_x, gs_in, q, sf, gs_out,
                                       static_cast<float*>(ws), static_cast<hipStream_t>(stream)),
                "nvfp4_quantize launch");
}

size_t nvfp4_moe_route_workspace_size(int64_t T, int k, int E) {
  if (T < 0 || k < 1 || E < 1) return 0;
  return nvfp4::route_ws_bytes(T, k, E);
}

size_t nvfp4_quantize_scatter_workspace_size(int64_t T, int64_t H) {
  if (T <= 0 || H < 16 || H % 16) return 0;
  return sizeof(float) * (size_t)nvfp4::quantize_parts(1, T, H);
}

nvfp4_status nvfp4_quantize_scatter(const void* x_bf16, int64_t T, int64_t H, int k,
                                    const int32_t* inv_perm, const int32_t* expert_offsets, int E,
                                    uint8_t* q, uint8_t* sf, float* gs_out, void* ws,
                                    size_t ws_bytes, void* stream) {
  if (T < 0) return fail(NVFP4_ERR_SHAPE, "T must be >= 0");
  if (H < 16 || H % 16) return fail(NVFP4_ERR_SHAPE, "H must be a positive multiple of 16 (got %lld)", (long long)H);
  if (k < 1 || k > 64) return fail(NVFP4_ERR_SHAPE, "k must be in [1, 64] (got %d)", k);
  if (E < 1 || E > 4096) return fail(NVFP4_ERR_SHAPE, "E must be in [1, 4096] (got %d)", E);
  if (T * k >= (int64_t(1) << 31)) return fail(NVFP4_ERR_SHAPE, "T*k must be < 2^31");
  if (!gs_out) return fail(NVFP4_ERR_INVALID_ARG, "gs_out is NULL");
  if (T > 0 && (!x_bf16 || !inv_perm || !expert_offsets || !q || !sf))
    return fail(NVFP4_ERR_INVALID_ARG, "x, inv_perm, expert_offsets, q and sf must be non-NULL");
  if (T > 0 && (!aligned(x_bf16, 16) || !aligned(q, 8)))
    return fail(NVFP4_ERR_INVALID_ARG, "x must be 16-byte and q 8-byte aligned");
  const size_t need = nvfp4_quantize_scatter_workspace_size(T, H);
  if (T > 0 && (ws == nullptr || ws_bytes < need || !aligned(ws, 4)))
    return fail(NVFP4_ERR_WORKSPACE, "quantize_scatter needs %zu 4-byte aligned workspace bytes (got %zu)", need, ws_bytes);
  nvfp4_status st = check_arch();
  if (st != NVFP4_OK) return st;
  return finish(nvfp4::launch_quantize_scatter(x_bf16, T, H, k, inv_perm, expert_offsets, E, q, sf,
                                               gs_out, static_cast<float*>(ws),
                                               static_cast<hipStream_t>(stream)),
                "nvfp4_quantize_scatter launch");
}

nvfp4_status nvfp4_moe_route(const int32_t* topk_ids, int64_t T, int k, int E,
                             int32_t* expert_offsets, int32_t* perm, int32_t* inv_perm,
                             int32_t* invalid_count, void* ws, size_t ws_bytes, void* stream) {
  nvfp4_status st = check_route(topk_ids, T, k, E, expert_offsets, perm, inv_perm);
  if (st != NVFP4_OK) return st;
  const size_t need = nvfp4::route_ws_bytes(T, k, E);
  if (ws == nullptr || ws_bytes < need)
    return fail(NVFP4_ERR_WORKSPACE, "route needs %zu workspace bytes (got %zu)", need, ws_bytes);
  if (!aligned(ws, 4)) return fail(NVFP4_ERR_WORKSPACE, "workspace must be 4-byte aligned");
  st = check_arch();
  if (st != NVFP4_OK) return st;
  return finish(nvfp4::launch_route(topk_ids, T, k, E, expert_offsets, perm, inv_perm,
                                    invalid_count, ws, static_cast<hipStream_t>(stream)),
                "nvfp4_moe_route launch");
}

nvfp4_status nvfp4_router_topk(const float* logits, int64_t T, int E, int k, int32_t* topk_ids,
                               float* topk_w, void* stream) {
  if (T < 0) return fail(NVFP4_ERR_SHAPE, "T must be >= 0");
  if (E < 1 || E > nvfp4::kRouterMaxExperts)
    return fail(NVFP4_ERR_SHAPE, "E must be in [1, %d] (got %d)", nvfp4::kRouterMaxExperts, E);
  if (k < 1 || k > 64 || k > E) return fail(NVFP4_ERR_SHAPE, "k must be in [1, min(E, 64)] (got %d)", k);
  if (T == 0) return NVFP4_OK;
  if (!logits || !topk_ids || !topk_w)
    return fail(NVFP4_ERR_INVALID_ARG, "logits, topk_ids and topk_w must be non-NULL");
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4))
    return fail(NVFP4_ERR_INVALID_ARG, "logits, topk_ids and topk_w must be 4-byte aligned");
  nvfp4_status st = check_arch();
  if (st != NVFP4_OK) return st;
  return finish(nvfp4::launch_router_topk(logits, T, E, k, topk_ids, topk_w,
                                          static_cast<hipStream_t>(stream)),
                "nvfp4_router_topk launch");
}

size_t nvfp4_grouped_gemm_workspace_size(void) { return nvfp4::kGemmWorkspaceBytes; }

size_t nvfp4_grouped_gemm_splitk_workspace_size(int epilogue, int64_t M, int64_t N, int64_t K,
                                                int E) {
  if (M < 0 || N < 32 || K < 128 || E < 1) return nvfp4::kGemmWorkspaceBytes;
  return nvfp4::gemm_splitk_ws_bytes(epilogue, M, N, K, E);
}

}  // extern "C"

namespace {
nvfp4_status grouped_gemm_impl(int mx, int epilogue, const uint8_t* a_q, const uint8_t* a_sf,
                               const float* gs_a, const int32_t* a_row_src, int a_row_div,
                               const int32_t* expert_offsets, int E, int64_t M, int64_t N,
                               int64_t K, const uint8_t* b_q, const uint8_t* b_sf,
                               const float* gs_b, const float* gs_out, void* c_bf16,
                               uint8_t* c_q, uint8_t* c_sf, float* c_debug_f32, void* ws,
                               size_t ws_bytes, void* stream) {
  nvfp4::GemmArgs a{epilogue, a_q, a_sf, gs_a, a_row_src, a_row_div, expert_offsets, E, M, N, K,
                    b_q, b_sf, gs_b, gs_out, c_bf16, c_q, c_sf, c_debug_f32, ws, ws_bytes, mx};
  nvfp4_status st = check_gemm(a);
  if (st != NVFP4_OK) return st;
  if (M == 0) return NVFP4_OK;
  if (ws == nullptr || ws_bytes < nvfp4::kGemmWorkspaceBytes)
    return fail(NVFP4_ERR_WORKSPACE, "grouped GEMM needs %zu workspace bytes (got %zu)",
                nvfp4::kGemmWorkspaceBytes, ws_bytes);
  if (!aligned(ws, 4)) return fail(NVFP4_ERR_WORKSPACE, "workspace must be 4-byte aligned");
  st = check_arch();
  if (st != NVFP4_OK) return st;
  return finish(nvfp4::launch_grouped_gemm(a, static_cast<hipStream_t>(stream)),
                mx ? "nvfp4_mx_grouped_gemm launch" : "nvfp4_grouped_gemm launch");
}
}  // namespace

extern "C" {

nvfp4_status nvfp4_grouped_gemm(int epilogue, const uint8_t* a_q, const uint8_t* a_sf,
                                const float* gs_a, const int32_t* a_row_src, int a_row_div,
                                const int32_t* expert_offsets, int E, int64_t M, int64_t N,
                                int64_t K, const uint8_t* b_q, const uint8_t* b_sf,
                                const float* gs_b, const float* gs_out, void* c_bf16,
                                uint8_t* c_q, uint8_t* c_sf, float* c_debug_f32, void* ws,
                                size_t ws_bytes, void* stream) {
  return grouped_gemm_impl(0, epilogue, a_q, a_sf, gs_a, a_row_src, a_row_div, expert_offsets, E,
                           M, N, K, b_q, b_sf, gs_b, gs_out, c_bf16, c_q, c_sf, c_debug_f32, ws,
                           ws_bytes, stream);
}

nvfp4_status nvfp4_mx_grouped_gemm(int epilogue, const uint8_t* a_q, const uint8_t* a_sc,
                                   const float* gs_a, const int32_t* a_row_src, int a_row_div,
                                   const int32_t* expert_offsets, int E, int64_t M, int64_t N,
                                   int64_t K, const uint8_t* b_q, const uint8_t* b_sc,
                                   const float* gs_b, const float* gs_out, void* c_bf16,
                                   uint8_t* c_q, uint8_t* c_sf, float* c_debug_f32, void* ws,
                                   size_t ws_bytes, void* stream) {
  return grouped_gemm_impl(1, epilogue, a_q, a_sc, gs_a, a_row_src, a_row_div, expert_offsets, E,
                           M, N, K, b_q, b_sc, gs_b, gs_out, c_bf16, c_q, c_sf, c_debug_f32, ws,
                           ws_bytes, stream);
}

nvfp4_status nvfp4_to_mx(const uint8_t* q, const uint8_t* sf, int64_t rows, int64_t cols,
                         uint8_t* q_mx, uint8_t* sc_mx, void* stream) {
  if (rows < 0) return fail(NVFP4_ERR_SHAPE, "rows must be >= 0");
  if (cols < 32 || cols % 32) return fail(NVFP4_ERR_SHAPE, "cols must be a positive multiple of 32 (got %lld)", (long long)cols);
  if (rows * (cols / 32) >= (int64_t(1) << 40)) return fail(NVFP4_ERR_SHAPE, "tensor too large");
  if (rows == 0) return NVFP4_OK;
  if (!q || !sf || !q_mx || !sc_mx) return fail(NVFP4_ERR_INVALID_ARG, "all pointers must be non-NULL");
  if (!aligned(q, 16) || !aligned(q_mx, 16) || !aligned(sf, 2) || !aligned(sc_mx, 2))
    return fail(NVFP4_ERR_INVALID_ARG, "codes must be 16-byte and scales 2-byte aligned");
  const int64_t qb = rows * cols / 2, sb = rows * cols / 16;
  auto overlap = [](const uint8_t* a, int64_t na, const uint8_t* b, int64_t nb) {
    return a < b + nb && b < a + na;
  };
  if ((q != q_mx && overlap(q, qb, q_mx, qb)) || (sf != sc_mx && overlap(sf, sb, sc_mx, sb)))
    return fail(NVFP4_ERR_INVALID_ARG, "outputs must be the inputs (in place) or not overlap them");
  nvfp4_status st = check_arch();
  if (st != NVFP4_OK) return st;
  return finish(nvfp4::launch_mx_reencode(q, sf, rows, cols, q_mx, sc_mx,
                                          static_cast<hipStream_t>(stream)),
                "nvfp4_to_mx launch");
}

nvfp4_status nvfp4_moe_combine(const void* y_bf16, const int32_t* inv_perm, const float* topk_w,
                               const int32_t* expert_offsets, int64_t T, int k, int E, int64_t H,
                               void* out_bf16, void* stream) {
  nvfp4_status st = check_combine(y_bf16, inv_perm, topk_w, expert_offsets, T, k, E, H, out_bf16);
  if (st != NVFP4_OK) return st;
  if (T == 0) return NVFP4_OK;
  st = check_arch();
  if (st != NVFP4_OK) return st;
  return finish(nvfp4::launch_combine(y_bf16, inv_perm, topk_w, expert_offsets, T, k, E, H,
                                      out_bf16, static_cast<hipStream_t>(stream)),
                "nvfp4_moe_combine launch");
}

size_t moe_expert_forward_workspace_size(int64_t T, int64_t H, int64_t I, int E, int k) {
  if (T < 0 || H <= 0 || I <= 0 || E < 1 || k < 1) return 0;
  return fwd_layout(T, H, I, E, k).total;
}

}  // extern "C"

namespace {
nvfp4_status forward_impl(int mx, const void* x_bf16, int64_t T, int64_t H, int64_t I, int E,
                          int k, const int32_t* topk_ids, const float* topk_w, const uint8_t* w1_q,
                          const uint8_t* w1_sf, const float* gs_w1, const uint8_t* w2_q,
                          const uint8_t* w2_sf, const float* gs_w2, const float* gs_h,
                          void* out_bf16, const nvfp4_moe_taps* taps, void* ws, size_t ws_bytes,
                          void* stream, bool check_only = false) {
  if (T < 0) return fail(NVFP4_ERR_SHAPE, "T must be >= 0");
  if (H < 128 || H % 128) return fail(NVFP4_ERR_SHAPE, "H must be a positive multiple of 128 (got %lld)", (long long)H);
  if (I < 128 || I % 128) return fail(NVFP4_ERR_SHAPE, "I must be a positive multiple of 128 (got %lld)", (long long)I);
  if (k < 1 || k > 64) return fail(NVFP4_ERR_SHAPE, "k must be in [1, 64] (got %d)", k);
  if (E < 1 || E > 4096) return fail(NVFP4_ERR_SHAPE, "E must be in [1, 4096] (got %d)", E);
  if (T * k >= (int64_t(1) << 31)) return fail(NVFP4_ERR_SHAPE, "T*k must be < 2^31");
  // the GEMMs address their A rows with 32-bit byte offsets: the quantised x
  // (L1, gathered) and h (L2) must each stay below 4 GiB of codes
  if (T * (H / 2) >= (int64_t(1) << 32) || T * k * (I / 2) >= (int64_t(1) << 32))
    return fail(NVFP4_ERR_SHAPE, "quantised x (T*H/2 bytes) and h (T*k*I/2 bytes) must be below 4 GiB");
  if (H >= (int64_t(1) << 24) || I >= (int64_t(1) << 23)) return fail(NVFP4_ERR_SHAPE, "H must be < 2^24 and I < 2^23");
  if (T > 0 && (!x_bf16 || !topk_ids || !topk_w || !out_bf16))
    return fail(NVFP4_ERR_INVALID_ARG, "x, topk_ids, topk_w and out must be non-NULL");
  if (!w1_q || !w1_sf || !gs_w1 || !w2_q || !w2_sf || !gs_w2 || !gs_h)
    return fail(NVFP4_ERR_INVALID_ARG, "weights, their scales and gs_h must be non-NULL");
  const FwdLayout L = fwd_layout(T, H, I, E, k);
  if (ws == nullptr || ws_bytes < L.total)
    return fail(NVFP4_ERR_WORKSPACE, "moe_expert_forward needs %zu workspace bytes (got %zu)", L.total, ws_bytes);
  if (!aligned(ws, 256)) return fail(NVFP4_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (T > 0 && (!aligned(x_bf16, 16) || !aligned(out_bf16, 16)))
    return fail(NVFP4_ERR_INVALID_ARG, "x and out must be 16-byte aligned");
  if (!aligned(w1_q, 16) || !aligned(w2_q, 16) || !aligned(w1_sf, 8) || !aligned(w2_sf, 8))
    return fail(NVFP4_ERR_INVALID_ARG, "weight codes must be 16-byte and scales 8-byte aligned");
  nvfp4_moe_taps tp;
  std::memset(&tp, 0, sizeof(tp));
  if (taps) tp = *taps;
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint8_t* a_q = tp.a_q ? tp.a_q : base + L.a_q;
  uint8_t* a_sf = tp.a_sf ? tp.a_sf : base + L.a_sf;
  float* gs_a = tp.gs_a ? tp.gs_a : reinterpret_cast<float*>(base + L.gs_a);
  int32_t* off = tp.expert_offsets ? tp.expert_offsets : reinterpret_cast<int32_t*>(base + L.off);
  int32_t* perm = tp.perm ? tp.perm : reinterpret_cast<int32_t*>(base + L.perm);
  int32_t* inv = tp.inv_perm ? tp.inv_perm : reinterpret_cast<int32_t*>(base + L.inv);
  int32_t* bad = tp.invalid_count ? tp.invalid_count : reinterpret_cast<int32_t*>(base + L.bad);
  uint8_t* h_q = tp.h_q ? tp.h_q : base + L.h_q;
  uint8_t* h_sf = tp.h_sf ? tp.h_sf : base + L.h_sf;
  void* y = tp.y_bf16 ? tp.y_bf16 : static_cast<void*>(base + L.y);
  if (!aligned(a_q, 16) || !aligned(h_q, 16) || !aligned(y, 16) || !aligned(a_sf, 8) || !aligned(h_sf, 8))
    return fail(NVFP4_ERR_INVALID_ARG, "tap buffers must be 16-byte (codes, y) and 8-byte (scales) aligned");
  nvfp4_status st = check_arch();
  if (st != NVFP4_OK) return st;
  if (check_only) return NVFP4_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t M = T * k;
  hipError_t err = hipSuccess;
  uint8_t* gws1 = base + L.gws;
  uint8_t* gws2 = gws1 + nvfp4::kGemmWorkspaceBytes;
  if (T > 0) {
    // quantize x + route in three launches; the first also zeroes both
    // GEMMs' scheduler counters (both 256-byte slots)
    err = nvfp4::launch_forward_prologue(x_bf16, T, H, topk_ids, k, E, a_q, a_sf, gs_a,
                                         reinterpret_cast<float*>(base + L.qws), base + L.rws, off,
                                         perm, inv, bad, reinterpret_cast<int*>(gws1),
                                         (int)(2 * nvfp4::kGemmWorkspaceBytes / sizeof(int)), s);
    if (err != hipSuccess) return hip_fail(err, "moe_expert_forward quantize + route");
    if (mx) {
      err = nvfp4::launch_mx_reencode(a_q, a_sf, T, H, a_q, a_sf, s);
      if (err != hipSuccess) return hip_fail(err, "moe_expert_forward_mx re-encode x");
    }
  } else {
    nvfp4::fill_f32(gs_a, 1.0f, 1, s);
    err = nvfp4::launch_route(topk_ids, T, k, E, off, perm, inv, bad, base + L.rws, s);
    if (err != hipSuccess) return hip_fail(err, "moe_expert_forward route");
  }
  if (M > 0) {
    nvfp4::GemmArgs l1{NVFP4_EPI_SWIGLU_NVFP4, a_q, a_sf, gs_a, perm, k, off, E, M, 2 * I, H,
                       w1_q, w1_sf, gs_w1, gs_h, nullptr, h_q, h_sf, tp.h_f32, gws1,
                       nvfp4::kGemmWorkspaceBytes, mx, /*clear_sched=*/false};
    err = nvfp4::launch_grouped_gemm(l1, s);
    if (err != hipSuccess) return hip_fail(err, "moe_expert_forward L1");
    if (mx) {
      err = nvfp4::launch_mx_reencode(h_q, h_sf, M, I, h_q, h_sf, s);
      if (err != hipSuccess) return hip_fail(err, "moe_expert_forward_mx re-encode h");
    }
    nvfp4::GemmArgs l2{NVFP4_EPI_BF16, h_q, h_sf, gs_h, nullptr, 1, off, E, M, H, I,
                       w2_q, w2_sf, gs_w2, nullptr, y, nullptr, nullptr, nullptr, gws2,
                       nvfp4::kGemmWorkspaceBytes, mx, /*clear_sched=*/false};
    err = nvfp4::launch_grouped_gemm(l2, s);
    if (err != hipSuccess) return hip_fail(err, "moe_expert_forward L2");
  }
  err = nvfp4::launch_combine(y, inv, topk_w, off, T, k, E, H, out_bf16, s);
  return finish(err, "moe_expert_forward combine");
}
}  // namespace

extern "C" {

nvfp4_status moe_expert_forward(const void* x_bf16, int64_t T, int64_t H, int64_t I, int E, int k,
                                const int32_t* topk_ids, const float* topk_w, const uint8_t* w1_q,
                                const uint8_t* w1_sf, const float* gs_w1, const uint8_t* w2_q,
                                const uint8_t* w2_sf, const float* gs_w2, const float* gs_h,
                                void* out_bf16, const nvfp4_moe_taps* taps, void* ws,
                                size_t ws_bytes, void* stream) {
  return forward_impl(0, x_bf16, T, H, I, E, k, topk_ids, topk_w, w1_q, w1_sf, gs_w1, w2_q, w2_sf,
                      gs_w2, gs_h, out_bf16, taps, ws, ws_bytes, stream);
}

size_t moe_expert_forward_shared_workspace_size(int64_t T, int64_t H, int64_t I, int E, int k) {
  if (T < 0 || H <= 0 || I <= 0 || E < 1 || k < 1) return 0;
  return fwd_layout(T, H, I, E + 1, k + 1).total + 2 * align256(sizeof(int32_t) * (size_t)(T * (k + 1)));
}

nvfp4_status moe_expert_forward_shared(const void* x_bf16, int64_t T, int64_t H, int64_t I, int E,
                                       int k, const int32_t* topk_ids, const float* topk_w,
                                       const uint8_t* w1_q, const uint8_t* w1_sf,
                                       const float* gs_w1, const uint8_t* w2_q,
                                       const uint8_t* w2_sf, const float* gs_w2, const float* gs_h,
                                       void* out_bf16, const nvfp4_moe_taps* taps, void* ws,
                                       size_t ws_bytes, void* stream) {
  if (T < 0) return fail(NVFP4_ERR_SHAPE, "T must be >= 0");
  if (k < 1 || k > 63) return fail(NVFP4_ERR_SHAPE, "k must be in [1, 63] with a shared expert (got %d)", k);
  if (E < 1 || E > 4095) return fail(NVFP4_ERR_SHAPE, "E must be in [1, 4095] with a shared expert (got %d)", E);
  if (H <= 0 || I <= 0) return fail(NVFP4_ERR_SHAPE, "H and I must be positive");
  if (T * (k + 1) >= (int64_t(1) << 31)) return fail(NVFP4_ERR_SHAPE, "T*(k+1) must be < 2^31");
  if (T > 0 && (!topk_ids || !topk_w)) return fail(NVFP4_ERR_INVALID_ARG, "topk_ids and topk_w must be non-NULL");
  const size_t core = fwd_layout(T, H, I, E + 1, k + 1).total;
  const size_t need = moe_expert_forward_shared_workspace_size(T, H, I, E, k);
  if (ws == nullptr || ws_bytes < need)
    return fail(NVFP4_ERR_WORKSPACE, "moe_expert_forward_shared needs %zu workspace bytes (got %zu)", need, ws_bytes);
  if (!aligned(ws, 256)) return fail(NVFP4_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  uint8_t* base = static_cast<uint8_t*>(ws);
  int32_t* ids2 = reinterpret_cast<int32_t*>(base + core);
  float* w2 = reinterpret_cast<float*>(base + core + align256(sizeof(int32_t) * (size_t)(T * (k + 1))));
  if (T > 0) {
    // the checks of the routed forward run first, so nothing is enqueued on a bad call
    const nvfp4_status st = forward_impl(0, x_bf16, T, H, I, E + 1, k + 1, ids2, w2, w1_q, w1_sf,
                                         gs_w1, w2_q, w2_sf, gs_w2, gs_h, out_bf16, taps, ws, core,
                                         nullptr, /*check_only=*/true);
    if (st != NVFP4_OK) return st;
    const hipError_t err = nvfp4::launch_route_add_shared(topk_ids, topk_w, T, k, E, ids2, w2,
                                                          static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(err, "moe_expert_forward_shared routing");
  }
  return forward_impl(0, x_bf16, T, H, I, E + 1, k + 1, ids2, w2, w1_q, w1_sf, gs_w1, w2_q, w2_sf,
                      gs_w2, gs_h, out_bf16, taps, ws, core, stream, false);
}

nvfp4_status moe_expert_forward_mx(const void* x_bf16, int64_t T, int64_t H, int64_t I, int E,
                                   int k, const int32_t* topk_ids, const float* topk_w,
                                   const uint8_t* w1_q, const uint8_t* w1_sc, const float* gs_w1,
                                   const uint8_t* w2_q, const uint8_t* w2_sc, const float* gs_w2,
                                   const float* gs_h, void* out_bf16, const nvfp4_moe_taps* taps,
                                   void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(1, x_bf16, T, H, I, E, k, topk_ids, topk_w, w1_q, w1_sc, gs_w1, w2_q, w2_sc,
                      gs_w2, gs_h, out_bf16, taps, ws, ws_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------- without a workspace
//
// The forward's workspace for callers that cannot allocate device memory: a
// file-scope device array, one copy per GPU, held until the process ends.  In
// host code the name `scratch` stands for the host-side shadow of the symbol,
// not a device address: every use goes through the address that
// hipGetSymbolAddress returns on the device in question, cached per device.
namespace {

static __device__ __align__(256) uint8_t scratch[NVFP4_NOALLOC_SCRATCH_BYTES];

std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// device address of this device's `scratch` (looked up once per device, with
// that device current)
nvfp4_status scratch_address(void** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return hip_fail(err, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(NVFP4_ERR_ARCH, "device index %d out of range", dev);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
      err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (err != hipSuccess) return hip_fail(err, "hipGetSymbolAddress(scratch)");
      if (p == nullptr || !aligned(p, 256))
        return fail(NVFP4_ERR_HIP, "the scratch array has no 256-byte aligned device address");
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return NVFP4_OK;
}

}  // namespace

extern "C" nvfp4_status moe_expert_forward_noalloc(
    const void* x_bf16, int64_t T, int64_t H, int64_t I, int E, int k, const int32_t* topk_ids,
    const float* topk_w, const uint8_t* w1_q, const uint8_t* w1_sf, const float* gs_w1,
    const uint8_t* w2_q, const uint8_t* w2_sf, const float* gs_w2, const float* gs_h,
    void* out_bf16, const nvfp4_moe_taps* taps, void* stream) {
  const size_t need = moe_expert_forward_workspace_size(T, H, I, E, k);
  if (need > NVFP4_NOALLOC_SCRATCH_BYTES)
    return fail(NVFP4_ERR_WORKSPACE,
                "moe_expert_forward_noalloc: this shape needs %zu workspace bytes, the static "
                "scratch holds %zu; call moe_expert_forward with a workspace",
                need, (size_t)NVFP4_NOALLOC_SCRATCH_BYTES);
  // every argument check of the forward first, with a stand-in workspace
  // address that is never dereferenced (nothing is enqueued)
  void* const stand_in = reinterpret_cast<void*>(uintptr_t(256));
  nvfp4_status st = forward_impl(0, x_bf16, T, H, I, E, k, topk_ids, topk_w, w1_q, w1_sf, gs_w1,
                                 w2_q, w2_sf, gs_w2, gs_h, out_bf16, taps, stand_in,
                                 NVFP4_NOALLOC_SCRATCH_BYTES, nullptr, /*check_only=*/true);
  if (st != NVFP4_OK) return st;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != NVFP4_OK) return st;
  return forward_impl(0, x_bf16, T, H, I, E, k, topk_ids, topk_w, w1_q, w1_sf, gs_w1, w2_q, w2_sf,
                      gs_w2, gs_h, out_bf16, taps, ws, NVFP4_NOALLOC_SCRATCH_BYTES, stream);
}
