/*
 * nvfp4moe.h — C ABI of the NVFP4 block-scaled MoE expert forward for
 * AMD Instinct MI355X (gfx950).
 *
 * The method: the "NVFP4 MegaMoE Kernel" README (sections "What We Have",
 * "Fused SwiGLU — How It Works", "Correctness Bugs Fixed", "Key Lessons") and
 * the "CURRENT_BUG.md" page (section "What Works").
 *
 * NVFP4 tensor of R rows and C columns (C % 16 == 0), row-major:
 *   codes  uint8[R][C/2]   two E2M1 codes per byte along the row, element 2j
 *                          in the low nibble, bit 3 of a code is the sign;
 *   scales uint8[R][C/16]  one OCP E4M3 (bias 7, max 448) per 16 elements;
 *   gs     float           global scale; a value is E2M1 * E4M3 / gs.
 * BF16 tensors are passed as raw 16-bit patterns (uint16_t / void*).
 *
 * Common rules for every entry point:
 *   - all data pointers are DEVICE pointers owned by the caller; the library
 *     never frees or retains them;
 *   - work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     null stream); nothing allocates memory, synchronises the host or reads
 *     device data on the host, so every call can be captured in a hipGraph;
 *   - arguments are validated on the host BEFORE any HIP call; a failed check
 *     returns an error status and enqueues nothing; nvfp4_last_error()
 *     returns a thread-local description of the last failure;
 *   - the current HIP device must be a gfx950 (else NVFP4_ERR_ARCH);
 *   - inputs must be finite (no NaN/Inf in BF16 data).
 */
#ifndef NVFP4MOE_H
#define NVFP4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int nvfp4_status;
#define NVFP4_OK               0
#define NVFP4_ERR_INVALID_ARG (-1) /* null pointer, bad enum value         */
#define NVFP4_ERR_SHAPE       (-2) /* a size breaks the shape rules        */
#define NVFP4_ERR_WORKSPACE   (-3) /* workspace missing or too small       */
#define NVFP4_ERR_ARCH        (-4) /* current device is not gfx950         */
#define NVFP4_ERR_HIP         (-5) /* a HIP call failed (text in last_error) */

/* Static description of a status code. */
const char* nvfp4_status_string(nvfp4_status status);
/* Thread-local text of the last failure in this thread ("" if none). */
const char* nvfp4_last_error(void);
/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int nvfp4_version(void);

/* ------------------------------------------------------------------------
 * Weight layout (untimed preparation).
 * README "What We Have", bridge layer: gate/up interleave of the L1 weight
 * at granularity 8 and conversion of B to K-major; "Fused SwiGLU — How It
 * Works": the interleaved output alternates eight gate columns with the eight
 * matching up columns.
 *
 * For each of `groups` matrices src[g] (rows x cols, BF16, row-major),
 * writes dst[g] = transpose (cols x rows).  With interleave_gate_up != 0 the
 * src columns are [gate | up] (cols = 2I, I % 8 == 0) and dst row n holds
 * src column  8*(n/16) + n%8        for n%16 <  8  (gate),
 *             I + 8*(n/16) + n%8 - 8 for n%16 >= 8 (up).
 * Shapes: groups >= 0, rows >= 1, cols >= 1; with interleave cols % 16 == 0.
 * src and dst must not overlap.
 * ---------------------------------------------------------------------- */
nvfp4_status nvfp4_weight_layout(const void* src_bf16, int64_t groups, int64_t rows,
                                 int64_t cols, int interleave_gate_up, void* dst_bf16,
                                 void* stream);

/* ------------------------------------------------------------------------
 * Quantise BF16 -> NVFP4.
 * README "What We Have", bridge layer: BF16 -> NVFP4 with a global scale,
 * a variant with a pre-computed global scale, weights quantised along K;
 * README "Correctness Bugs Fixed": an all-zero 16-block gets scale exactly 0
 * (bug 3); a block whose amax after the global scale is below 6*2^-9 is
 * zeroed, scale 0 (bug 4); CURRENT_BUG.md "What Works": the activation global
 * scale is recomputed per call.
 *
 * x: BF16 [groups*rows_per_group][cols], row r at x + r*ld_x elements
 * (ld_x >= cols, a multiple of 8 so that rows stay 16-byte aligned; ld_x ==
 * cols for a contiguous tensor); every group is quantised along its rows
 * (the contiguous axis) with its own global scale:
 *   gs_in == NULL: gs[g] = fl32(2688 / amax(group g)), or 1 for an all-zero
 *                  group, computed on the device and written to gs_out[g];
 *   gs_in != NULL: device float[groups] used as given and copied to gs_out.
 * Per 16-block (fp32, round-to-nearest-even everywhere):
 *   a_s = amax*gs; zero/underflow (amax == 0 or a_s < 6*2^-9): scale 0x00 and
 *   codes 0; else sf = E4M3(min(a_s/6, 448)), r = gs/sf,
 *   code = signbit(x) << 3 | E2M1(min(|x*r|, 6)).
 * Outputs: q uint8 [groups*rows][cols/2], sf uint8 [groups*rows][cols/16],
 *   gs_out float [groups] (all device).
 * Shapes: groups >= 0, rows_per_group >= 0, cols >= 16, cols % 16 == 0,
 *   ld_x >= cols, ld_x % 8 == 0 (else NVFP4_ERR_SHAPE).
 * Workspace: nvfp4_quantize_workspace_size() bytes (0 allowed with NULL).
 * ---------------------------------------------------------------------- */
size_t nvfp4_quantize_workspace_size(int64_t groups, int64_t rows_per_group, int64_t cols);
nvfp4_status nvfp4_quantize(const void* x_bf16, int64_t groups, int64_t rows_per_group,
                            int64_t cols, int64_t ld_x, const float* gs_in, uint8_t* q,
                            uint8_t* sf, float* gs_out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Weight packing for the grouped GEMM (untimed preparation).
 * README "What We Have", bridge layer: scale assembly and layout conversion
 * of the B operand for the block-scaled MMA.  Here the B operand is re-blocked
 * so that each (n tile, K stage) of the GEMM is one contiguous block.
 *
 * Input: row-major NVFP4 weights q uint8 [E][N][K/2], sf uint8 [E][N][K/16]
 * (K-major, as written by nvfp4_quantize).
 * Output, with Np = N rounded up to NVFP4_PACK_ROWS and S = K / NVFP4_PACK_K:
 *   q_packed  uint8 [E][Np/NVFP4_PACK_ROWS][S][NVFP4_PACK_ROWS][NVFP4_PACK_K/2]
 *   sf_packed uint8 [E][Np/NVFP4_PACK_ROWS][S][NVFP4_PACK_ROWS][NVFP4_PACK_K/16]
 * i.e. byte c of stage s of row n goes to tile n / ROWS, stage s, row n % ROWS;
 * rows N..Np-1 are zero.  Sizes from nvfp4_packed_weight_bytes().
 * Shapes: E >= 1, N >= 1, K % NVFP4_PACK_K == 0.  In and out must not overlap.
 * ---------------------------------------------------------------------- */
#define NVFP4_PACK_ROWS 512
#define NVFP4_PACK_K 128
size_t nvfp4_packed_weight_bytes(int64_t E, int64_t N, int64_t K, size_t* sf_bytes);
nvfp4_status nvfp4_pack_weights(const uint8_t* q, const uint8_t* sf, int64_t E, int64_t N,
                                int64_t K, uint8_t* q_packed, uint8_t* sf_packed, void* stream);

/* ------------------------------------------------------------------------
 * Router: top-k expert ids and routing weights from router logits.
 * README "NVFP4 MegaMoE Kernel", "What We Have", MoE runner step 6 scatters
 * "with routing weights": ids and weights are inputs of the path; this is
 * the step that makes them.  The pages do not define it; the reading used
 * (as for the tiny workload) is top-k of the logits, then a softmax over the
 * k chosen:
 *   topk_ids[t][0..k) = the k largest logits[t][.] in decreasing order,
 *                       equal logits in increasing expert id;
 *   topk_w[t][j] = exp(l_j - l_0) / sum_i exp(l_i - l_0)   (fp32).
 * logits float [T][E] (finite), topk_ids int32 [T][k], topk_w float [T][k].
 * Shapes: T >= 0, 1 <= E <= 1024, 1 <= k <= min(E, 64).
 * No workspace.
 * ---------------------------------------------------------------------- */
nvfp4_status nvfp4_router_topk(const float* logits, int64_t T, int E, int k, int32_t* topk_ids,
                               float* topk_w, void* stream);

/* ------------------------------------------------------------------------
 * Expert offsets and expert-order permutation.
 * README "Correctness Bugs Fixed", bug 5: a histogram, not an O(n x E) mask;
 * README "Key Lessons" 4: quantise compact rows, then place them.
 *
 * topk_ids: device int32 [T][k].  Flat index f = t*k + j.
 * Outputs (device int32):
 *   expert_offsets [E+1]: rows of expert e are [off[e], off[e+1]);
 *                         off[E] = number of valid pairs;
 *   perm [T*k]:           perm[d] = f of row d; rows are ordered by expert,
 *                         and by increasing f inside an expert (stable);
 *   inv_perm [T*k]:       inv_perm[f] = d;
 *   invalid_count [1]:    (nullable) number of ids outside [0, E); those
 *                         pairs are placed after off[E] in increasing f and
 *                         are skipped by the GEMMs and the combine.
 * Shapes: T >= 0, 1 <= k <= 64, 1 <= E <= 4096, T*k < 2^31.
 * Workspace: nvfp4_moe_route_workspace_size() bytes.
 * ---------------------------------------------------------------------- */
size_t nvfp4_moe_route_workspace_size(int64_t T, int k, int E);
nvfp4_status nvfp4_moe_route(const int32_t* topk_ids, int64_t T, int k, int E,
                             int32_t* expert_offsets, int32_t* perm, int32_t* inv_perm,
                             int32_t* invalid_count, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Quantise-and-scatter: the activation quantisation writing expert order.
 * README "Key Lessons" 4: quantise the compact rows, then place them in the
 * expert layout.  Same quantisation as nvfp4_quantize with a per-call global
 * scale (one group); each token row t is quantised once and written to rows
 * d = inv_perm[t*k + j] (j < k) of q/sf that are below expert_offsets[E]
 * (routed pairs; rows of invalid expert ids are not written).  With these
 * rows the L1 grouped GEMM reads its A operand without a gather
 * (a_row_src = NULL), at the price of k copies of every quantised row.
 * moe_expert_forward keeps the compact rows and the gather, which costs the
 * L1 GEMM under 1% of its time, while the k copies cost more than that.
 * x BF16 [T][H]; inv_perm, expert_offsets from nvfp4_moe_route;
 * q uint8 [T*k][H/2], sf uint8 [T*k][H/16], gs_out float [1].
 * Shapes: T >= 0, H % 16 == 0, 1 <= k <= 64, 1 <= E <= 4096, T*k < 2^31.
 * Workspace: nvfp4_quantize_scatter_workspace_size() bytes (0 when T == 0).
 * ---------------------------------------------------------------------- */
size_t nvfp4_quantize_scatter_workspace_size(int64_t T, int64_t H);
nvfp4_status nvfp4_quantize_scatter(const void* x_bf16, int64_t T, int64_t H, int k,
                                    const int32_t* inv_perm, const int32_t* expert_offsets, int E,
                                    uint8_t* q, uint8_t* sf, float* gs_out, void* ws,
                                    size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Expert-grouped NVFP4 GEMM.
 * README "What We Have", grouped GEMM: A(M,K) x B(E,K,N) -> C(M,N), per-16
 * FP8 scales on A and B, per-expert global scales; "Fused SwiGLU — How It
 * Works": SwiGLU epilogue over columns interleaved at 8; "Remaining Steps" 2:
 * NVFP4 quantise in the epilogue (per-16 amax, FP8 scale, FP4 pack).
 *
 * Row d of the grouped operand (0 <= d < off[E], off = expert_offsets) is
 * A row  a_row_src[d] / a_row_div  (a_row_src != NULL, gather), or A row d.
 * For e in [0, E) and d in [off[e], off[e+1]):
 *   acc[d][n] = sum_k dec(A)[d][k] * dec(B[e])[n][k] / (gs_a[0] * gs_b[e]),
 *   dec = E2M1 * E4M3 (exact), fp32 accumulation.
 * A: a_q uint8 [rows_a][K/2], a_sf uint8 [rows_a][K/16], gs_a float[1].
 * B: b_q, b_sf packed by nvfp4_pack_weights from K-major NVFP4 weights
 *    [E][N][K/2] codes and [E][N][K/16] scales; gs_b float[E].
 * epilogue NVFP4_EPI_BF16: c_bf16 [M][N] = bf16_rne(acc).
 * epilogue NVFP4_EPI_SWIGLU_NVFP4: N = 2I interleaved at 8 (see
 *   nvfp4_weight_layout); h[d][c] = silu(gate) * up in fp32 with
 *   gate = acc[d][16*(c/8) + c%8], up = acc[d][16*(c/8) + 8 + c%8];
 *   h is quantised along c with the pre-computed global scale gs_out[0]
 *   (same block rule as nvfp4_quantize) into c_q uint8 [M][I/2] and
 *   c_sf uint8 [M][I/16]; c_debug_f32 (nullable) [M][I] receives h.
 * Rows d >= off[E] are not written.  Requires off[E] <= M (M = rows of C).
 * Shapes: E >= 1, M >= 0, K % 128 == 0, 128 <= K < 2^24, N % 32 == 0,
 *   32 <= N < 2^30; SwiGLU: N % 32 == 0 (I % 16 == 0).
 * A rows are addressed with 32-bit byte offsets, so the A codes must span
 *   less than 4 GiB: without a gather M*K/2 < 2^32 (checked, else
 *   NVFP4_ERR_SHAPE); with a gather every a_row_src[d]/a_row_div must be a
 *   row r of A with (r+1)*K/2 <= 2^32 (a precondition on device data, which
 *   the host cannot read).
 * Unused output pointers of the other epilogue may be NULL.
 * Workspace: at least nvfp4_grouped_gemm_workspace_size() bytes, 4-byte
 *   aligned, caller-owned: the tile scheduler's counters.  Each call first
 *   zeroes them (a small kernel on `stream`), so the contents need no
 *   set-up; calls that share a workspace must be ordered on one stream.  May
 *   be NULL only when M == 0.
 * Tiles: 512 weight rows x 128 token rows; 32-token tiles when the experts
 *   average at most 32 rows (decode-sized batches); 64-token tiles for a
 *   BF16-epilogue launch whose 128-token tiles would leave half the CUs idle
 *   (a dense linear of a few thousand rows).
 * Split K (BF16 epilogue only): when even 64-token tiles leave half the CUs
 *   idle (e.g. a dense linear of about a thousand rows) and
 *   ws_bytes >= nvfp4_grouped_gemm_splitk_workspace_size
 *   (same epilogue, M, N, K, E; current device), each tile's K range is cut
 *   into up to 4 parts whose fp32 partial sums (scaled by the global scales)
 *   go to the workspace; a second kernel on `stream` sums them in part order
 *   and rounds to BF16.  The result differs from the unsplit one only by
 *   fp32 summation order.  With a smaller workspace K is never split.
 * ---------------------------------------------------------------------- */
#define NVFP4_EPI_BF16 0
#define NVFP4_EPI_SWIGLU_NVFP4 1
size_t nvfp4_grouped_gemm_workspace_size(void);
/* Workspace that lets a launch of this shape split K on the current device
 * (nvfp4_grouped_gemm_workspace_size() when it would not split, or when the
 * device cannot be queried). */
size_t nvfp4_grouped_gemm_splitk_workspace_size(int epilogue, int64_t M, int64_t N, int64_t K,
                                                int E);
nvfp4_status nvfp4_grouped_gemm(int epilogue, const uint8_t* a_q, const uint8_t* a_sf,
                                const float* gs_a, const int32_t* a_row_src, int a_row_div,
                                const int32_t* expert_offsets, int E, int64_t M, int64_t N,
                                int64_t K, const uint8_t* b_q, const uint8_t* b_sf,
                                const float* gs_b, const float* gs_out, void* c_bf16,
                                uint8_t* c_q, uint8_t* c_sf, float* c_debug_f32, void* ws,
                                size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * MX variant: NVFP4 re-encoded for the block-scaled FP4 matrix instructions.
 * README "What We Have", grouped GEMM, carries E2M1 values with E4M3 scales
 * per 16 elements; gfx950's scaled FP4 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4)
 * takes E2M1 values with one power-of-two E8M0 scale per 32 elements (OCP
 * Microscaling).  These entry points re-encode NVFP4 data into that form and
 * run the grouped GEMM and the whole forward on it.  The re-encoding rounds:
 * results approximate the NVFP4 ones (they are not the NVFP4 results up to
 * summation order, as nvfp4_grouped_gemm's are).
 *
 * nvfp4_to_mx: q uint8 [rows][cols/2] E2M1 codes and sf uint8 [rows][cols/16]
 * E4M3 scales (as written by nvfp4_quantize) -> q_mx [rows][cols/2] and
 * sc_mx [rows][cols/16].  Per 32-block j of a row (NVFP4 blocks 2j, 2j+1):
 *   u_i = E2M1(q_i) * E4M3(sf) (exact); amax = max |u_i|;
 *   amax == 0: scale byte 0, codes 0;
 *   else X = 2^(floor(log2 amax) - 2) (MX conversion, E2M1 emax 2), E8M0 byte
 *   floor(log2 amax) - 2 + 127, code_i = signbit(q_i) << 3 | E2M1(min(|u_i|/X, 6))
 *   (nearest, ties to the even code);
 *   the E8M0 byte is stored at sc_mx bytes 2j and 2j+1 (the NVFP4 scale
 *   layout, so nvfp4_pack_weights packs MX weights unchanged).
 * The global scale of the NVFP4 data carries over unchanged.
 * Shapes: rows >= 0, cols % 32 == 0.  In place (q_mx == q, sc_mx == sf) is
 * allowed; otherwise outputs must not overlap inputs.  No workspace.
 *
 * nvfp4_mx_grouped_gemm: nvfp4_grouped_gemm (same arguments, rules, shapes,
 * split K and workspace) on MXFP4 operands: a_q/a_sc from nvfp4_to_mx,
 * b_q/b_sc = nvfp4_pack_weights of nvfp4_to_mx output;
 *   acc[d][n] = sum_k E2M1(a) * E8M0(a) * E2M1(b) * E8M0(b) / (gs_a * gs_b[e]).
 * The SwiGLU epilogue still writes NVFP4 (E4M3 scales) with gs_out.
 *
 * moe_expert_forward_mx: moe_expert_forward (same arguments, workspace and
 * taps) with w1/w2 packed from nvfp4_to_mx of the NVFP4 weights; the
 * quantised x and the requantised h are re-encoded in place with nvfp4_to_mx
 * before the GEMM that reads them, so the taps a_q/a_sf and h_q/h_sf receive
 * the MX forms.
 * ---------------------------------------------------------------------- */
nvfp4_status nvfp4_to_mx(const uint8_t* q, const uint8_t* sf, int64_t rows, int64_t cols,
                         uint8_t* q_mx, uint8_t* sc_mx, void* stream);
nvfp4_status nvfp4_mx_grouped_gemm(int epilogue, const uint8_t* a_q, const uint8_t* a_sc,
                                   const float* gs_a, const int32_t* a_row_src, int a_row_div,
                                   const int32_t* expert_offsets, int E, int64_t M, int64_t N,
                                   int64_t K, const uint8_t* b_q, const uint8_t* b_sc,
                                   const float* gs_b, const float* gs_out, void* c_bf16,
                                   uint8_t* c_q, uint8_t* c_sf, float* c_debug_f32, void* ws,
                                   size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Routing-weighted combine.
 * README "What We Have", MoE runner step 6: scatter with routing weights.
 *
 * out[t][n] = bf16_rne( sum_{j=0..k-1} w[t][j] * y[inv_perm[t*k+j]][n] ),
 * fp32 sum in slot order j; rows inv_perm >= expert_offsets[E] (invalid
 * expert ids) contribute nothing.
 * y: BF16 [T*k][H] in expert order; topk_w float [T][k]; out BF16 [T][H].
 * Shapes: T >= 0, 1 <= k <= 64, E >= 1, H >= 8, H % 8 == 0.
 * ---------------------------------------------------------------------- */
nvfp4_status nvfp4_moe_combine(const void* y_bf16, const int32_t* inv_perm,
                               const float* topk_w, const int32_t* expert_offsets, int64_t T,
                               int k, int E, int64_t H, void* out_bf16, void* stream);

/* ------------------------------------------------------------------------
 * The whole expert forward.
 * README "What We Have", MoE runner: quantise -> L1 -> SiLU(gate)*up ->
 * requantise -> L2 -> weighted scatter; here L1, SwiGLU and the requantise
 * are one fused kernel.
 *
 * x BF16 [T][H]; topk_ids int32 [T][k]; topk_w float [T][k];
 * w1_q, w1_sf: nvfp4_pack_weights of the interleaved, K-major L1 weight
 *   ([E][2I][H/2] codes, [E][2I][H/16] scales); gs_w1 [E];
 * w2_q, w2_sf: nvfp4_pack_weights of the K-major L2 weight ([E][H][I/2],
 *   [E][H][I/16]); gs_w2 [E];
 * gs_h float[1]: global scale of the requantised L2 input (pre-computed);
 * out BF16 [T][H].
 * Steps on `stream`: quantize x with a per-call gs and route (the bytes of
 *   nvfp4_quantize + nvfp4_moe_route, in three launches that also clear the
 *   GEMMs' tile counters) -> grouped GEMM L1 (SwiGLU + NVFP4 epilogue, A rows
 *   gathered by perm/k) -> grouped GEMM L2 (BF16) -> combine.
 * taps (nullable): every non-NULL member receives that intermediate (the
 *   kernels write straight into it instead of the workspace).
 * Shapes: T >= 0, H % 128 == 0, I % 128 == 0, 1 <= k <= 64, 1 <= E <= 4096,
 *   T*k < 2^31, H < 2^24, I < 2^23, and the quantised x and h below 4 GiB
 *   each (T*H/2 < 2^32, T*k*I/2 < 2^32; else NVFP4_ERR_SHAPE).
 * Workspace: moe_expert_forward_workspace_size() bytes.
 * ---------------------------------------------------------------------- */
typedef struct nvfp4_moe_taps {
    uint8_t* a_q;            /* [T][H/2]   */
    uint8_t* a_sf;           /* [T][H/16]  */
    float* gs_a;             /* [1]        */
    int32_t* expert_offsets; /* [E+1]      */
    int32_t* perm;           /* [T*k]      */
    int32_t* inv_perm;       /* [T*k]      */
    int32_t* invalid_count;  /* [1]        */
    float* h_f32;            /* [T*k][I]   */
    uint8_t* h_q;            /* [T*k][I/2] */
    uint8_t* h_sf;           /* [T*k][I/16]*/
    void* y_bf16;            /* [T*k][H]   */
} nvfp4_moe_taps;

size_t moe_expert_forward_workspace_size(int64_t T, int64_t H, int64_t I, int E, int k);
nvfp4_status moe_expert_forward(const void* x_bf16, int64_t T, int64_t H, int64_t I, int E,
                                int k, const int32_t* topk_ids, const float* topk_w,
                                const uint8_t* w1_q, const uint8_t* w1_sf, const float* gs_w1,
                                const uint8_t* w2_q, const uint8_t* w2_sf, const float* gs_w2,
                                const float* gs_h, void* out_bf16, const nvfp4_moe_taps* taps,
                                void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * The expert forward with a shared expert.
 * README "NVFP4 MegaMoE Kernel", "What We Have": the single-expert NVFP4
 * linear serves the shared experts; CURRENT_BUG.md "What Works" lists the
 * shared expert among the NVFP4 layers.  Every token also goes through one
 * shared expert (an expert MLP of the same shape), whose output is added in
 * the combine:
 *   out[t] = bf16_rne( sum_{j<k} w[t][j] * y[route j of t] + y_shared[t] ),
 * fp32 sum in slot order with the shared term last.
 * Weights: E + 1 experts packed as for moe_expert_forward, the routed ones
 * first and the shared expert last (index E); gs_w1, gs_w2 [E+1].
 * Internally every token gets slot k = expert E with weight 1 (routed ids
 * outside [0, E) stay invalid) and the forward runs with E + 1 experts and
 * k + 1 slots: taps are sized for T*(k+1) rows and E+2 offsets.
 * Shapes: as moe_expert_forward with 1 <= k <= 63, 1 <= E <= 4095.
 * Workspace: moe_expert_forward_shared_workspace_size() bytes.
 * ---------------------------------------------------------------------- */
size_t moe_expert_forward_shared_workspace_size(int64_t T, int64_t H, int64_t I, int E, int k);
nvfp4_status moe_expert_forward_shared(const void* x_bf16, int64_t T, int64_t H, int64_t I, int E,
                                       int k, const int32_t* topk_ids, const float* topk_w,
                                       const uint8_t* w1_q, const uint8_t* w1_sf,
                                       const float* gs_w1, const uint8_t* w2_q,
                                       const uint8_t* w2_sf, const float* gs_w2, const float* gs_h,
                                       void* out_bf16, const nvfp4_moe_taps* taps, void* ws,
                                       size_t ws_bytes, void* stream);

/* MX variant of moe_expert_forward (see nvfp4_to_mx above). */
nvfp4_status moe_expert_forward_mx(const void* x_bf16, int64_t T, int64_t H, int64_t I, int E,
                                   int k, const int32_t* topk_ids, const float* topk_w,
                                   const uint8_t* w1_q, const uint8_t* w1_sc, const float* gs_w1,
                                   const uint8_t* w2_q, const uint8_t* w2_sc, const float* gs_w2,
                                   const float* gs_h, void* out_bf16, const nvfp4_moe_taps* taps,
                                   void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * The expert forward without a caller workspace.
 * For callers that cannot allocate device memory: code under hipGraph
 * capture, tight serving loops, harnesses that forbid allocation.
 *
 * Same arguments (without ws / ws_bytes), steps, taps, results and error
 * behaviour as moe_expert_forward.  Its workspace is a static device array
 * of NVFP4_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds
 * until the process ends; the call allocates and frees nothing (its first
 * call on a device looks up the array's address on that device).
 * Requires moe_expert_forward_workspace_size(T, H, I, E, k) <=
 *   NVFP4_NOALLOC_SCRATCH_BYTES (at H = 7168, I = 2048, k = 8 that is
 *   T <= 524), else NVFP4_ERR_WORKSPACE and nothing is enqueued.
 * All calls on one GPU share its array, which keeps the last call's
 * contents (nothing in it needs to start at zero: every region is written
 * before it is read, and the GEMMs' tile counters are cleared by the first
 * kernel of each call).  Calls ordered on one stream are safe; calls that overlap on
 * one GPU (unordered streams, several host threads) race on the array and
 * give wrong results.
 * ---------------------------------------------------------------------- */
#define NVFP4_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
nvfp4_status moe_expert_forward_noalloc(const void* x_bf16, int64_t T, int64_t H, int64_t I, int E,
                                        int k, const int32_t* topk_ids, const float* topk_w,
                                        const uint8_t* w1_q, const uint8_t* w1_sf,
                                        const float* gs_w1, const uint8_t* w2_q,
                                        const uint8_t* w2_sf, const float* gs_w2,
                                        const float* gs_h, void* out_bf16,
                                        const nvfp4_moe_taps* taps, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4MOE_H */
