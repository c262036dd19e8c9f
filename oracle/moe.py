"""The MoE expert forward: quantise -> L1 -> SwiGLU -> requantise -> L2 -> combine.

README ("NVFP4 MegaMoE Kernel"), section "What We Have", MoE runner: the
forward quantises the BF16 input to NVFP4, runs the L1 grouped GEMM over the
interleaved gate/up weight, applies SiLU(gate) * up, re-quantises to NVFP4,
runs the L2 (down) grouped GEMM to BF16 and scatters back with the routing
weights.  Section "What We Have", grouped GEMM: A(M,K) x B(E,K,N) -> C(M,N)
with per-16 FP8 scales on both sides and per-expert global scales.
Section "Fused SwiGLU — How It Works": gate and up are paired explicitly;
"Key Lessons" 10: SiLU on all columns is not SwiGLU.

Precision: operands are decoded exactly (E2M1 * E4M3 in float64); sums run in
float64; the global scales divide the sum.  Readings of what the pages leave
open:
  * the requantised L2 input uses a caller-supplied global scale gs_h (the
    pre-computed-scale quantiser mode), and is quantised from the float32
    rounding of the float64 SwiGLU value (no BF16 step in between);
  * L2 output y and the combined output are rounded to BF16 (nearest, ties to
    even) from float64; the combine sums in slot order j = 0..k-1;
  * only h (I columns) is produced; the README's BF16 stage also kept
    silu(gate) in the gate columns, which the next GEMM never reads.
"""

import numpy as np

from .formats import round_to_bf16, bf16_bits_to_f32
from .quantize import quantize_nvfp4, quantize_blocks, pack_codes, block_values
from .layout import interleave_l1, k_major, deinterleave_cols
from .route import route

F32 = np.float32


def silu(z):
    """SiLU in float64: z / (1 + exp(-z))."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def prepare_expert_weights(w1_e, w2_e):
    """One expert's weights, logical BF16 bits W1 (K, 2I) = [gate | up] and
    W2 (I, K), to the NVFP4 operands the grouped GEMMs read:
    W1 interleaved at 8 and K-major (2I, K); W2 K-major (K, I); each quantised
    along its contiguous axis with its own per-call global scale."""
    w1i = interleave_l1(w1_e[None])[0]
    w2k = k_major(w2_e[None])[0]
    w1_q, w1_sf, gs1 = quantize_nvfp4(w1i)
    w2_q, w2_sf, gs2 = quantize_nvfp4(w2k)
    return dict(w1_q=w1_q, w1_sf=w1_sf, gs_w1=gs1[0], w2_q=w2_q, w2_sf=w2_sf, gs_w2=gs2[0])


def prepare_weights(w1, w2):
    """All experts: W1 (E, K, 2I), W2 (E, I, K) BF16 bits -> stacked operands."""
    per = [prepare_expert_weights(w1[e], w2[e]) for e in range(w1.shape[0])]
    return {k: np.stack([p[k] for p in per]) for k in per[0]}


def nvfp4_matmul(a_q, a_sf, gs_a, b_q, b_sf, gs_b):
    """C = dec(A) @ dec(B).T / (gs_a * gs_b) in float64, A (R, K), B (N, K)."""
    acc = block_values(a_q, a_sf) @ block_values(b_q, b_sf).T
    return acc / (np.float64(gs_a) * np.float64(gs_b))


def dense_linear(a_q, a_sf, gs_a, b_q, b_sf, gs_b):
    """Single-expert NVFP4 linear with BF16 output (E = 1 grouped GEMM)."""
    return round_to_bf16(nvfp4_matmul(a_q, a_sf, gs_a, b_q, b_sf, gs_b))


def l1_swiglu(a_rows_q, a_rows_sf, gs_a, w1_q, w1_sf, gs_w1):
    """L1 for one expert's rows, then SwiGLU.  Returns h as float32 (R, I)."""
    acc = nvfp4_matmul(a_rows_q, a_rows_sf, gs_a, w1_q, w1_sf, gs_w1)
    gate, up = deinterleave_cols(acc)
    return (silu(gate) * up).astype(F32)


def l2(h_q, h_sf, gs_h, w2_q, w2_sf, gs_w2):
    """L2 for one expert's rows: BF16 bits (R, K)."""
    return round_to_bf16(nvfp4_matmul(h_q, h_sf, gs_h, w2_q, w2_sf, gs_w2))


def combine(y_bits, inv_perm, topk_w, n_valid):
    """out[t] = sum_j w[t, j] * y[inv_perm[t*k + j]] in float64, slot order,
    rows d >= n_valid (invalid expert ids) contributing nothing; BF16 bits."""
    T, k = topk_w.shape
    y = bf16_bits_to_f32(y_bits).astype(np.float64)
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    w = np.asarray(topk_w, dtype=np.float32).astype(np.float64)
    for j in range(k):
        d = inv_perm.reshape(T, k)[:, j]
        ok = d < n_valid
        rows = np.where(ok[:, None], y[np.minimum(d, y.shape[0] - 1)], 0.0)
        out += w[:, j:j + 1] * rows
    return round_to_bf16(out)


def moe_forward(x_bits, topk_ids, topk_w, wts, gs_h, E, experts=None):
    """The whole expert forward on the CPU.

    x_bits (T, K) BF16 bits; topk_ids (T, k); topk_w (T, k) float32;
    wts: per-expert operands as returned by ``prepare_weights`` (indexable by
    expert); gs_h: float32 global scale of the requantised L2 input.
    ``experts`` restricts L1/L2 to a subset (rows of other experts stay zero
    in h/y and the combine is then only meaningful for tokens whose experts
    are all in the subset).
    Returns a dict with every intermediate.
    """
    T, k = topk_ids.shape
    K = x_bits.shape[1]
    a_q, a_sf, gs_a = quantize_nvfp4(x_bits)
    gs_a = gs_a[0]
    offsets, perm, inv_perm, n_invalid = route(topk_ids, E)
    M = T * k
    I = wts["w1_q"][0].shape[0] // 2
    h = np.zeros((M, I), dtype=F32)
    h_q = np.zeros((M, I // 2), dtype=np.uint8)
    h_sf = np.zeros((M, I // 16), dtype=np.uint8)
    y = np.zeros((M, K), dtype=np.uint16)
    gs_h = F32(gs_h)
    for e in range(E) if experts is None else experts:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        tok = perm[lo:hi] // k
        h_e = l1_swiglu(a_q[tok], a_sf[tok], gs_a,
                        wts["w1_q"][e], wts["w1_sf"][e], wts["gs_w1"][e])
        c_e, s_e = quantize_blocks(h_e, gs_h)
        h[lo:hi], h_q[lo:hi], h_sf[lo:hi] = h_e, pack_codes(c_e), s_e
        y[lo:hi] = l2(h_q[lo:hi], s_e, gs_h, wts["w2_q"][e], wts["w2_sf"][e], wts["gs_w2"][e])
    out = combine(y, inv_perm, topk_w, int(offsets[E]))
    return dict(a_q=a_q, a_sf=a_sf, gs_a=gs_a, offsets=offsets, perm=perm,
                inv_perm=inv_perm, n_invalid=n_invalid, h=h, h_q=h_q, h_sf=h_sf,
                y=y, out=out)


def moe_forward_shared(x_bits, topk_ids, topk_w, wts, gs_h, E):
    """The expert forward with one shared expert added in the combine.

    README ("NVFP4 MegaMoE Kernel"), section "What We Have": the single-expert
    NVFP4 linear serves the shared experts; CURRENT_BUG.md, "What Works",
    lists the shared expert among the NVFP4 layers.  Reading: the shared
    expert is an expert MLP of the routed shape (L1 -> SwiGLU -> requantise
    -> L2) applied to every token's quantised row, and its BF16 output is
    added with weight 1 after the k routed terms:
        out[t] = bf16( sum_j w[t, j] * y[route j of t] + y_shared[t] ).
    ``wts`` holds E + 1 experts; index E is the shared one.
    """
    T, k = topk_ids.shape
    routed = moe_forward(x_bits, topk_ids, topk_w, wts, gs_h, E)
    a_q, a_sf, gs_a = routed["a_q"], routed["a_sf"], routed["gs_a"]
    gs_h = F32(gs_h)
    h_s = l1_swiglu(a_q, a_sf, gs_a, wts["w1_q"][E], wts["w1_sf"][E], wts["gs_w1"][E])
    c_s, s_s = quantize_blocks(h_s, gs_h)
    y_s = l2(pack_codes(c_s), s_s, gs_h, wts["w2_q"][E], wts["w2_sf"][E], wts["gs_w2"][E])
    y = bf16_bits_to_f32(routed["y"]).astype(np.float64)
    w = np.asarray(topk_w, dtype=np.float32).astype(np.float64)
    n_valid = int(routed["offsets"][E])
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    for j in range(k):
        d = routed["inv_perm"].reshape(T, k)[:, j]
        ok = d < n_valid
        out += w[:, j:j + 1] * np.where(ok[:, None], y[np.minimum(d, y.shape[0] - 1)], 0.0)
    out += bf16_bits_to_f32(y_s).astype(np.float64)
    routed.update(h_shared=h_s, y_shared=y_s, out=round_to_bf16(out))
    return routed
