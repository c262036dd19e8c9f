"""MX variant: NVFP4 re-encoded to MXFP4 (E2M1 values, one E8M0 scale per 32).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Why this exists.  The project's grouped GEMM carries NVFP4: E2M1 values with
one E4M3 scale per 16 elements and a global scale (README "NVFP4 MegaMoE
Kernel", section "What We Have", grouped GEMM).  CDNA4's block-scaled matrix
instructions take E2M1 operands with one power-of-two (E8M0) scale per 32
elements instead, the OCP Microscaling (MX) layout.  This module defines the
re-encoding of NVFP4 data into that layout and the exact product of the
result, so that a GPU path built on those instructions has an oracle of its
own, and so the error the re-encoding adds can be measured against the exact
NVFP4 product.

Formats (OCP Microscaling Formats (MX) v1.0 specification):
  * E8M0 scale byte b: value 2**(b - 127); 0xFF is NaN;
  * an MX block is 32 consecutive elements along the contiguous axis sharing
    one E8M0 scale X; element value = E2M1(code) * X.

Readings (the pages do not define an MX encoding at all):
  * what is re-encoded is the NVFP4 block value u = E2M1 * E4M3, without the
    global scale, which stays a separate fp32 factor of the GEMM;
  * the shared scale follows the MX specification's conversion: X =
    2**(floor(log2(amax32)) - 2), where 2 is the exponent of E2M1's largest
    normal value 6 = 1.5 * 2**2; elements are then rounded to the nearest
    E2M1 value of u / X with ties to the even code, magnitudes above 6
    saturating to 6; the sign is the sign bit of the NVFP4 code;
  * a 32-block whose values are all zero gets scale byte 0x00 and zero codes;
  * MX block j covers NVFP4 blocks 2j and 2j + 1 of the same row.
"""

import numpy as np

from .formats import e2m1_decode, e2m1_encode_magnitude
from .quantize import unpack_codes, pack_codes, block_values

MX_BLOCK = 32
E2M1_EMAX = 2           # 6 = 1.5 * 2**2


def e8m0_decode(byte):
    """Value (float64) of an E8M0 scale byte: 2**(b - 127); 0xFF is NaN."""
    b = np.asarray(byte, dtype=np.int64)
    v = np.ldexp(1.0, (b - 127).astype(np.int32))
    return np.where(b == 0xFF, np.nan, v)


def mx_encode_values(u, sign):
    """MX-encode rows of exact values.

    u: float64 (R, C) magnitudes-with-sign of the elements, C % 32 == 0;
    sign: (R, C) 0/1 sign bits (kept also for zero magnitudes).
    Returns (codes uint8 (R, C) 4-bit, sc uint8 (R, C/32) E8M0 bytes).
    """
    u = np.asarray(u, dtype=np.float64)
    R, C = u.shape
    if C % MX_BLOCK:
        raise ValueError("cols must be a multiple of 32")
    blocks = np.abs(u).reshape(R, C // MX_BLOCK, MX_BLOCK)
    amax = np.max(blocks, axis=-1)
    zero = amax == 0
    # floor(log2(amax)) exactly: frexp gives amax = m * 2**e with 0.5 <= m < 1
    _, e = np.frexp(np.where(zero, 1.0, amax))
    shared = (e - 1) - E2M1_EMAX
    sc = np.where(zero, 0, shared + 127).astype(np.int64)
    if np.any((sc < 1) & ~zero) or np.any(sc > 254):
        raise ValueError("shared exponent outside the E8M0 range")
    X = np.ldexp(1.0, np.where(zero, 0, shared).astype(np.int32))
    v = blocks / X[..., None]                         # exact: X is a power of two
    mag = e2m1_encode_magnitude(np.minimum(v, 6.0))
    codes = (np.asarray(sign, dtype=np.uint8).reshape(R, C // MX_BLOCK, MX_BLOCK) << 3) | mag
    codes = np.where(zero[..., None], np.uint8(0), codes).astype(np.uint8)
    return codes.reshape(R, C), sc.astype(np.uint8)


def nvfp4_to_mx(q, sf):
    """Re-encode packed NVFP4 data (q (R, C/2), sf (R, C/16) E4M3) to MXFP4:
    returns (q_mx (R, C/2) packed like NVFP4 codes, sc (R, C/32) E8M0)."""
    u = block_values(q, sf)                           # exact E2M1 * E4M3
    sign = unpack_codes(q) >> 3
    codes, sc = mx_encode_values(u, sign)
    return pack_codes(codes), sc


def mx_block_values(q_mx, sc):
    """Exact float64 E2M1 * E8M0 values of packed MXFP4 data."""
    codes = unpack_codes(q_mx)
    R, C = codes.shape
    vals = e2m1_decode(codes).reshape(R, C // MX_BLOCK, MX_BLOCK)
    return (vals * e8m0_decode(sc)[..., None]).reshape(R, C)


def mx_matmul(a_q, a_sc, gs_a, b_q, b_sc, gs_b):
    """C = dec(A) @ dec(B).T / (gs_a * gs_b) in float64 on MXFP4 operands,
    A (R, K), B (N, K); the global scales are those of the NVFP4 data."""
    a = mx_block_values(a_q, a_sc)
    b = mx_block_values(b_q, b_sc)
    return (a @ b.T) / (np.float64(gs_a) * np.float64(gs_b))


def prepare_weights_mx(wts):
    """Per-expert NVFP4 weight operands (``moe.prepare_weights``) re-encoded:
    the global scales carry over."""
    out = dict(wts)
    for q, s in (("w1_q", "w1_sf"), ("w2_q", "w2_sf")):
        pairs = [nvfp4_to_mx(wts[q][e], wts[s][e]) for e in range(len(wts[q]))]
        out[q] = np.stack([p[0] for p in pairs])
        out[s] = np.stack([p[1] for p in pairs])
    return out


def moe_forward_mx(x_bits, topk_ids, topk_w, wts_mx, gs_h, E):
    """The MX variant of ``moe.moe_forward``: x is quantised to NVFP4 as
    there and re-encoded; L1 and L2 are exact products of MX operands
    (``wts_mx`` from ``prepare_weights_mx``); the SwiGLU output is requantised
    to NVFP4 with gs_h as there and re-encoded before L2.  Returns the same
    intermediates (a_q/a_sf and h_q/h_sf in their MX forms, scales per 32)."""
    from .moe import silu, combine
    from .layout import deinterleave_cols
    from .route import route
    from .formats import round_to_bf16
    from .quantize import quantize_nvfp4, quantize_blocks

    T, k = topk_ids.shape
    K = x_bits.shape[1]
    a_q, a_sf, gs_a = quantize_nvfp4(x_bits)
    gs_a = gs_a[0]
    a_q, a_sc = nvfp4_to_mx(a_q, a_sf)
    offsets, perm, inv_perm, n_invalid = route(topk_ids, E)
    M = T * k
    I = wts_mx["w1_q"][0].shape[0] // 2
    h = np.zeros((M, I), dtype=np.float32)
    h_q = np.zeros((M, I // 2), dtype=np.uint8)
    h_sc = np.zeros((M, I // 32), dtype=np.uint8)
    y = np.zeros((M, K), dtype=np.uint16)
    gs_h = np.float32(gs_h)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        tok = perm[lo:hi] // k
        acc = mx_matmul(a_q[tok], a_sc[tok], gs_a, wts_mx["w1_q"][e], wts_mx["w1_sf"][e],
                        wts_mx["gs_w1"][e])
        gate, up = deinterleave_cols(acc)
        h_e = (silu(gate) * up).astype(np.float32)
        c_e, s_e = quantize_blocks(h_e, gs_h)
        hq_e, hsc_e = nvfp4_to_mx(pack_codes(c_e), s_e)
        h[lo:hi], h_q[lo:hi], h_sc[lo:hi] = h_e, hq_e, hsc_e
        y[lo:hi] = round_to_bf16(mx_matmul(hq_e, hsc_e, gs_h, wts_mx["w2_q"][e],
                                           wts_mx["w2_sf"][e], wts_mx["gs_w2"][e]))
    out = combine(y, inv_perm, topk_w, int(offsets[E]))
    return dict(a_q=a_q, a_sc=a_sc, gs_a=gs_a, offsets=offsets, perm=perm, inv_perm=inv_perm,
                n_invalid=n_invalid, h=h, h_q=h_q, h_sc=h_sc, y=y, out=out)
