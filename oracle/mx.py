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
