"""NVFP4 quantisation: global scale, per-16 E4M3 block scales, E2M1 codes.

Follows the README ("NVFP4 MegaMoE Kernel"):
  * section "What We Have" (bridge layer): BF16 -> NVFP4 with a global scale,
    a variant with a pre-computed global scale, weights quantised along K;
  * section "What We Have" (grouped GEMM): one FP8 scale per 16 elements and
    per-expert global scales;
  * section "Correctness Bugs Fixed", bug 3: an all-zero block gets the exact
    FP8 scale 0 (no clamp to a tiny positive value);
  * same table, bug 4: an underflow block (amax < 6 * 2**-9) is zeroed
    instead of dividing by a tiny scale;
  * same table, bug 2: requantising the dequantised values reproduces every
    byte;
  * CURRENT_BUG.md, "What Works": the activation global scale is recomputed
    on every call.

Readings of what the pages leave open (each also listed in the design notes):
  * global scale gs = fl32(2688 / amax) with 2688 = 448 * 6 (E4M3 max times
    E2M1 max); gs = 1 for an all-zero tensor;
  * the underflow test compares the block amax AFTER the global scale,
    fl32(amax_b * gs), with 6 * 2**-9, strictly (<), in fp32;
  * an underflow block also gets scale byte 0x00, so sf == 0 <=> all codes 0;
  * fp32 operation order: a_s = amax_b*gs; t = a_s/6; sf = E4M3(min(t,448));
    r = gs/dec(sf); v = x*r; code = sign(x) | E2M1(min(|v|, 6)); every
    operation rounds to nearest even; the sign is the sign bit of x (so -0.0
    and negative values that round to magnitude 0 keep code 0x8);
  * packing: two codes per byte along the contiguous axis, the even element in
    the low nibble.
"""

import numpy as np

from .formats import (e2m1_decode, e2m1_encode_magnitude, e4m3_decode,
                      e4m3_encode_nonneg, bf16_bits_to_f32)

F32 = np.float32
BLOCK = 16
UNDERFLOW = F32(6.0 * 2.0 ** -9)     # E2M1 max times E4M3 smallest subnormal
GS_NUMERATOR = F32(448.0 * 6.0)      # E4M3 max times E2M1 max


def as_f32(x):
    """float32 view of the input: raw bfloat16 bit patterns (uint16) are
    widened exactly; float arrays must already hold float32 values."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x)
    if x.dtype != np.float32:
        raise TypeError("quantiser input must be bf16 bits (uint16) or float32")
    return x


def global_scale(x):
    """Per-tensor global scale gs = fl32(2688 / max|x|), or 1 if x is all zero."""
    xf = as_f32(x)
    amax = F32(np.max(np.abs(xf))) if xf.size else F32(0)
    if amax == 0:
        return F32(1.0)
    return F32(GS_NUMERATOR / amax)


def quantize_blocks(x, gs):
    """Quantise the rows of x (R, C), C % 16 == 0, with global scale(s) gs.

    gs is a float32 scalar or a float32 array broadcastable to (R,).
    Returns (codes uint8 (R, C) one 4-bit code per element, sf uint8 (R, C/16)).
    """
    xf = as_f32(x)
    R, C = xf.shape
    if C % BLOCK:
        raise ValueError("cols must be a multiple of 16")
    gs = np.asarray(gs, dtype=F32)
    if gs.ndim == 0:
        gs = np.full((R,), gs, dtype=F32)
    gs = gs.reshape(R, 1)
    blocks = xf.reshape(R, C // BLOCK, BLOCK)

    amax_b = np.max(np.abs(blocks), axis=-1)                 # exact
    a_s = (amax_b * gs).astype(F32)                          # fl32(amax_b * gs)
    zeroed = (amax_b == 0) | (a_s < UNDERFLOW)               # bugs 3 and 4
    t = (a_s / F32(6.0)).astype(F32)                         # fl32(a_s / 6)
    t_sat = np.minimum(t, F32(448.0))
    sf = e4m3_encode_nonneg(np.where(zeroed, 0.0, t_sat))
    sf = np.where(zeroed, np.uint8(0), sf).astype(np.uint8)
    sd = e4m3_decode(sf).astype(F32)                         # exact
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (gs / np.where(zeroed, F32(1.0), sd)).astype(F32)  # fl32(gs / sd)
    v = (blocks * r[..., None]).astype(F32)                  # fl32(x * r)
    mag = e2m1_encode_magnitude(np.minimum(np.abs(v), F32(6.0)))
    sign = np.signbit(blocks).astype(np.uint8) << 3
    codes = (sign | mag).astype(np.uint8)
    codes = np.where(zeroed[..., None], np.uint8(0), codes)
    return codes.reshape(R, C), sf


def pack_codes(codes):
    """(R, C) 4-bit codes -> (R, C/2) bytes; element 2j in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def unpack_codes(q):
    """(R, C/2) bytes -> (R, C) 4-bit codes."""
    q = np.asarray(q, dtype=np.uint8)
    out = np.empty((q.shape[0], q.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = q & 0xF
    out[:, 1::2] = q >> 4
    return out


def quantize_nvfp4(x, groups=1, gs_in=None):
    """Quantise x (groups*rows, C) group by group (a group is a tensor, or one
    expert's weight matrix), each with its own global scale.

    gs_in None: the global scale of each group comes from the group's amax
    (the per-call mode); otherwise gs_in (float32, shape (groups,)) is used as
    given (the pre-computed-scale mode).
    Returns (q (R, C/2) uint8, sf (R, C/16) uint8, gs (groups,) float32).
    """
    xf = as_f32(x)
    R, C = xf.shape
    if R % groups:
        raise ValueError("rows must divide evenly into groups")
    rpg = R // groups
    if gs_in is None:
        gs = np.array([global_scale(xf[g * rpg:(g + 1) * rpg]) for g in range(groups)],
                      dtype=F32)
    else:
        gs = np.asarray(gs_in, dtype=F32).reshape(groups)
    codes, sf = quantize_blocks(xf, np.repeat(gs, rpg))
    return pack_codes(codes), sf, gs


def block_values(q, sf):
    """Exact float64 E2M1 * E4M3 products (no global scale) of packed data."""
    codes = unpack_codes(q)
    R, C = codes.shape
    vals = e2m1_decode(codes).reshape(R, C // BLOCK, BLOCK)
    scale = e4m3_decode(sf)[..., None]
    return (vals * scale).reshape(R, C)


def dequantize(q, sf, gs):
    """float64 values x_hat = E2M1 * E4M3 / gs; gs scalar or per row."""
    gs = np.asarray(gs, dtype=np.float64)
    if gs.ndim == 1:
        gs = gs.reshape(-1, 1)
    return block_values(q, sf) / gs


# --------------------------------------------------- decision margins (tests)

_E2M1_MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def _e4m3_midpoints():
    vals = e4m3_decode(np.arange(0x7F))
    return (vals[:-1] + vals[1:]) / 2.0


def near_ties(x, gs, tau):
    """Where a perturbation of relative size ``tau`` in x could change the
    quantised result, from the oracle's own fp32 quantities.

    Returns (elem (R, C) bool, block (R, C/16) bool): ``block`` marks blocks
    whose scale decision (underflow test or E4M3 rounding of a_s/6) lies within
    tau (relative) of a boundary; ``elem`` marks elements whose scaled value v
    lies within tau (relative) of an E2M1 rounding midpoint.
    """
    xf = as_f32(x)
    R, C = xf.shape
    gs = np.asarray(gs, dtype=F32)
    if gs.ndim == 0:
        gs = np.full((R,), gs, dtype=F32)
    gs = gs.reshape(R, 1)
    blocks = xf.reshape(R, C // BLOCK, BLOCK).astype(np.float64)
    amax_b = np.max(np.abs(blocks), axis=-1)
    a_s = amax_b * gs
    t = np.minimum(a_s / 6.0, 448.0)
    mids = _e4m3_midpoints()
    j = np.clip(np.searchsorted(mids, t), 1, len(mids) - 1)
    dmid = np.minimum(np.abs(t - mids[j - 1]), np.abs(t - mids[j]))
    block = (np.abs(a_s - float(UNDERFLOW)) <= tau * float(UNDERFLOW)) | (dmid <= tau * t)
    codes, sf = quantize_blocks(xf, gs.reshape(R))
    sd = e4m3_decode(sf).astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(sf > 0, gs / np.where(sf > 0, sd, 1.0), 0.0)
    v = np.abs(blocks) * r[..., None]
    dm = np.min(np.abs(v[..., None] - _E2M1_MIDPOINTS), axis=-1)
    vmid = _E2M1_MIDPOINTS[np.argmin(np.abs(v[..., None] - _E2M1_MIDPOINTS), axis=-1)]
    elem = (dm <= tau * vmid) | block[..., None]
    return elem.reshape(R, C), block
