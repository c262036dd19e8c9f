"""Helpers for the GPU parity tests: host copies, the floating-point bar and
the requantisation comparison with certified near-ties.

The floating-point bar (cosine >= 0.9999 and max|gpu - oracle| <= 2e-2 * RMS
of the oracle output) applies to results computed from identical quantised
operands.  Integer, byte and index results must be bit-exact.
"""

import numpy as np
import torch

from oracle import quantize as Q
from oracle import formats as F

COS_MIN = 0.9999
MAXABS_RMS = 2e-2
# a GPU requant code may differ from the oracle's only where the oracle's
# scaled value lies within TAU (relative) of a rounding boundary
TAU = 1e-4
MAX_TIE_FRACTION = 1e-3


def host(t):
    """Device tensor -> numpy (bf16 as uint16 bit patterns)."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_values(bits):
    return F.bf16_bits_to_f32(bits).astype(np.float64)


def cosine(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float(a @ b / (na * nb))


# BF16 outputs (y, the combined output, the dense linear): both sides round
# their own sum to BF16, the GPU from fp32 and the oracle from fp64; where the
# two unrounded values straddle a rounding boundary the results differ by one
# BF16 step, which exceeds MAXABS_RMS * RMS for elements above about 5 * RMS.
# Such an element may differ by one step of its value; at most
# MAX_BF16_STEP_FRACTION of the elements may exceed the plain bound.
MAX_BF16_STEP_FRACTION = 1e-3


def bf16_step(v):
    """One BF16 step (unit in the last place) at each |v| (v nonzero)."""
    _, e = np.frexp(np.abs(np.asarray(v, np.float64)))   # |v| = m * 2**e, 0.5 <= m < 1
    return np.ldexp(1.0, e - 8)


def assert_close(gpu, ref, what, log=True, bf16=False):
    """The floating-point parity bar; gpu/ref are float arrays.  bf16=True for
    BF16 outputs compared with the oracle's BF16 rounding (see above)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    d = np.abs(gpu - ref)
    err = float(np.max(d)) if ref.size else 0.0
    cos = cosine(gpu, ref)
    over = d > MAXABS_RMS * rms
    if log or over.any():
        print(f"[parity] {what}: cos={cos:.7f} maxabs/rms={err / rms if rms else 0:.3e} n={ref.size}"
              + (f" ({int(over.sum())} elements one BF16 step apart above the bound)" if over.any() else ""))
    assert cos >= COS_MIN, f"{what}: cosine {cos} < {COS_MIN}"
    if bf16 and over.any():
        assert np.all(d[over] <= bf16_step(ref[over])), \
            f"{what}: max abs err {err} > {MAXABS_RMS} * rms {rms} and beyond one BF16 step"
        assert over.mean() <= MAX_BF16_STEP_FRACTION, f"{what}: {int(over.sum())} elements above the bound"
    else:
        assert err <= MAXABS_RMS * rms, f"{what}: max abs err {err} > {MAXABS_RMS} * rms {rms}"


def assert_requant_matches(gpu_q, gpu_sf, ref_h, gs_h, what, log=True):
    """GPU-requantised h vs the oracle's requantisation of its own h.

    Scale bytes must be equal except in blocks whose scale decision is a
    certified near-tie; codes must be equal except at certified near-tie
    elements, where they must be adjacent on the E2M1 grid with the same sign
    (or both magnitude 0).  Returns the boolean mask of rows that contain a
    certified near-tie (their downstream results may differ by one step)."""
    ref_codes, ref_sf = Q.quantize_blocks(ref_h, np.float32(gs_h))
    elem, block = Q.near_ties(ref_h, np.float32(gs_h), TAU)
    g_codes = Q.unpack_codes(gpu_q)
    R, C = ref_codes.shape
    sf_bad = (gpu_sf != ref_sf) & ~block
    assert not sf_bad.any(), f"{what}: {int(sf_bad.sum())} scale bytes differ outside near-ties"
    same = (g_codes == ref_codes) | (((g_codes & 7) == 0) & ((ref_codes & 7) == 0))
    diff = ~same
    outside = diff & ~elem
    assert not outside.any(), (f"{what}: {int(outside.sum())} codes differ outside certified "
                               f"near-ties (first at {np.argwhere(outside)[:3].tolist()})")
    blk_rep = np.repeat(block, 16, axis=1)
    e_only = diff & ~blk_rep
    adj = (np.abs((g_codes & 7).astype(int) - (ref_codes & 7).astype(int)) <= 1) & \
          (((g_codes ^ ref_codes) & 8) == 0)
    assert np.all(adj[e_only]), f"{what}: a near-tie code moved by more than one grid step"
    frac = diff.sum() / max(1, diff.size)
    if log or diff.any():
        print(f"[parity] {what}: requant codes differ at {int(diff.sum())} certified near-ties "
              f"({frac:.2e}), {int((gpu_sf != ref_sf).sum())} scale bytes")
    assert frac <= MAX_TIE_FRACTION
    return diff.any(axis=1) | (gpu_sf != ref_sf).any(axis=1)


def assert_mx_requant_matches(gpu_q, gpu_sc, ref_h, gs_h, what):
    """GPU-requantised and MX re-encoded h vs the oracle's (NVFP4 requant of
    its own h, then the MX re-encoding).  A 32-element MX block may differ
    only where the NVFP4 requant holds a certified near-tie inside it (one
    flipped code can move the block's E8M0 scale and so every code of the
    block).  gpu_sc holds each E8M0 byte twice (the NVFP4 scale layout).
    Returns the boolean mask of rows whose bytes differ from the oracle's."""
    from oracle import mx as X
    codes, sf = Q.quantize_blocks(ref_h, np.float32(gs_h))
    ref_q, ref_sc = X.nvfp4_to_mx(Q.pack_codes(codes), sf)
    elem, _ = Q.near_ties(ref_h, np.float32(gs_h), TAU)
    R, C = ref_h.shape
    tie32 = elem.reshape(R, C // 32, 32).any(axis=-1)
    dq = (np.asarray(gpu_q) != ref_q).reshape(R, C // 32, 16).any(axis=-1)
    ds = (np.asarray(gpu_sc).reshape(R, C // 32, 2) != ref_sc[..., None]).any(axis=-1)
    diff = dq | ds
    outside = diff & ~tie32
    assert not outside.any(), (f"{what}: {int(outside.sum())} MX blocks differ outside certified "
                               f"near-ties (first at {np.argwhere(outside)[:3].tolist()})")
    if diff.any():
        print(f"[parity] {what}: {int(diff.sum())} MX blocks differ at certified near-ties")
    assert diff.mean() <= MAX_TIE_FRACTION * 32
    return diff.any(axis=1)
