"""Pins of the oracle quantiser against the pages' rules, hand-worked examples,
exact-rational brute force and invariants that hold for any correct NVFP4
quantiser."""

import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import quantize as Q
from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quant_worked_examples.txt")


def _load_examples():
    ex, cur = [], None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, _, val = line.partition(":")
        val = val.strip()
        if key == "example":
            cur = {"name": val}
            ex.append(cur)
        elif key == "x":
            cur["x"] = np.array([float(v) for v in val.split()], dtype=np.float32)
        elif key == "gs":
            cur["gs"] = None if val == "auto" else np.float32(float(val))
        else:
            cur[key] = np.array([int(v, 16) for v in val.split()], dtype=np.uint8)
    return ex


def _bf16_bits(x32):
    b = x32.astype(np.float32).view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "fixture values must be bf16-exact"
    return (b >> 16).astype(np.uint16)


@pytest.mark.parametrize("ex", _load_examples(), ids=lambda e: e["name"])
def test_worked_examples(ex):
    x = _bf16_bits(ex["x"]).reshape(1, -1)
    gs_in = None if ex["gs"] is None else np.array([ex["gs"]], dtype=np.float32)
    q, sf, gs = Q.quantize_nvfp4(x, gs_in=gs_in)
    assert sf.ravel().tolist() == ex["sf"].tolist()
    assert q.ravel().tolist() == ex["q"].tolist()


def _randn_bf16(shape, seed, std=1.0):
    x = (np.random.default_rng(seed).standard_normal(shape) * std).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)   # truncation: any bf16 is fine


def test_global_scale_definition():
    x = _randn_bf16((8, 64), 1)
    xf = F.bf16_bits_to_f32(x)
    amax = np.float32(np.abs(xf).max())
    assert Q.global_scale(x) == np.float32(np.float32(2688.0) / amax)
    assert Q.global_scale(np.zeros((2, 16), np.uint16)) == 1.0


def test_zero_block_gets_exact_zero_scale():
    # README "Correctness Bugs Fixed", bug 3
    x = _randn_bf16((4, 64), 2)
    x[1, 16:32] = 0
    x[2, 0:16] = 0x8000                      # -0.0 is a zero block too
    q, sf, _ = Q.quantize_nvfp4(x)
    assert sf[1, 1] == 0 and sf[2, 0] == 0
    assert np.all(Q.unpack_codes(q)[1, 16:32] == 0)
    assert np.all(Q.unpack_codes(q)[2, 0:16] == 0)


def test_underflow_block_is_zeroed():
    # README "Correctness Bugs Fixed", bug 4: amax (after the global scale)
    # below 6 * 2**-9 -> the block is zeroed, scale byte 0
    x = _randn_bf16((2, 64), 3).view(np.uint16)
    xf = F.bf16_bits_to_f32(x).copy()
    xf[0, 32:48] *= np.float32(1e-7)
    xb = (xf.view(np.uint32) >> 16).astype(np.uint16)
    q, sf, gs = Q.quantize_nvfp4(xb)
    blk = F.bf16_bits_to_f32(xb)[0, 32:48]
    assert np.float32(np.abs(blk).max() * gs[0]) < np.float32(6 * 2 ** -9)
    assert sf[0, 2] == 0 and np.all(Q.unpack_codes(q)[0, 32:48] == 0)
    # every other block keeps a nonzero scale
    assert np.count_nonzero(sf) == sf.size - 1


def test_sf_zero_iff_codes_zero_iff_zeroed():
    x = _randn_bf16((64, 256), 4)
    xf = F.bf16_bits_to_f32(x).copy()
    rng = np.random.default_rng(4)
    for r, b in rng.integers(0, [64, 16], size=(40, 2)):
        xf[r, 16 * b:16 * b + 16] *= np.float32(10.0 ** -rng.integers(1, 9))
    xb = (xf.view(np.uint32) >> 16).astype(np.uint16)
    q, sf, gs = Q.quantize_nvfp4(xb)
    codes = Q.unpack_codes(q).reshape(64, 16, 16)
    mag = codes & 7
    assert np.array_equal(sf == 0, np.all(mag == 0, axis=-1) & np.all(codes == 0, axis=-1))
    # nonzero scale => the block's largest magnitude code is at least 4 (value 2)
    assert np.all(mag.max(-1)[sf != 0] >= 4)
    # normal scales => largest code is 6 (magnitude code 7)
    normal = sf >= 0x08
    assert np.all(mag.max(-1)[normal] == 7)


def test_max_block_gets_max_scale():
    x = _randn_bf16((16, 128), 5)
    q, sf, gs = Q.quantize_nvfp4(x)
    xf = F.bf16_bits_to_f32(x)
    r, c = np.unravel_index(np.argmax(np.abs(xf)), xf.shape)
    assert sf[r, c // 16] == 0x7E
    assert Q.unpack_codes(q)[r, c] & 7 == 7


def test_power_of_two_scale_invariance():
    # scaling x by 2^j scales gs by 2^-j exactly and leaves every byte alone
    x = _randn_bf16((32, 128), 6)
    q0, s0, g0 = Q.quantize_nvfp4(x)
    xf = F.bf16_bits_to_f32(x)
    for j in (-3, 5):
        xs = (xf * np.float32(2.0 ** j)).view(np.uint32) >> 16
        q1, s1, g1 = Q.quantize_nvfp4(xs.astype(np.uint16))
        assert np.array_equal(q0, q1) and np.array_equal(s0, s1)
        assert g1[0] == g0[0] * np.float32(2.0 ** -j)


def test_sign_symmetry():
    x = _randn_bf16((16, 64), 7)
    q0, s0, _ = Q.quantize_nvfp4(x)
    q1, s1, _ = Q.quantize_nvfp4(x ^ np.uint16(0x8000))
    c0, c1 = Q.unpack_codes(q0), Q.unpack_codes(q1)
    assert np.array_equal(s0, s1)
    nz = s0.repeat(16, axis=1) != 0
    assert np.array_equal(c0[nz] ^ 8, c1[nz])


def test_packing_low_nibble_first():
    codes = np.array([[1, 2, 3, 4, 15, 0, 0, 9]], dtype=np.uint8)
    assert Q.pack_codes(codes).tolist() == [[0x21, 0x43, 0x0F, 0x90]]
    assert np.array_equal(Q.unpack_codes(Q.pack_codes(codes)), codes)


def _exact_block(x_vals, gs):
    """Exact-rational quantisation of one block (no fp32 rounding anywhere);
    returns (sf byte, codes, distances of x*gs/sd to the nearest E2M1 midpoint)."""
    e4 = [Fraction(float(v)) for v in F.e4m3_decode(np.arange(0x7F))]
    e2 = [Fraction(v) for v in (0, .5, 1, 1.5, 2, 3, 4, 6)]
    fx = [Fraction(float(v)) for v in x_vals]
    gsf = Fraction(float(gs))
    amax = max(abs(v) for v in fx)
    a_s = amax * gsf
    if amax == 0 or a_s < Fraction(6, 512):
        return 0, [0] * 16, None
    t = min(a_s / 6, Fraction(448))

    def nearest(tab, v):
        best = None
        for i, c in enumerate(tab):
            d = abs(c - v)
            if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
                best = (d, i)
        return best[1]

    sf = nearest(e4, t)
    sd = e4[sf]
    codes, margin = [], []
    mids = [(e2[i] + e2[i + 1]) / 2 for i in range(7)]
    for v in fx:
        u = min(abs(v) * gsf / sd, Fraction(6))
        c = nearest(e2, u)
        codes.append(c | (8 if v < 0 else 0))
        margin.append(min(abs(u - m) / m for m in mids))
    return sf, codes, margin


def test_fp32_sequence_matches_exact_rational_away_from_ties():
    rng = np.random.default_rng(8)
    x = _randn_bf16((6, 64), 8)
    xf = F.bf16_bits_to_f32(x)
    q, sf, gs = Q.quantize_nvfp4(x)
    codes = Q.unpack_codes(q)
    checked = 0
    for r in range(6):
        for b in range(4):
            blk = xf[r, 16 * b:16 * b + 16]
            esf, ecodes, margin = _exact_block(blk, gs[0])
            assert esf == sf[r, b]
            for i in range(16):
                if margin is not None and margin[i] < 2.0 ** -20:
                    continue          # fp32 rounding of r may move an exact tie
                assert ecodes[i] == codes[r, 16 * b + i]
                checked += 1
    assert checked > 350


def test_dequant_requant_byte_identical():
    # README "Correctness Bugs Fixed", bug 2: requantising the dequantised
    # values gives back every byte.  Weight-like data; requantise from the BF16 rounding of
    # the dequantised values with a freshly computed global scale.
    x = _randn_bf16((2 * 128, 512), 9, std=0.02)
    q, sf, gs = Q.quantize_nvfp4(x, groups=2)
    xd = Q.dequantize(q, sf, np.repeat(gs, 128))
    xb = F.round_to_bf16(xd)
    q2, sf2, gs2 = Q.quantize_nvfp4(xb, groups=2)
    assert np.array_equal(q, q2) and np.array_equal(sf, sf2)
    # and from float32 dequantised values, with the same global scale
    q3, sf3, _ = Q.quantize_nvfp4(xd.astype(np.float32), groups=2, gs_in=gs)
    assert np.array_equal(q, q3) and np.array_equal(sf, sf3)


def test_dequant_error_bound():
    # away from saturation every element is within half an E2M1 step of its
    # scaled value: |x - x_hat| <= step/2 * sd / gs with step <= 2
    x = _randn_bf16((32, 256), 10)
    q, sf, gs = Q.quantize_nvfp4(x)
    xf = F.bf16_bits_to_f32(x).astype(np.float64)
    xd = Q.dequantize(q, sf, gs[0])
    sd = F.e4m3_decode(sf).repeat(16, axis=1)
    assert np.all(np.abs(xf - xd) <= 1.0 * sd / gs[0] * (1 + 1e-6))


def test_groups_have_independent_scales():
    x = _randn_bf16((3 * 16, 64), 11)
    xf = F.bf16_bits_to_f32(x).copy()
    xf[16:32] *= np.float32(8.0)
    xb = (xf.view(np.uint32) >> 16).astype(np.uint16)
    q, sf, gs = Q.quantize_nvfp4(xb, groups=3)
    for g in range(3):
        qg, sfg, gsg = Q.quantize_nvfp4(xb[16 * g:16 * g + 16])
        assert gsg[0] == gs[g]
        assert np.array_equal(qg, q[16 * g:16 * g + 16])


def test_dequant_requant_byte_identical_at_the_underflow_boundary():
    # README "Correctness Bugs Fixed", bugs 2 and 4 together.  Weight-scale
    # blocks (std 0.02, gs ~ 2.7e4) whose raw amax sits 0-7% above 6*2^-9: the
    # E4M3 rounding of their scale can bring the dequantised amax below
    # 6*2^-9, so a rule that tested the raw amax would zero them on the second
    # pass.  With the test after the global scale (a_s ~ 300) nothing
    # underflows and the round trip is exact.
    rng = np.random.default_rng(12)
    x = F.bf16_bits_to_f32(_randn_bf16((256, 512), 12, std=0.02)).copy()
    thr = 6.0 * 2.0 ** -9
    blocks = x.reshape(256, 32, 16)
    picks = rng.choice(256 * 32, size=200, replace=False)
    for p in picks:
        r, b = divmod(int(p), 32)
        blk = blocks[r, b]
        blk *= np.float32(thr * (1.0 + rng.uniform(0.0, 0.07)) / np.abs(blk).max())
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)      # truncate to bf16
    raw = F.bf16_bits_to_f32(xb).reshape(256, 32, 16)
    near = np.abs(raw).max(-1)[np.unravel_index(picks, (256, 32))]
    assert np.all(near >= np.float32(thr) * 0.999) and np.all(near <= thr * 1.07)
    q, sf, gs = Q.quantize_nvfp4(xb)
    assert np.all(sf != 0)                                 # nothing underflows at a_s ~ 300
    xd = Q.dequantize(q, sf, gs[0])
    # some dequantised blocks fall below the raw threshold: those are the
    # blocks a raw-amax rule would zero on requantisation
    assert np.sum(np.abs(xd).reshape(256, 32, 16).max(-1) < thr) > 0
    q2, sf2, _ = Q.quantize_nvfp4(F.round_to_bf16(xd))
    assert np.array_equal(q, q2) and np.array_equal(sf, sf2)
    q3, sf3, _ = Q.quantize_nvfp4(xd.astype(np.float32), gs_in=gs)
    assert np.array_equal(q, q3) and np.array_equal(sf, sf3)


def test_near_ties_marks_exactly_the_values_near_a_boundary():
    # near_ties certifies which requantisation differences the parity tests
    # excuse; every expectation below follows from the block rule at gs = 1.
    tau = 1e-3
    row = np.zeros(64, np.float32)
    # block 0: amax 6 -> t = 1 (an E4M3 value, far from its midpoints
    # 0.96875 and 1.0625), r = 1, so v = |x|
    row[0:8] = [6.0, 2.5, 2.5 * (1 + tau / 4), 2.5 * (1 + 8 * tau), 2.75, 0.1, 1.2501, 0.0]
    elem_expect = [False, True, True, False, False, False, True, False]
    # block 1: amax 6.375 -> t = 1.0625, the midpoint of E4M3 1 and 1.125
    row[16:19] = [6.375, 1.0, 0.3]
    # block 2: amax just above 6*2^-9: the underflow decision is a near tie
    row[32] = np.float32(6.0 * 2.0 ** -9 * (1 + tau / 2))
    # block 3: amax 3 -> t = 0.5 (an E4M3 value), r = 2; 1.0 -> v = 2, far
    row[48:50] = [3.0, 1.0]
    elem, block = Q.near_ties(row.reshape(1, 64), np.float32(1.0), tau)
    assert block.ravel().tolist() == [False, True, True, False]
    assert elem[0, 0:8].tolist() == elem_expect
    assert np.all(elem[0, 16:48])                      # every element of a near-tie block
    assert not elem[0, 48:64].any()
    assert not elem[0, 8:16].any()                     # zeros: 0.25 is far from 0
