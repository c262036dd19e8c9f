"""Pins of the MX re-encoding oracle (oracle/mx.py) to facts outside it: the
E8M0 and E2M1 definitions, hand-worked examples (tests/golden), the MX
conversion's defining properties checked by brute force over the E2M1 grid,
a lossless special case, the block pairing, and a triple-loop GEMM."""

import os

import numpy as np
import pytest

from oracle import mx as X
from oracle import quantize as Q
from oracle.formats import e2m1_decode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mx_worked_examples.txt")
GRID = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])


def _examples():
    ex, cur = [], None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, val = line.split(":", 1)
        if key == "example":
            cur = {"name": val.strip()}
            ex.append(cur)
        else:
            cur[key] = np.array([int(t, 16) for t in val.split()], dtype=np.uint8)
    return ex


def test_e8m0_anchors():
    assert X.e8m0_decode(127) == 1.0
    assert X.e8m0_decode(130) == 8.0
    assert X.e8m0_decode(0) == 2.0 ** -127
    assert X.e8m0_decode(254) == 2.0 ** 127
    assert np.isnan(X.e8m0_decode(255))


@pytest.mark.parametrize("ex", _examples(), ids=lambda e: e["name"])
def test_hand_worked_examples(ex):
    q, sc = X.nvfp4_to_mx(ex["nv_q"][None], ex["nv_sf"][None])
    assert q[0].tolist() == ex["mx_q"].tolist()
    assert sc[0].tolist() == ex["mx_sc"].tolist()


def _random_nvfp4(rows, cols, seed, spread=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    if spread:   # blocks of very different magnitudes
        x *= np.exp2(rng.integers(-12, 6, size=(rows, cols // 16, 1))).repeat(16, 2).reshape(rows, cols)
    x[0, :16] = 0.0                                   # a zero 16-block
    q, sf, gs = Q.quantize_nvfp4(x)
    return q, sf


def test_shared_scale_puts_amax_in_4_to_8():
    """X = 2^(floor(log2 amax) - 2) <=> 4 <= amax / X < 8 (E2M1 emax 2)."""
    q, sf = _random_nvfp4(64, 512, 1)
    u = Q.block_values(q, sf).reshape(64, 16, 32)
    amax = np.abs(u).max(-1)
    _, sc = X.nvfp4_to_mx(q, sf)
    Xs = X.e8m0_decode(sc)
    nz = amax > 0
    r = amax[nz] / Xs[nz]
    assert np.all((r >= 4) & (r < 8))
    assert np.all(sc[~nz] == 0)


def test_elements_are_nearest_grid_points_ties_even_saturating():
    """Brute force over the E2M1 grid: every element is the nearest multiple
    g * X (g in the grid, same sign) of its NVFP4 value, ties to the even
    code; values beyond 6X become 6X."""
    q, sf = _random_nvfp4(32, 256, 2)
    u = Q.block_values(q, sf)
    sign = Q.unpack_codes(q) >> 3
    qm, sc = X.nvfp4_to_mx(q, sf)
    codes = Q.unpack_codes(qm)
    Xs = np.repeat(X.e8m0_decode(sc), 32, axis=1)
    dec = e2m1_decode(codes) * Xs
    for r in range(u.shape[0]):
        for c in range(u.shape[1]):
            x, s = abs(u[r, c]), Xs[r, c]
            if np.all(u[r, (c // 32) * 32:(c // 32 + 1) * 32] == 0):
                assert codes[r, c] == 0
                continue
            assert (codes[r, c] >> 3) == sign[r, c]
            if x / s > 6:
                assert abs(dec[r, c]) == 6 * s
                continue
            d = np.abs(GRID * s - x)
            best = np.flatnonzero(d == d.min())
            want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
            assert (codes[r, c] & 7) == want, (r, c, x, s)


def test_lossless_when_nvfp4_scales_are_one_power_of_two():
    """Both 16-blocks with the same power-of-two E4M3 scale and a code 6 in
    the pair: X equals that scale and every value survives exactly."""
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 16, size=(8, 64)).astype(np.uint8)
    codes[:, 0] = 7
    codes[:, 32] = 15
    sf = np.full((8, 4), 0x40, np.uint8)              # E4M3 2.0
    sf[:, 2:] = 0x28                                  # E4M3 0.25
    q = Q.pack_codes(codes)
    qm, sc = X.nvfp4_to_mx(q, sf)
    assert np.all(X.mx_block_values(qm, sc) == Q.block_values(q, sf))
    assert np.all(sc[:, 0] == 128) and np.all(sc[:, 1] == 125)


def test_pairs_adjacent_nvfp4_blocks():
    """MX block j is NVFP4 blocks 2j and 2j+1: a value only in block 1 sets
    MX scale 0 and leaves MX block 1 (NVFP4 blocks 2, 3) zero."""
    codes = np.zeros((1, 64), np.uint8)
    codes[0, 20] = 7                                   # NVFP4 block 1
    sf = np.array([[0x00, 0x38, 0x00, 0x00]], np.uint8)
    qm, sc = X.nvfp4_to_mx(Q.pack_codes(codes), sf)
    assert sc.tolist() == [[0x7F, 0x00]]
    out = Q.unpack_codes(qm)[0]
    assert out[20] == 7 and out.sum() == 7


def test_mx_matmul_matches_triple_loop():
    rng = np.random.default_rng(4)
    a_codes = rng.integers(0, 16, size=(3, 64)).astype(np.uint8)
    b_codes = rng.integers(0, 16, size=(5, 64)).astype(np.uint8)
    a_sc = rng.integers(120, 135, size=(3, 2)).astype(np.uint8)
    b_sc = rng.integers(120, 135, size=(5, 2)).astype(np.uint8)
    ga, gb = np.float32(3.0), np.float32(0.5)
    got = X.mx_matmul(Q.pack_codes(a_codes), a_sc, ga, Q.pack_codes(b_codes), b_sc, gb)
    for i in range(3):
        for j in range(5):
            s = 0.0
            for k in range(64):
                s += (e2m1_decode(a_codes[i, k]) * 2.0 ** (int(a_sc[i, k // 32]) - 127) *
                      e2m1_decode(b_codes[j, k]) * 2.0 ** (int(b_sc[j, k // 32]) - 127))
            assert got[i, j] == pytest.approx(s / 1.5, rel=1e-12)


def test_mx_forward_is_close_to_but_not_the_exact_path():
    """Composition check of the MX forward on the tiny workload: its output
    lies within the error a 32-element power-of-two re-encoding of x, W1, h
    and W2 can add (cosine 0.952 against the exact NVFP4 forward at this
    seed; the band is 0.9-0.99999), and differs from it (a path that skipped
    a re-encoding, or read E8M0 bytes as E4M3, lands far outside this band or
    on the exact result)."""
    from nvfp4_block_scaled_04_amd import inputs as I
    from oracle import moe as O
    from oracle.formats import bf16_bits_to_f32
    w = I.WORKLOADS["tiny"]
    x = I.bf16_to_bits(I.make_x(w))
    ids, tw = I.make_routing(w)
    pairs = [I.make_expert_weights(w, e) for e in range(w.E)]
    w1 = np.stack([I.bf16_to_bits(p[0]) for p in pairs])
    w2 = np.stack([I.bf16_to_bits(p[1]) for p in pairs])
    wts = O.prepare_weights(w1, w2)
    ref = O.moe_forward(x, ids, tw, wts, np.float32(w.gs_h), w.E)
    got = X.moe_forward_mx(x, ids, tw, X.prepare_weights_mx(wts), np.float32(w.gs_h), w.E)
    a = bf16_bits_to_f32(ref["out"]).astype(np.float64).ravel()
    b = bf16_bits_to_f32(got["out"]).astype(np.float64).ravel()
    cos = a @ b / np.linalg.norm(a) / np.linalg.norm(b)
    assert 0.9 < cos < 0.99999, cos
