"""Pins of the oracle's GEMM, SwiGLU, combine and whole forward."""

import math

import numpy as np
import pytest

from oracle import moe as O
from oracle import quantize as Q
from oracle import formats as F
from oracle import layout as L
from oracle import route as R


def _bf16(x):
    return F.round_to_bf16(np.asarray(x, dtype=np.float64))


def _randn(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def test_gemm_matches_triple_loop():
    a = _bf16(_randn((5, 32), 1))
    b = _bf16(_randn((3, 32), 2, 0.02))
    aq, asf, ga = Q.quantize_nvfp4(a)
    bq, bsf, gb = Q.quantize_nvfp4(b)
    got = O.nvfp4_matmul(aq, asf, ga[0], bq, bsf, gb[0])
    ca, cb = Q.unpack_codes(aq), Q.unpack_codes(bq)
    for i in range(5):
        for j in range(3):
            s = 0.0
            for kk in range(32):
                va = F.e2m1_decode(ca[i, kk]) * F.e4m3_decode(asf[i, kk // 16])
                vb = F.e2m1_decode(cb[j, kk]) * F.e4m3_decode(bsf[j, kk // 16])
                s += float(va) * float(vb)
            assert got[i, j] == pytest.approx(s / (float(ga[0]) * float(gb[0])), rel=1e-12)


def test_gemm_one_hot_selects_columns():
    a = _bf16(_randn((4, 64), 3))
    aq, asf, ga = Q.quantize_nvfp4(a)
    # B rows are one-hot with value 6 * 448: quantised exactly (sf 0x7E, code 7)
    b = np.zeros((3, 64))
    for j, c in enumerate((0, 17, 63)):
        b[j, c] = 2688.0
    bq, bsf, gb = Q.quantize_nvfp4(_bf16(b))
    assert gb[0] == 1.0
    got = O.nvfp4_matmul(aq, asf, ga[0], bq, bsf, gb[0])
    deq = Q.dequantize(aq, asf, ga[0])
    for j, c in enumerate((0, 17, 63)):
        np.testing.assert_allclose(got[:, j], deq[:, c] * 2688.0, rtol=1e-14, atol=0)


def test_silu_closed_form():
    assert O.silu(0.0) == 0.0
    assert O.silu(30.0) == pytest.approx(30.0, rel=1e-12)
    assert abs(O.silu(-800.0)) == 0.0
    assert O.silu(1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)


def _tiny_moe(T=6, K=32, I=16, E=3, k=2, seed=0):
    rng = np.random.default_rng(seed)
    x = _bf16(rng.standard_normal((T, K)))
    w1 = _bf16(rng.standard_normal((E, K, 2 * I)) * 0.05)
    w2 = _bf16(rng.standard_normal((E, I, K)) * 0.05)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    return x, w1, w2, ids, w


def test_swiglu_pairs_gate_and_up():
    # zero gate weights -> h == 0 (SiLU on all columns would give silu(up) != 0:
    # README "Key Lessons" 10); zero up weights -> h == 0 as well.
    x, w1, w2, ids, w = _tiny_moe()
    K, I = 32, 16
    for zero in (slice(0, I), slice(I, 2 * I)):
        w1z = w1.copy()
        w1z[:, :, zero] = 0
        wts = O.prepare_weights(w1z, w2)
        res = O.moe_forward(x, ids, w, wts, np.float32(64.0), 3)
        assert np.all(res["h"] == 0)
        assert np.all(F.bf16_bits_to_f32(res["out"]) == 0)


def test_swiglu_value_against_plain_formula():
    x, w1, w2, ids, w = _tiny_moe(seed=1)
    wts = O.prepare_weights(w1, w2)
    res = O.moe_forward(x, ids, w, wts, np.float32(64.0), 3)
    aq, asf, ga = Q.quantize_nvfp4(x)
    xd = Q.dequantize(aq, asf, ga[0])
    off, perm = res["offsets"], res["perm"]
    for e in range(3):
        # dequantised logical weight: de-interleave the K-major operand
        wd = Q.dequantize(wts["w1_q"][e], wts["w1_sf"][e], wts["gs_w1"][e])   # (2I, K)
        gate_w, up_w = L.deinterleave_cols(wd.T)                               # (K, I) each
        for d in range(off[e], off[e + 1]):
            t = perm[d] // 2
            g = xd[t] @ gate_w
            u = xd[t] @ up_w
            ref = (g / (1 + np.exp(-g))) * u
            np.testing.assert_allclose(res["h"][d], ref.astype(np.float32), rtol=1e-6, atol=1e-30)


def test_combine_k1_unit_weight_is_unpermute():
    rng = np.random.default_rng(5)
    T, H = 9, 32
    y = _bf16(rng.standard_normal((T, H)))
    ids = rng.integers(0, 4, (T, 1))
    offs, perm, inv, _ = R.route(ids, 4)
    # rows stored in expert order d = inv[t]; out[t] must be y[t] exactly
    yd = np.empty_like(y)
    yd[inv] = y
    out = O.combine(yd, inv, np.ones((T, 1), np.float32), T)
    assert np.array_equal(out, y)


def test_combine_identical_rows_convex_weights():
    T, k, H = 4, 3, 16
    row = _bf16(np.linspace(-2, 2, H))
    y = np.tile(row, (T * k, 1))
    w = np.array([[0.5, 0.25, 0.25]] * T, dtype=np.float32)
    inv = np.random.default_rng(0).permutation(T * k).astype(np.int32)
    out = O.combine(y, inv, w, T * k)
    assert np.array_equal(out, np.tile(row, (T, 1)))


def test_combine_skips_invalid_rows():
    y = _bf16(np.ones((4, 16)))
    inv = np.array([0, 3, 1, 2], dtype=np.int32)       # row 3 is past n_valid
    out = O.combine(y, inv, np.ones((2, 2), np.float32), 3)
    assert F.bf16_bits_to_f32(out)[0, 0] == 1.0 and F.bf16_bits_to_f32(out)[1, 0] == 2.0


def test_single_expert_equals_dense_linear():
    x, w1, w2, ids, w = _tiny_moe(T=5, E=1, k=1, seed=2)
    wts = O.prepare_weights(w1, w2)
    res = O.moe_forward(x, ids, w, wts, np.float32(64.0), 1)
    aq, asf, ga = Q.quantize_nvfp4(x)
    acc = O.nvfp4_matmul(aq, asf, ga[0], wts["w1_q"][0], wts["w1_sf"][0], wts["gs_w1"][0])
    gate, up = L.deinterleave_cols(acc)
    h = (O.silu(gate) * up).astype(np.float32)
    assert np.array_equal(res["h"], h)


def test_empty_expert_produces_no_rows():
    x, w1, w2, ids, w = _tiny_moe(T=4, E=3, k=1, seed=3)
    ids[:] = 0
    wts = O.prepare_weights(w1, w2)
    res = O.moe_forward(x, ids, w, wts, np.float32(64.0), 3)
    assert res["offsets"].tolist() == [0, 4, 4, 4]


def _cos(a, b):
    a, b = a.ravel().astype(np.float64), b.ravel().astype(np.float64)
    return float(a @ b / np.linalg.norm(a) / np.linalg.norm(b))


def test_nvfp4_forward_close_to_bf16_math():
    # Sanity (not parity): the NVFP4 path tracks unquantised math about as
    # closely as the README's layer test (cosine 0.988 vs BF16).
    rng = np.random.default_rng(11)
    T, K, I, E, k = 64, 256, 128, 4, 2
    x = _bf16(rng.standard_normal((T, K)))
    w1 = _bf16(rng.standard_normal((E, K, 2 * I)) * 0.02)
    w2 = _bf16(rng.standard_normal((E, I, K)) * 0.02)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.dirichlet(np.ones(k), T).astype(np.float32)
    wts = O.prepare_weights(w1, w2)
    res = O.moe_forward(x, ids, w, wts, np.float32(2048.0), E)
    xf = F.bf16_bits_to_f32(x).astype(np.float64)
    ref = np.zeros((T, K))
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            gu = xf[t] @ F.bf16_bits_to_f32(w1[e]).astype(np.float64)
            h = O.silu(gu[:I]) * gu[I:]
            ref[t] += w[t, j] * (h @ F.bf16_bits_to_f32(w2[e]).astype(np.float64))
    got = F.bf16_bits_to_f32(res["out"]).astype(np.float64)
    c = _cos(got, ref)
    assert 0.97 < c < 0.9999
    # the global scales are divided out: magnitudes agree too
    assert 0.95 < np.linalg.norm(got) / np.linalg.norm(ref) < 1.05


def _shared_case(seed=5, T=24, H=128, I=128, E=4, k=2):
    rng = np.random.default_rng(seed)
    bits = lambda a: (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    x = bits(rng.standard_normal((T, H)))
    w1 = bits(rng.standard_normal((E + 1, H, 2 * I)) * 0.05)
    w2 = bits(rng.standard_normal((E + 1, I, H)) * 0.05)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    tw = rng.random((T, k)).astype(np.float32)
    return x, w1, w2, ids, tw


def test_shared_expert_with_zero_weights_is_the_routed_forward():
    x, w1, w2, ids, tw = _shared_case()
    w1[-1] = 0
    w2[-1] = 0
    wts = O.prepare_weights(w1, w2)
    a = O.moe_forward_shared(x, ids, tw, wts, np.float32(64.0), 4)["out"]
    b = O.moe_forward(x, ids, tw, wts, np.float32(64.0), 4)["out"]
    assert np.array_equal(a, b)


def test_shared_expert_alone_is_the_dense_mlp():
    """Routing weights 0: out is the shared expert's own BF16 output,
    composed here from the quantiser and the GEMMs on all tokens."""
    x, w1, w2, ids, tw = _shared_case(6)
    wts = O.prepare_weights(w1, w2)
    got = O.moe_forward_shared(x, ids, np.zeros_like(tw), wts, np.float32(64.0), 4)["out"]
    aq, asf, ga = Q.quantize_nvfp4(x)
    h = O.l1_swiglu(aq, asf, ga[0], wts["w1_q"][4], wts["w1_sf"][4], wts["gs_w1"][4])
    c, s = Q.quantize_blocks(h, np.float32(64.0))
    y = O.l2(Q.pack_codes(c), s, np.float32(64.0), wts["w2_q"][4], wts["w2_sf"][4], wts["gs_w2"][4])
    assert np.array_equal(got, y)


def test_shared_expert_equals_one_more_routed_slot():
    """The shared expert is an expert every token visits with weight 1, added
    after the routed slots: routing each token to it as slot k gives the same
    output bit for bit."""
    x, w1, w2, ids, tw = _shared_case(7)
    wts = O.prepare_weights(w1, w2)
    got = O.moe_forward_shared(x, ids, tw, wts, np.float32(64.0), 4)["out"]
    T, k = ids.shape
    ids2 = np.concatenate([ids, np.full((T, 1), 4, np.int32)], axis=1)
    tw2 = np.concatenate([tw, np.ones((T, 1), np.float32)], axis=1)
    ref = O.moe_forward(x, ids2, tw2, wts, np.float32(64.0), 5)["out"]
    assert np.array_equal(got, ref)
