"""Pins of the oracle's routing and weight layout.

Routing is checked against the O(n x E) equality mask the README replaced
("Correctness Bugs Fixed", bug 5) and a pure-Python stable scatter; the
interleave against one-hot probes that the granularity-4 bug of README
"Fused SwiGLU — How It Works" ("The //2 Bug") fails.
"""

import numpy as np
import pytest

from oracle import route as R
from oracle import layout as L


def _mask_route(ids, E):
    """The superseded O(n x E) mask, plus a pure-Python stable scatter."""
    flat = ids.reshape(-1)
    mask = flat[:, None] == np.arange(E)[None, :]
    counts = mask.sum(axis=0)
    perm = []
    for e in range(E):
        for f in range(flat.size):
            if flat[f] == e:
                perm.append(f)
    for f in range(flat.size):
        if not (0 <= flat[f] < E):
            perm.append(f)
    return counts, np.array(perm)


@pytest.mark.parametrize("T,k,E,seed", [(1, 1, 1, 0), (7, 2, 4, 1), (33, 8, 16, 2), (50, 3, 64, 3)])
def test_route_matches_mask(T, k, E, seed):
    ids = np.random.default_rng(seed).integers(0, E, size=(T, k))
    offsets, perm, inv_perm, bad = R.route(ids, E)
    counts, perm_ref = _mask_route(ids, E)
    assert bad == 0
    assert np.array_equal(np.diff(offsets), counts)
    assert offsets[0] == 0 and offsets[-1] == T * k
    assert np.array_equal(perm, perm_ref)
    assert np.array_equal(inv_perm[perm], np.arange(T * k))


def test_route_empty_and_single_expert():
    ids = np.full((10, 2), 3)
    offsets, perm, inv_perm, _ = R.route(ids, 5)
    assert offsets.tolist() == [0, 0, 0, 0, 20, 20]
    assert perm.tolist() == list(range(20))


def test_route_invalid_ids_are_counted_and_last():
    ids = np.array([[0, 9], [-1, 1], [1, 0]])
    offsets, perm, inv_perm, bad = R.route(ids, 2)
    counts, perm_ref = _mask_route(ids, 2)
    assert bad == 2 and offsets.tolist() == [0, 2, 4]
    assert np.array_equal(perm, perm_ref)
    assert sorted(perm[4:].tolist()) == [1, 2]


def test_route_zero_tokens():
    offsets, perm, inv_perm, bad = R.route(np.zeros((0, 4), np.int32), 3)
    assert offsets.tolist() == [0, 0, 0, 0] and perm.size == 0


def test_interleave_pattern():
    # README "Fused SwiGLU": eight gate columns, then their eight up columns, ...
    src = L.interleave_src(64)
    half = 32
    assert src[:8].tolist() == list(range(8))
    assert src[8:16].tolist() == list(range(half, half + 8))
    assert src[16:24].tolist() == list(range(8, 16))
    assert src[24:32].tolist() == list(range(half + 8, half + 16))
    assert sorted(src.tolist()) == list(range(64))


def _granularity4(w):
    """The buggy interleave (granularity 4) used as a planted mistake."""
    two_i = w.shape[-1]
    n = np.arange(two_i)
    grp, pos = n // 8, n % 8
    col = grp * 4 + pos % 4
    src = np.where(pos < 4, col, two_i // 2 + col)
    return np.ascontiguousarray(np.swapaxes(w, -1, -2)[..., src, :])


def test_one_hot_gate_up_probe():
    # a one-hot gate column c and up column c must land 8 apart in one
    # 16-wide group: the pairing the fused epilogue relies on
    K, I = 4, 32
    for c in range(I):
        w = np.zeros((1, K, 2 * I))
        w[0, 0, c] = 1.0            # gate c
        w[0, 1, I + c] = 1.0        # up c
        wi = L.interleave_l1(w)[0]
        g_row = np.nonzero(wi[:, 0])[0].tolist()
        u_row = np.nonzero(wi[:, 1])[0].tolist()
        assert g_row == [16 * (c // 8) + c % 8]
        assert u_row == [g_row[0] + 8]
        gate, up = L.deinterleave_cols(wi.T)
        assert gate[0, c] == 1 and up[1, c] == 1
        bad = _granularity4(w)[0]
        if c % 8 >= 4:
            assert np.nonzero(bad[:, 0])[0].tolist() != g_row


def test_deinterleave_inverts_interleave():
    w = np.random.default_rng(0).standard_normal((2, 5, 48))
    wi = L.interleave_l1(w)
    gate, up = L.deinterleave_cols(np.swapaxes(wi, -1, -2))
    assert np.array_equal(np.concatenate([gate, up], axis=-1), w)


def test_k_major():
    w = np.arange(24).reshape(1, 4, 6)
    assert np.array_equal(L.k_major(w)[0], w[0].T)


def _brute_topk(row, k):
    """Selection by repeated scan: the largest remaining value, lowest index
    among equals."""
    left = list(range(len(row)))
    out = []
    for _ in range(k):
        best = left[0]
        for e in left[1:]:
            if row[e] > row[best]:
                best = e
        out.append(best)
        left.remove(best)
    return out


@pytest.mark.parametrize("T,E,k,seed", [(5, 4, 2, 0), (7, 64, 8, 1), (3, 384, 6, 2), (4, 9, 9, 3)])
def test_router_topk_matches_brute_force(T, E, k, seed):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[0, : E // 2] = lg[0, 0]                       # a run of equal logits
    ids, w = R.router_topk(lg, k)
    for t in range(T):
        assert ids[t].tolist() == _brute_topk(lg[t].tolist(), k)
        sel = lg[t, ids[t]].astype(np.float64)
        ref = [np.exp(v - sel.max()) for v in sel]
        np.testing.assert_allclose(w[t], np.array(ref) / sum(ref), rtol=1e-15)
    assert np.all(np.diff(w, axis=1) <= 0)            # weights follow the logit order


def test_router_topk_ties_shift_and_k1():
    lg = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]], np.float32)
    ids, w = R.router_topk(lg, 3)
    assert ids.tolist() == [[1, 2, 4]]                # equal logits: lower id first
    np.testing.assert_array_equal(w, np.full((1, 3), 1 / 3))
    ids2, w2 = R.router_topk(lg + np.float32(5.0), 3)   # softmax is shift-invariant
    assert np.array_equal(ids, ids2)
    np.testing.assert_allclose(w, w2, rtol=1e-15)
    ids1, w1 = R.router_topk(lg, 1)
    assert ids1.tolist() == [[1]] and w1[0, 0] == 1.0
