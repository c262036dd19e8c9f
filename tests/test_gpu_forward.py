"""GPU parity of the whole expert forward (moe_expert_forward) against the
oracle: full comparison on small workloads, sampled tokens at full size."""

import concurrent.futures as cf
import multiprocessing as mp

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_04_amd as nv
from nvfp4_block_scaled_04_amd import inputs as I
from oracle import moe as O
from oracle import quantize as Q
from oracle import route as R
from parity import host, bf16_values, assert_close, assert_requant_matches, TAU
import oracle_pool

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _gpu_weights(w, chunk=16):
    w1s, w2s = [], []
    for e0 in range(0, w.E, chunk):
        es = range(e0, min(w.E, e0 + chunk))
        pairs = [I.make_expert_weights(w, e, DEV) for e in es]
        w1s.append(torch.stack([p[0] for p in pairs]))
        w2s.append(torch.stack([p[1] for p in pairs]))
    return nv.prepare_expert_weights(w1s, w2s, DEV)


def _run(w, ew, ids=None):
    """GPU forward with every tap."""
    x = I.make_x(w, DEV)
    if ids is None:
        ids, tw = I.make_routing(w)
    else:
        tw = np.random.default_rng(0).random(ids.shape).astype(np.float32)
    T, k, H, Iw, E = w.T, w.k, w.H, w.I, w.E
    M = T * k
    z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=DEV)
    taps = dict(a_q=z((T, H // 2), torch.uint8), a_sf=z((T, H // 16), torch.uint8),
                gs_a=z((1,), torch.float32), expert_offsets=z((E + 1,), torch.int32),
                perm=z((M,), torch.int32), inv_perm=z((M,), torch.int32),
                invalid_count=z((1,), torch.int32), h_f32=z((M, Iw), torch.float32),
                h_q=z((M, Iw // 2), torch.uint8), h_sf=z((M, Iw // 16), torch.uint8),
                y_bf16=z((M, H), torch.bfloat16))
    gs_h = torch.tensor([w.gs_h], dtype=torch.float32, device=DEV)
    print(f"[case] forward {w.name} T={T} H={H} I={Iw} E={E} k={k}", flush=True)
    out = nv.moe_expert_forward(x, torch.from_numpy(ids).to(DEV), torch.from_numpy(tw).to(DEV),
                                ew, gs_h, taps=taps)
    torch.cuda.synchronize()
    return x, ids, tw, out, {n: host(t) for n, t in taps.items()}


def _check_full(w, ids=None):
    """Whole workload against the whole oracle (small shapes only)."""
    ew = _gpu_weights(w)
    x, ids, tw, out, tp = _run(w, ew, ids)
    w1 = np.stack([host(I.make_expert_weights(w, e, DEV)[0]) for e in range(w.E)])
    w2 = np.stack([host(I.make_expert_weights(w, e, DEV)[1]) for e in range(w.E)])
    wts = O.prepare_weights(w1, w2)
    for n in ("w1_q", "w1_sf", "w2_q", "w2_sf"):
        assert np.array_equal(host(ew.rowmajor[n]), wts[n]), n
    assert np.array_equal(host(ew.gs_w1), wts["gs_w1"]) and np.array_equal(host(ew.gs_w2), wts["gs_w2"])
    ref = O.moe_forward(host(x), ids, tw, wts, np.float32(w.gs_h), w.E)
    # bit-exact steps
    assert np.array_equal(tp["a_q"], ref["a_q"]) and np.array_equal(tp["a_sf"], ref["a_sf"])
    assert tp["gs_a"][0] == ref["gs_a"]
    assert np.array_equal(tp["expert_offsets"], ref["offsets"])
    assert np.array_equal(tp["perm"], ref["perm"]) and np.array_equal(tp["inv_perm"], ref["inv_perm"])
    assert tp["invalid_count"][0] == ref["n_invalid"]
    nv_rows = int(ref["offsets"][-1])
    # fused L1 + SwiGLU + requant
    assert_close(tp["h_f32"][:nv_rows], ref["h"][:nv_rows], f"{w.name} h")
    tie_rows = assert_requant_matches(tp["h_q"][:nv_rows], tp["h_sf"][:nv_rows],
                                      ref["h"][:nv_rows], w.gs_h, f"{w.name} requant")
    clean = ~tie_rows
    assert_close(bf16_values(tp["y_bf16"][:nv_rows])[clean], bf16_values(ref["y"][:nv_rows])[clean],
                 f"{w.name} y")
    tok_clean = np.ones(w.T, bool)
    for d in np.nonzero(tie_rows)[0]:
        tok_clean[ref["perm"][d] // w.k] = False
    assert_close(bf16_values(host(out))[tok_clean], bf16_values(ref["out"])[tok_clean],
                 f"{w.name} out")
    assert tok_clean.mean() > 0.9


def test_forward_tiny_workload():
    _check_full(I.WORKLOADS["tiny"])


@pytest.mark.parametrize("w", [
    I.custom("one_token", T=1, H=128, I=128, E=1, k=1, seed=1),
    I.custom("ragged", T=77, H=384, I=256, E=6, k=3, seed=2),
    I.custom("skewed_small", T=200, H=256, I=128, E=16, k=4, routing="zipf", special="blocks", seed=3),
    I.custom("many_experts", T=50, H=128, I=128, E=64, k=8, seed=4),
], ids=lambda w: w.name)
def test_forward_small_edge_workloads(w):
    _check_full(w)


def test_forward_invalid_expert_ids_are_skipped_and_counted():
    w = I.custom("invalid", T=40, H=128, I=128, E=4, k=2, seed=5)
    ids, _ = I.make_routing(w)
    ids = ids.copy()
    ids[3, 1] = 9
    ids[17, 0] = -1
    _check_full(w, ids)


def test_forward_zero_tokens():
    w = I.custom("empty", T=0, H=128, I=128, E=4, k=2, seed=6)
    ew = _gpu_weights(w)
    x = torch.zeros((0, 128), dtype=torch.bfloat16, device=DEV)
    out = nv.moe_expert_forward(x, torch.zeros((0, 2), dtype=torch.int32, device=DEV),
                                torch.zeros((0, 2), dtype=torch.float32, device=DEV), ew,
                                torch.tensor([64.0], device=DEV))
    torch.cuda.synchronize()
    assert out.shape == (0, 128)


# ----------------------------------------------------------- full-size, sampled

_BIG = {}


def _big_weights(w):
    """Full-size weights, built once per weight set (decode/prefill/skewed
    share one)."""
    key = (w.weight_seed, w.E, w.H, w.I)
    if key not in _BIG:
        _BIG.clear()                     # one full-size weight set resident at a time
        torch.cuda.empty_cache()
        _BIG[key] = _gpu_weights(w)
    return _BIG[key]


def _sample_tokens(name, ids):
    T = ids.shape[0]
    if name == "skewed":
        top = np.bincount(ids.ravel(), minlength=256).argmax()
        return [int(np.nonzero((ids == top).any(axis=1))[0][0])]
    return [0, T - 1] if name == "decode" else [T // 3]


@pytest.mark.parametrize("name", ["decode", "prefill", "skewed", "moe384"])
def test_forward_full_size_sampled_tokens(name):
    w = I.WORKLOADS[name]
    ew = _big_weights(w)
    x, ids, tw, out, tp = _run(w, ew)
    # routing is cheap to check in full
    roff, rperm, rinv, _ = R.route(ids, w.E)
    assert np.array_equal(tp["expert_offsets"], roff)
    assert np.array_equal(tp["perm"], rperm) and np.array_equal(tp["inv_perm"], rinv)
    xb = host(x)
    gs_a = Q.global_scale(xb)
    assert tp["gs_a"][0] == gs_a
    toks = _sample_tokens(name, ids)
    jobs = []
    for t in toks:
        aq, asf = Q.quantize_blocks(xb[t:t + 1], gs_a)
        aq = Q.pack_codes(aq)
        assert np.array_equal(tp["a_q"][t], aq[0]) and np.array_equal(tp["a_sf"][t], asf[0])
        for j in range(w.k):
            jobs.append((t, j, int(ids[t, j]), aq, asf))
    experts = sorted({e for _, _, e, _, _ in jobs})
    bf = {e: tuple(host(a) for a in I.make_expert_weights(w, e, DEV)) for e in experts}
    print(f"[case] {name}: oracle for tokens {toks} over {len(experts)} experts", flush=True)
    ctx = mp.get_context("spawn")
    with cf.ProcessPoolExecutor(max_workers=min(8, len(jobs)), mp_context=ctx) as ex:
        futs = [ex.submit(oracle_pool.expert_rows, bf[e][0], bf[e][1], aq, asf, gs_a,
                          np.float32(w.gs_h)) for (_, _, e, aq, asf) in jobs]
        res = [f.result() for f in futs]
    for (t, j, e, _, _), r in zip(jobs, res):
        for n in ("w1_q", "w1_sf", "w2_q", "w2_sf"):
            assert np.array_equal(host(ew.rowmajor[n][e]), r[n]), (n, e)
        assert host(ew.gs_w1)[e] == r["gs_w1"] and host(ew.gs_w2)[e] == r["gs_w2"]
    for t in toks:
        rows = [(j, r) for (tt, j, _, _, _), r in zip(jobs, res) if tt == t]
        acc = np.zeros(w.H)
        tie = False
        for j, r in rows:
            d = int(rinv[t * w.k + j])
            assert_close(tp["h_f32"][d:d + 1], r["h"], f"{name} t={t} j={j} h")
            tie |= bool(assert_requant_matches(tp["h_q"][d:d + 1], tp["h_sf"][d:d + 1], r["h"],
                                               w.gs_h, f"{name} t={t} j={j} requant").any())
            if not tie:
                assert_close(bf16_values(tp["y_bf16"][d:d + 1]), bf16_values(r["y"]),
                             f"{name} t={t} j={j} y")
            acc += np.float64(tw[t, j]) * bf16_values(r["y"][0])
        ref_out = bf16_values(O.round_to_bf16(acc))
        if not tie:
            assert_close(bf16_values(host(out)[t]), ref_out, f"{name} t={t} out")


# ----------------------------------------------------------- shared expert

@pytest.mark.parametrize("name,invalid", [("tiny", False), ("tiny", True)])
def test_forward_with_shared_expert(name, invalid):
    """Every token also through a shared expert (index E of E + 1 experts),
    added in the combine; against the oracle's own formulation (routed sum
    plus the shared MLP per token)."""
    w = I.WORKLOADS[name]
    pairs = [I.make_expert_weights(w, e, DEV) for e in range(w.E + 1)]
    w1 = torch.stack([p[0] for p in pairs])
    w2 = torch.stack([p[1] for p in pairs])
    ew = nv.prepare_expert_weights([w1], [w2], DEV)
    x = I.make_x(w, DEV)
    ids, tw = I.make_routing(w)
    if invalid:                       # an id equal to E must not reach the shared expert
        ids = ids.copy()
        ids[3, 0] = w.E
        ids[5, 1] = -2
    T, k, H, Iw = w.T, w.k, w.H, w.I
    M = T * (k + 1)
    z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=DEV)
    taps = dict(expert_offsets=z((w.E + 2,), torch.int32), invalid_count=z((1,), torch.int32),
                h_f32=z((M, Iw), torch.float32), y_bf16=z((M, H), torch.bfloat16))
    print(f"[case] forward + shared expert {name} invalid={invalid}", flush=True)
    out = nv.moe_expert_forward_shared(x, torch.from_numpy(ids).to(DEV), torch.from_numpy(tw).to(DEV),
                                       ew, torch.tensor([w.gs_h], dtype=torch.float32, device=DEV),
                                       taps=taps)
    torch.cuda.synchronize()
    wts = O.prepare_weights(host(w1), host(w2))
    ref = O.moe_forward_shared(host(x), ids, tw, wts, np.float32(w.gs_h), w.E)
    off = host(taps["expert_offsets"])
    assert off[w.E + 1] - off[w.E] == T                      # every token in the shared expert
    assert host(taps["invalid_count"])[0] == (2 if invalid else 0)
    assert np.array_equal(off[:w.E + 1], ref["offsets"][:w.E + 1])
    # shared rows are the last T valid rows, in token order
    hs = host(taps["h_f32"])[off[w.E]:off[w.E + 1]]
    assert_close(hs, ref["h_shared"], "shared h")
    assert_close(bf16_values(host(out)), bf16_values(ref["out"]), "out with shared expert")


@pytest.mark.parametrize("name", ["prefill", "decode", "skewed"])
def test_mx_forward_sampled_token(name):
    """The MX variant at full size: one token's k expert rows and its output
    against the MX oracle (weights re-encoded on both sides and compared
    bit-exactly)."""
    from oracle import mx as X
    w = I.WORKLOADS[name]
    ew_mx = nv.mx_expert_weights(_big_weights(w))
    x = I.make_x(w, DEV)
    ids, tw = I.make_routing(w)
    T, k, H, Iw = w.T, w.k, w.H, w.I
    M = T * k
    z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=DEV)
    taps = dict(a_q=z((T, H // 2), torch.uint8), a_sf=z((T, H // 16), torch.uint8),
                gs_a=z((1,), torch.float32), inv_perm=z((M,), torch.int32),
                h_f32=z((M, Iw), torch.float32), y_bf16=z((M, H), torch.bfloat16))
    print(f"[case] mx forward {name} (sampled token)", flush=True)
    out = nv.moe_expert_forward(x, torch.from_numpy(ids).to(DEV), torch.from_numpy(tw).to(DEV),
                                ew_mx, torch.tensor([w.gs_h], dtype=torch.float32, device=DEV),
                                taps=taps)
    torch.cuda.synchronize()
    tp = {n: host(t) for n, t in taps.items()}
    xb = host(x)
    gs_a = Q.global_scale(xb)
    assert tp["gs_a"][0] == gs_a
    t = _sample_tokens(name, ids)[0] if name == "skewed" else T // 5
    aq, asf = Q.quantize_blocks(xb[t:t + 1], gs_a)
    amq, amsc = X.nvfp4_to_mx(Q.pack_codes(aq), asf)
    assert np.array_equal(tp["a_q"][t], amq[0])
    assert np.array_equal(tp["a_sf"][t], np.repeat(amsc[0], 2))
    experts = [int(e) for e in ids[t]]
    bf = {e: tuple(host(a) for a in I.make_expert_weights(w, e, DEV)) for e in experts}
    ctx = mp.get_context("spawn")
    with cf.ProcessPoolExecutor(max_workers=len(experts), mp_context=ctx) as ex:
        res = list(ex.map(oracle_pool.expert_rows_mx, [bf[e][0] for e in experts],
                          [bf[e][1] for e in experts], [amq] * k, [amsc] * k, [gs_a] * k,
                          [np.float32(w.gs_h)] * k))
    rw = ew_mx.rowmajor
    acc = np.zeros(H)
    tie = False
    for j, (e, r) in enumerate(zip(experts, res)):
        assert np.array_equal(host(rw["w1_q"][e]), r["w1_q"])
        assert np.array_equal(host(rw["w1_sf"][e]), np.repeat(r["w1_sc"], 2, axis=1))
        d = int(tp["inv_perm"][t * k + j])
        assert_close(tp["h_f32"][d:d + 1], r["h"], f"mx t={t} j={j} h")
        # a requant decision within TAU of a rounding boundary may go either
        # way; such rows are reported and kept out of the strict y/out bound
        near = bool(Q.near_ties(r["h"], np.float32(w.gs_h), TAU)[0].any())
        tie |= near
        if not near:
            assert_close(bf16_values(tp["y_bf16"][d:d + 1]), bf16_values(r["y"]), f"mx t={t} j={j} y")
        acc += np.float64(tw[t, j]) * bf16_values(r["y"][0])
    print(f"[case] mx {name} token {t}: near-tie rows present: {tie}", flush=True)
    if not tie:
        assert_close(bf16_values(host(out)[t]), bf16_values(O.round_to_bf16(acc)), f"mx t={t} out")


@pytest.mark.parametrize("name", ["prefill", "skewed"])
def test_shared_forward_sampled_token(name):
    """The shared-expert forward at full size: one token's k routed rows plus
    its shared-expert row, and its output, against the oracle."""
    w = I.WORKLOADS[name]
    print(f"[case] shared forward {name} (sampled token)", flush=True)
    base = _big_weights(w)                                  # routed experts 0..E-1
    sw1, sw2 = I.make_expert_weights(w, w.E, DEV)          # the shared expert
    shared = nv.prepare_expert_weights([sw1[None]], [sw2[None]], DEV)
    cat = lambda a, b: torch.cat([a, b])
    rw, rs = base.rowmajor, shared.rowmajor
    w1 = nv.pack_weights(cat(rw["w1_q"], rs["w1_q"]), cat(rw["w1_sf"], rs["w1_sf"]))
    w2 = nv.pack_weights(cat(rw["w2_q"], rs["w2_q"]), cat(rw["w2_sf"], rs["w2_sf"]))
    both = nv.ExpertWeights(w1, cat(base.gs_w1, shared.gs_w1), w2, cat(base.gs_w2, shared.gs_w2))
    x = I.make_x(w, DEV)
    ids, tw = I.make_routing(w)
    T, k, H, Iw = w.T, w.k, w.H, w.I
    M = T * (k + 1)
    z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=DEV)
    taps = dict(inv_perm=z((M,), torch.int32), h_f32=z((M, Iw), torch.float32),
                y_bf16=z((M, H), torch.bfloat16))
    out = nv.moe_expert_forward_shared(x, torch.from_numpy(ids).to(DEV),
                                       torch.from_numpy(tw).to(DEV), both,
                                       torch.tensor([w.gs_h], dtype=torch.float32, device=DEV),
                                       taps=taps)
    torch.cuda.synchronize()
    tp = {n: host(t) for n, t in taps.items()}
    xb = host(x)
    gs_a = Q.global_scale(xb)
    t = _sample_tokens(name, ids)[0] if name == "skewed" else T // 7
    aq, asf = Q.quantize_blocks(xb[t:t + 1], gs_a)
    aq = Q.pack_codes(aq)
    experts = [int(e) for e in ids[t]] + [w.E]
    bf = {e: tuple(host(a) for a in I.make_expert_weights(w, e, DEV)) for e in experts}
    ctx = mp.get_context("spawn")
    with cf.ProcessPoolExecutor(max_workers=len(experts), mp_context=ctx) as ex:
        res = list(ex.map(oracle_pool.expert_rows, [bf[e][0] for e in experts],
                          [bf[e][1] for e in experts], [aq] * (k + 1), [asf] * (k + 1),
                          [gs_a] * (k + 1), [np.float32(w.gs_h)] * (k + 1)))
    acc = np.zeros(H)
    tie = False
    for j, r in enumerate(res):
        d = int(tp["inv_perm"][t * (k + 1) + j])
        assert_close(tp["h_f32"][d:d + 1], r["h"], f"shared t={t} slot {j} h")
        near = bool(Q.near_ties(r["h"], np.float32(w.gs_h), TAU)[0].any())
        tie |= near
        if not near:
            assert_close(bf16_values(tp["y_bf16"][d:d + 1]), bf16_values(r["y"]), f"shared t={t} y {j}")
        wj = np.float64(tw[t, j]) if j < k else 1.0
        acc += wj * bf16_values(r["y"][0])
    print(f"[case] shared {name} token {t}: near-tie rows present: {tie}", flush=True)
    if not tie:
        assert_close(bf16_values(host(out)[t]), bf16_values(O.round_to_bf16(acc)), f"shared t={t} out")
