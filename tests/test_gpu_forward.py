"""GPU parity of the whole expert forward (moe_expert_forward) against the
oracle: full comparison on small workloads, sampled tokens at full size."""

import concurrent.futures as cf
import functools
import multiprocessing as mp

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_04_amd as nv
from nvfp4_block_scaled_04_amd import inputs as I
from oracle import moe as O
from oracle import quantize as Q
from oracle import route as R
from parity import host, bf16_values, assert_close, assert_requant_matches, assert_mx_requant_matches
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
                 f"{w.name} y", bf16=True)
    tok_clean = np.ones(w.T, bool)
    for d in np.nonzero(tie_rows)[0]:
        tok_clean[ref["perm"][d] // w.k] = False
    assert_close(bf16_values(host(out))[tok_clean], bf16_values(ref["out"])[tok_clean],
                 f"{w.name} out", bf16=True)
    assert tok_clean.mean() > 0.9


def test_forward_tiny_workload():
    _check_full(I.WORKLOADS["tiny"])


@pytest.mark.parametrize("w", [
    I.custom("one_token", T=1, H=128, I=128, E=1, k=1, seed=1),
    I.custom("ragged", T=77, H=384, I=256, E=6, k=3, seed=2),
    I.custom("skewed_small", T=200, H=256, I=128, E=16, k=4, routing="zipf", special="blocks", seed=3),
    I.custom("many_experts", T=50, H=128, I=128, E=64, k=8, seed=4),
    # more experts than the 32-token tiles take (E > 1024), mostly empty, and
    # two routing chunks in the forward's fused histogram and scan
    I.custom("wide_E", T=64, H=128, I=128, E=1500, k=6, seed=7),
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


# ----------------------------------------------------------- full size

_BIG = {}
POOL = 16                                  # oracle worker processes (a GPU machine's CPU share)
CHUNK_ROWS = 2048                          # rows of one expert per oracle job


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
        return [int(np.nonzero((ids == top).any(axis=1))[0][0]), T // 2]
    return [0, T - 1] if name == "decode" else [T // 3, T - 1]


def _quantize_x(name, xb, chunk=2048):
    """The oracle's quantisation of the whole x (per-call global scale)."""
    gs_a = Q.global_scale(xb)
    T, H = xb.shape
    aq = np.empty((T, H // 2), np.uint8)
    asf = np.empty((T, H // 16), np.uint8)
    for r0 in range(0, T, chunk):
        c, sc = Q.quantize_blocks(xb[r0:r0 + chunk], gs_a)
        aq[r0:r0 + chunk] = Q.pack_codes(c)
        asf[r0:r0 + chunk] = sc
    return aq, asf, gs_a


# experts by row count: m tiles of 1, 2, 3 and 4 32-row blocks, then 2, 3 and
# more 128-row m tiles; plus the smallest and the largest expert
_CATEGORIES = [(1, 32), (33, 64), (65, 96), (97, 128), (129, 256), (257, 384), (385, 1 << 30)]


def _pick_experts(name, offsets):
    counts = np.diff(offsets.astype(np.int64))
    live = np.nonzero(counts)[0]
    if name == "decode":
        return [int(e) for e in live]                    # every routed row
    picks = set()
    for lo, hi in _CATEGORIES:
        sel = live[(counts[live] >= lo) & (counts[live] <= hi)]
        if sel.size:
            picks.add(int(sel[0]))
    picks.add(int(live[np.argmax(counts[live])]))
    picks.add(int(live[np.argmin(counts[live])]))
    return sorted(picks)


def _oracle_rows(w, ew, jobs, worker, check_weights, a_rows):
    """Run the oracle for (expert, rows) jobs in a process pool, a batch of
    experts at a time (their BF16 weights are generated on the device and
    copied to the host per batch), and yield (expert, rows, result).
    check_weights(e, result) compares the expert's prepared weights once."""
    ctx = mp.get_context("spawn")
    by_e = {}
    for e, rows in jobs:
        by_e.setdefault(e, []).append(rows)
    experts = sorted(by_e)
    done = set()
    with cf.ProcessPoolExecutor(max_workers=POOL, mp_context=ctx,
                                initializer=oracle_pool.init_worker) as ex:
        for b0 in range(0, len(experts), 2 * POOL):
            batch = experts[b0:b0 + 2 * POOL]
            futs = []
            for e in batch:
                w1, w2 = (host(t) for t in I.make_expert_weights(w, e, DEV))
                for rows in by_e[e]:
                    aq, asf = a_rows(rows)
                    futs.append((e, rows, ex.submit(worker, w1, w2, aq, asf)))
            for e, rows, f in futs:
                r = f.result()
                if e not in done:
                    check_weights(e, r)
                    done.add(e)
                yield e, rows, r
            print(f"[case] {w.name}: oracle done for {min(b0 + 2 * POOL, len(experts))} of "
                  f"{len(experts)} experts", flush=True)


def _jobs(offsets, experts, extra_rows):
    """All rows of `experts` (cut into chunks) and the rows in extra_rows
    (expert -> row list) of the others."""
    jobs = []
    for e in experts:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        for c0 in range(lo, hi, CHUNK_ROWS):
            jobs.append((e, np.arange(c0, min(hi, c0 + CHUNK_ROWS))))
    for e, rows in extra_rows.items():
        if e not in experts:
            jobs.append((e, np.array(sorted(set(rows)))))
    return jobs


def _token_rows(ids, inv, k, toks):
    extra = {}
    for t in toks:
        for j in range(k):
            extra.setdefault(int(ids[t, j]), []).append(int(inv[t * k + j]))
    return extra


def _check_out(name, w, out_gpu, tw, inv, y_ref, same, toks, slots):
    """out of every token whose `slots` rows were all checked with identical
    quantised h: the oracle's combine of the oracle's y rows."""
    got, ref = [], []
    for t in toks:
        ds = [int(inv[t * slots + j]) for j in range(slots)]
        if not all(d in y_ref and same[d] for d in ds):
            continue
        acc = np.zeros(w.H)
        for j, d in enumerate(ds):
            wj = np.float64(tw[t, j]) if j < tw.shape[1] else 1.0
            acc += wj * bf16_values(y_ref[d])
        got.append(bf16_values(out_gpu[t]))
        ref.append(bf16_values(O.round_to_bf16(acc)))
    assert got, f"{name}: no token had all its rows checked"
    assert_close(np.stack(got), np.stack(ref), f"{name} out ({len(got)} tokens)", bf16=True)
    return len(got)


def _check_rows_nvfp4(name, w, tp, e, rows, r, y_ref, same):
    assert_close(tp["h_f32"][rows], r["h"], f"{name} h e={e}", log=False)
    tie = assert_requant_matches(tp["h_q"][rows], tp["h_sf"][rows], r["h"], w.gs_h,
                                 f"{name} requant e={e}", log=False)
    # identical quantised operands: the GPU's h bytes equal the oracle's
    ok = (tp["h_q"][rows] == r["h_q"]).all(axis=1) & (tp["h_sf"][rows] == r["h_sf"]).all(axis=1)
    assert not (ok & tie).any()
    if ok.any():
        assert_close(bf16_values(tp["y_bf16"][rows][ok]), bf16_values(r["y"][ok]),
                     f"{name} y e={e}", log=False, bf16=True)
    for i, d in enumerate(rows):
        y_ref[int(d)] = r["y"][i]
        same[int(d)] = bool(ok[i])
    return int(ok.sum())


@pytest.mark.timeout(1500)
@pytest.mark.parametrize("name", ["decode", "prefill", "skewed", "moe384"])
def test_forward_full_size(name):
    """A full-size workload: the whole quantised x and the routing bit-exact;
    every row of experts chosen across the row-count categories (every
    expert on the decode batch) through L1 + SwiGLU (f32 h, to the bar), the
    requant (certified near-ties) and L2 (to the bar, wherever the GPU's
    requantised h equals the oracle's byte for byte, i.e. identical operands);
    the output of sampled tokens (all tokens on the decode batch)."""
    w = I.WORKLOADS[name]
    ew = _big_weights(w)
    x, ids, tw, out, tp = _run(w, ew)
    roff, rperm, rinv, _ = R.route(ids, w.E)
    assert np.array_equal(tp["expert_offsets"], roff)
    assert np.array_equal(tp["perm"], rperm) and np.array_equal(tp["inv_perm"], rinv)
    aq, asf, gs_a = _quantize_x(name, host(x))
    assert tp["gs_a"][0] == gs_a
    assert np.array_equal(tp["a_q"], aq) and np.array_equal(tp["a_sf"], asf)
    print(f"[rows] {name}: quantised x bit-exact on all {w.T} tokens "
          f"({int((asf == 0).sum())} zero/underflow blocks)", flush=True)
    experts = _pick_experts(name, roff)
    toks = list(range(w.T)) if name == "decode" else _sample_tokens(name, ids)
    jobs = _jobs(roff, experts, _token_rows(ids, rinv, w.k, toks))
    counts = np.diff(roff)
    print(f"[case] {name}: oracle for {len(jobs)} jobs, experts {experts[:12]} "
          f"(rows {[int(counts[e]) for e in experts[:12]]})", flush=True)

    rw = ew.rowmajor
    gw1, gw2 = host(ew.gs_w1), host(ew.gs_w2)

    def check_weights(e, r):
        for n in ("w1_q", "w1_sf", "w2_q", "w2_sf"):
            assert np.array_equal(host(rw[n][e]), r[n]), (n, e)
        assert gw1[e] == r["gs_w1"] and gw2[e] == r["gs_w2"]

    def worker_args(rows):
        tok = rperm[rows] // w.k
        return aq[tok], asf[tok]

    y_ref, same = {}, {}
    n_h = n_y = 0
    worker = functools.partial(oracle_pool.expert_rows, gs_a=gs_a, gs_h=np.float32(w.gs_h))
    for e, rows, r in _oracle_rows(w, ew, jobs, worker, check_weights, worker_args):
        n_h += rows.size
        n_y += _check_rows_nvfp4(name, w, tp, e, rows, r, y_ref, same)
    n_out = _check_out(name, w, host(out), tw, rinv, y_ref, same, toks, w.k)
    print(f"[rows] {name}: h and requant on {n_h} rows, y on {n_y} rows "
          f"({n_h - n_y} rows with a certified near-tie difference), out on {n_out} tokens",
          flush=True)
    assert n_h - n_y <= max(2, n_h // 100)


@pytest.mark.timeout(600)
def test_combine_full_size_prefill():
    """The combine alone over the whole prefill output: seeded y rows, the
    prefill routing, against the oracle's combine of the same y."""
    w = I.WORKLOADS["prefill"]
    T, k, H = w.T, w.k, w.H
    ids, tw = I.make_routing(w)
    g = torch.Generator(device=DEV).manual_seed(77)
    y = torch.randn((T * k, H), generator=g, device=DEV).to(torch.bfloat16)
    off, perm, inv, bad = nv.moe_route(torch.from_numpy(ids).to(DEV), w.E)
    print("[case] combine full size prefill", flush=True)
    out = nv.moe_combine(y, inv, torch.from_numpy(tw).to(DEV), off)
    torch.cuda.synchronize()
    roff, _, rinv, _ = R.route(ids, w.E)
    assert np.array_equal(host(inv), rinv)
    yb, ob = host(y), host(out)
    n_valid = int(roff[-1])
    for t0 in range(0, T, 1024):
        sl = slice(t0, min(T, t0 + 1024))
        d = rinv.reshape(T, k)[sl]
        ref = O.combine(yb[d.ravel()], np.arange(d.size, dtype=np.int32), tw[sl], d.size)
        assert_close(bf16_values(ob[sl]), bf16_values(ref), f"combine tokens {t0}..", log=t0 == 0, bf16=True)
        # the fp32 sum in slot order rounds to the oracle's bf16 almost everywhere
        assert (ob[sl] == ref).mean() > 0.999
    print(f"[rows] combine: all {T} tokens x {H} columns to the bar ({n_valid} valid rows)", flush=True)


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
    assert_close(bf16_values(host(out)), bf16_values(ref["out"]), "out with shared expert", bf16=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["prefill", "decode", "skewed"])
def test_mx_forward_full_size(name):
    """The MX variant at full size: the whole re-encoded x bit-exact; sampled
    tokens' k expert rows (weights re-encoded on both sides and compared
    bit-exactly) through h (to the bar), requant + re-encode (certified), y
    (to the bar wherever the GPU's MX h equals the oracle's) and the output."""
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
                h_f32=z((M, Iw), torch.float32), h_q=z((M, Iw // 2), torch.uint8),
                h_sf=z((M, Iw // 16), torch.uint8), y_bf16=z((M, H), torch.bfloat16))
    print(f"[case] mx forward {name} (full size)", flush=True)
    out = nv.moe_expert_forward(x, torch.from_numpy(ids).to(DEV), torch.from_numpy(tw).to(DEV),
                                ew_mx, torch.tensor([w.gs_h], dtype=torch.float32, device=DEV),
                                taps=taps)
    torch.cuda.synchronize()
    tp = {n: host(t) for n, t in taps.items()}
    aq, asf, gs_a = _quantize_x(name, host(x))
    assert tp["gs_a"][0] == gs_a
    amq, amsc = X.nvfp4_to_mx(aq, asf)
    assert np.array_equal(tp["a_q"], amq)
    assert np.array_equal(tp["a_sf"], np.repeat(amsc, 2, axis=1))
    print(f"[rows] mx {name}: re-encoded x bit-exact on all {T} tokens", flush=True)
    _, rperm, rinv, _ = R.route(ids, w.E)
    assert np.array_equal(tp["inv_perm"], rinv)
    toks = _sample_tokens(name, ids)
    rw = ew_mx.rowmajor
    y_ref, same = {}, {}
    n_h = n_y = 0
    jobs = [(e, np.array(sorted(rows))) for e, rows in _token_rows(ids, rinv, k, toks).items()]

    def check_weights(e, r):
        assert np.array_equal(host(rw["w1_q"][e]), r["w1_q"])
        assert np.array_equal(host(rw["w1_sf"][e]), np.repeat(r["w1_sc"], 2, axis=1))
        assert np.array_equal(host(rw["w2_q"][e]), r["w2_q"])

    def worker_args(rows):
        tok = rperm[rows] // k
        return amq[tok], amsc[tok]

    worker = functools.partial(oracle_pool.expert_rows_mx, gs_a=gs_a, gs_h=np.float32(w.gs_h))
    for e, rows, r in _oracle_rows(w, ew_mx, jobs, worker, check_weights, worker_args):
        n_h += rows.size
        assert_close(tp["h_f32"][rows], r["h"], f"mx {name} h e={e}", log=False)
        assert_mx_requant_matches(tp["h_q"][rows], tp["h_sf"][rows], r["h"], w.gs_h,
                                  f"mx {name} requant e={e}")
        ok = (tp["h_q"][rows] == r["h_q"]).all(axis=1) & \
             (tp["h_sf"][rows] == np.repeat(r["h_sc"], 2, axis=1)).all(axis=1)
        if ok.any():
            assert_close(bf16_values(tp["y_bf16"][rows][ok]), bf16_values(r["y"][ok]),
                         f"mx {name} y e={e}", log=False, bf16=True)
        n_y += int(ok.sum())
        for i, d in enumerate(rows):
            y_ref[int(d)] = r["y"][i]
            same[int(d)] = bool(ok[i])
    n_out = _check_out(f"mx {name}", w, host(out), tw, rinv, y_ref, same, toks, k)
    print(f"[rows] mx {name}: h on {n_h} rows, y on {n_y}, out on {n_out} tokens", flush=True)
    assert n_h - n_y <= max(1, n_h // 100)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["prefill", "skewed"])
def test_shared_forward_full_size(name):
    """The shared-expert forward at full size: the shared expert's rows for
    every 64th token and sampled tokens' routed rows, h / requant / y as in
    the routed test, and the sampled tokens' outputs (k routed terms plus the
    shared term)."""
    w = I.WORKLOADS[name]
    print(f"[case] shared forward {name} (full size)", flush=True)
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
    K1 = k + 1
    M = T * K1
    z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=DEV)
    taps = dict(inv_perm=z((M,), torch.int32), perm=z((M,), torch.int32),
                expert_offsets=z((w.E + 2,), torch.int32), h_f32=z((M, Iw), torch.float32),
                h_q=z((M, Iw // 2), torch.uint8), h_sf=z((M, Iw // 16), torch.uint8),
                y_bf16=z((M, H), torch.bfloat16))
    out = nv.moe_expert_forward_shared(x, torch.from_numpy(ids).to(DEV),
                                       torch.from_numpy(tw).to(DEV), both,
                                       torch.tensor([w.gs_h], dtype=torch.float32, device=DEV),
                                       taps=taps)
    torch.cuda.synchronize()
    tp = {n: host(t) for n, t in taps.items()}
    aq, asf, gs_a = _quantize_x(name, host(x))
    # the routing with the shared slot appended: every token in expert E, last
    ids2 = np.concatenate([ids, np.full((T, 1), w.E, np.int32)], axis=1)
    roff, rperm, rinv, _ = R.route(ids2, w.E + 1)
    assert np.array_equal(tp["expert_offsets"], roff)
    assert np.array_equal(tp["perm"], rperm) and np.array_equal(tp["inv_perm"], rinv)
    toks = _sample_tokens(name, ids)
    extra = _token_rows(ids2, rinv, K1, toks)
    extra.setdefault(w.E, []).extend(int(rinv[t * K1 + k]) for t in range(0, T, 64))
    jobs = _jobs(roff, [], extra)

    def check_weights(e, r):
        src = rs if e == w.E else rw
        ee = 0 if e == w.E else e
        for n in ("w1_q", "w1_sf", "w2_q", "w2_sf"):
            assert np.array_equal(host(src[n][ee]), r[n]), (n, e)

    def worker_args(rows):
        tok = rperm[rows] // K1
        return aq[tok], asf[tok]

    y_ref, same = {}, {}
    n_h = n_y = 0
    worker = functools.partial(oracle_pool.expert_rows, gs_a=gs_a, gs_h=np.float32(w.gs_h))
    for e, rows, r in _oracle_rows(w, both, jobs, worker, check_weights, worker_args):
        n_h += rows.size
        n_y += _check_rows_nvfp4(f"shared {name}", w, tp, e, rows, r, y_ref, same)
    twx = np.concatenate([tw, np.ones((T, 1), np.float32)], axis=1)
    n_out = _check_out(f"shared {name}", w, host(out), twx, rinv, y_ref, same, toks, K1)
    print(f"[rows] shared {name}: h on {n_h} rows, y on {n_y}, out on {n_out} tokens", flush=True)
    assert n_h - n_y <= max(1, n_h // 100)
