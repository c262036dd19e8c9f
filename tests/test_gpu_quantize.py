"""GPU parity of quantisation, routing and weight layout: bit-exact against
the oracle on the same seeded inputs."""

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_04_amd as nv
from nvfp4_block_scaled_04_amd import inputs as I
from oracle import quantize as Q
from oracle import route as R
from oracle import layout as L
from parity import host

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bits_to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def _check_quant(x_dev, groups=1, gs_in=None, what=""):
    print(f"[case] quantize {what} shape={tuple(x_dev.shape)} groups={groups}", flush=True)
    q, sf, gs = nv.quantize(x_dev, groups=groups, gs_in=gs_in)
    torch.cuda.synchronize()
    xb = host(x_dev)
    rq, rsf, rgs = Q.quantize_nvfp4(xb, groups=groups,
                                    gs_in=None if gs_in is None else host(gs_in))
    assert np.array_equal(host(gs).view(np.uint32), rgs.view(np.uint32)), what
    assert np.array_equal(host(sf), rsf), what
    assert np.array_equal(host(q), rq), what
    return rq, rsf


def test_quantize_tiny_workload_special_blocks():
    w = I.WORKLOADS["tiny"]
    x = I.make_x(w, DEV)
    rq, rsf = _check_quant(x, what="tiny")
    assert (rsf == 0).sum() >= 1                  # the all-zero block


@pytest.mark.parametrize("shape", [(1, 16), (3, 48), (37, 272), (130, 1040), (1000, 7168)])
def test_quantize_ragged_shapes(shape):
    g = torch.Generator(device=DEV).manual_seed(shape[0] * 7 + shape[1])
    x = torch.randn(shape, generator=g, device=DEV).to(torch.bfloat16)
    _check_quant(x, what=str(shape))


@pytest.mark.parametrize("R,C,ld,col0,groups,given", [
    (37, 272, 280, 0, 1, False), (64, 256, 1024, 8, 4, False), (130, 1040, 1048, 8, 2, True),
    (1000, 7168, 7176, 0, 1, False)])
def test_quantize_row_stride(R, C, ld, col0, groups, given):
    """Rows ld_x elements apart (a column slice of a wider tensor): the same
    bytes as the oracle's quantisation of the slice."""
    g = torch.Generator(device=DEV).manual_seed(R + C + ld)
    wide = torch.randn((R, ld), generator=g, device=DEV).to(torch.bfloat16)
    x = wide[:, col0:col0 + C]
    assert x.stride(0) == ld and not x.is_contiguous()
    gs_in = torch.tensor([0.5, 3.0][:groups], dtype=torch.float32, device=DEV) if given else None
    _check_quant(x, groups=groups, gs_in=gs_in, what=f"ld_x={ld} col0={col0}")


def test_quantize_zero_underflow_and_negative_zero_blocks():
    g = torch.Generator(device=DEV).manual_seed(3)
    x = torch.randn((64, 256), generator=g, device=DEV)
    x[1, 0:16] = 0.0
    x[2, 16:32] = -0.0
    x[3, 32:48] *= 1e-7                          # far below the underflow threshold
    x[4, 48:64] *= 3e-5                          # subnormal E4M3 scales
    x[5, 64:80] = torch.linspace(-1e-4, 1e-4, 16, device=DEV)
    _check_quant(x.to(torch.bfloat16), what="special")


def _golden_examples():
    # the hand-worked fixtures of the oracle's pins (tests/golden)
    import test_oracle_quantize as T
    return T._load_examples()


@pytest.mark.parametrize("ex", _golden_examples(), ids=lambda e: e["name"])
def test_quantize_hand_worked_examples(ex):
    """The device quantiser on the hand-worked fixtures: the expected bytes
    were derived from the block rule, not by any quantiser program."""
    x32 = ex["x"].astype(np.float32).reshape(1, -1)
    bits = (x32.view(np.uint32) >> 16).astype(np.uint16)
    x = _bits_to_dev(bits)
    gs_in = None if ex["gs"] is None else torch.tensor([ex["gs"]], dtype=torch.float32, device=DEV)
    print(f"[case] quantize worked example {ex['name']}", flush=True)
    q, sf, gs = nv.quantize(x, gs_in=gs_in)
    torch.cuda.synchronize()
    assert host(sf).ravel().tolist() == ex["sf"].tolist()
    assert host(q).ravel().tolist() == ex["q"].tolist()


def test_quantize_all_zero_tensor():
    x = torch.zeros((8, 64), dtype=torch.bfloat16, device=DEV)
    q, sf, gs = nv.quantize(x)
    assert host(gs)[0] == 1.0 and not host(q).any() and not host(sf).any()


def test_quantize_groups_per_expert_scale():
    g = torch.Generator(device=DEV).manual_seed(5)
    x = torch.randn((6 * 32, 256), generator=g, device=DEV)
    x[32:64] *= 50.0
    x[128:160] = 0.0                              # an all-zero group: gs = 1
    _check_quant(x.to(torch.bfloat16), groups=6, what="groups")


def test_quantize_precomputed_scale():
    g = torch.Generator(device=DEV).manual_seed(6)
    x = torch.randn((96, 512), generator=g, device=DEV).to(torch.bfloat16)
    gs = torch.tensor([3.0, 700.0, 0.125], device=DEV)
    _check_quant(x, groups=3, gs_in=gs, what="gs_in")


def _all_bf16_in(lo, hi):
    b = np.arange(1 << 15, dtype=np.uint32)            # non-negative bf16 patterns
    v = (b << 16).view(np.float32)
    keep = (v >= lo) & (v <= hi) & np.isfinite(v)
    return b[keep].astype(np.uint16)


def test_e2m1_encoder_exhaustive_over_bf16():
    # gs = 1 and a leading 6 in every block: scale byte 0x38 (1.0), r = 1, so
    # every code is E2M1 of the bf16 value itself
    vals = _all_bf16_in(0.0, 6.0)
    n = -(-len(vals) // 60) * 4                     # blocks, a multiple of 4 (64-wide rows)
    pad = np.zeros(n * 15, np.uint16)
    pad[:len(vals)] = vals
    blocks = np.concatenate([np.full((n, 1), 0x40C0, np.uint16), pad.reshape(n, 15)], axis=1)
    signs = np.where(np.arange(n)[:, None] % 2 == 1, np.uint16(0x8000), np.uint16(0))
    blocks = blocks | signs
    x = _bits_to_dev(blocks.reshape(-1, 64))
    _check_quant(x, gs_in=torch.ones(1, device=DEV), what="e2m1 sweep")


def test_e4m3_encoder_exhaustive_over_bf16():
    # gs = 1: a block holding only its amax a gets sf = E4M3(a / 6) for every
    # bf16 a from the underflow threshold to E4M3's saturation point
    amax = _all_bf16_in(6 * 2.0 ** -9 * 0.5, 448.0 * 6 * 1.01)
    blocks = np.zeros((len(amax), 16), np.uint16)
    blocks[:, 0] = amax
    blocks[:, 5] = amax ^ 0x8000
    rows = -(-len(blocks) // 4) * 4
    full = np.zeros((rows, 16), np.uint16)
    full[:len(blocks)] = blocks
    x = _bits_to_dev(full.reshape(-1, 64))
    _check_quant(x, gs_in=torch.ones(1, device=DEV), what="e4m3 sweep")


def test_route_all_workloads_bit_exact():
    for name in ("tiny", "decode", "prefill", "skewed"):
        w = I.WORKLOADS[name]
        ids, _ = I.make_routing(w)
        print(f"[case] route {name} T={w.T} k={w.k} E={w.E}", flush=True)
        off, perm, inv, bad = nv.moe_route(torch.from_numpy(ids).to(DEV), w.E)
        torch.cuda.synchronize()
        roff, rperm, rinv, rbad = R.route(ids, w.E)
        assert np.array_equal(host(off), roff), name
        assert np.array_equal(host(perm), rperm), name
        assert np.array_equal(host(inv), rinv), name
        assert host(bad)[0] == rbad == 0


@pytest.mark.parametrize("T,k,E,mode", [
    (0, 4, 8, "uniform"), (1, 1, 1, "uniform"), (5, 3, 7, "uniform"), (3000, 8, 256, "same"),
    (2000, 6, 384, "uniform"), (777, 2, 16, "invalid"), (40000, 8, 4096, "uniform"),
])
def test_route_edge_cases(T, k, E, mode):
    rng = np.random.default_rng(T + k + E)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    if mode == "same":
        ids[:] = E - 1
    if mode == "invalid":
        ids[rng.random((T, k)) < 0.05] = -3
        ids[rng.random((T, k)) < 0.05] = E + 2
    print(f"[case] route edge T={T} k={k} E={E} {mode}", flush=True)
    off, perm, inv, bad = nv.moe_route(torch.from_numpy(ids).to(DEV), E)
    torch.cuda.synchronize()
    roff, rperm, rinv, rbad = R.route(ids, E)
    assert np.array_equal(host(off), roff)
    assert np.array_equal(host(perm), rperm)
    assert np.array_equal(host(inv), rinv)
    assert host(bad)[0] == rbad


@pytest.mark.parametrize("G,Rr,C,inter", [(1, 7, 16, False), (3, 256, 96, True),
                                          (2, 130, 4096, True), (1, 2048, 7168, False)])
def test_weight_layout_bit_exact(G, Rr, C, inter):
    g = torch.Generator(device=DEV).manual_seed(G * Rr + C)
    w = torch.randn((G, Rr, C), generator=g, device=DEV).to(torch.bfloat16)
    print(f"[case] layout G={G} R={Rr} C={C} interleave={inter}", flush=True)
    out = nv.weight_layout(w, inter)
    torch.cuda.synchronize()
    wb = host(w)
    ref = L.interleave_l1(wb) if inter else L.k_major(wb)
    assert np.array_equal(host(out), ref)


def test_expert_weight_prep_bit_exact_tiny():
    w = I.WORKLOADS["tiny"]
    from oracle import moe as O
    w1s, w2s = zip(*[I.make_expert_weights(w, e, DEV) for e in range(w.E)])
    w1 = torch.stack(w1s)
    w2 = torch.stack(w2s)
    ew = nv.prepare_expert_weights([w1], [w2], DEV)
    torch.cuda.synchronize()
    ref = O.prepare_weights(host(w1), host(w2))
    for name in ("w1_q", "w1_sf", "w2_q", "w2_sf"):
        assert np.array_equal(host(ew.rowmajor[name]), ref[name]), name
    assert np.array_equal(host(ew.gs_w1), ref["gs_w1"]) and np.array_equal(host(ew.gs_w2), ref["gs_w2"])


def _pack_reference(q, sf, rows=512, kstage=128):
    """The packed layout written out with NumPy reshapes (a pure re-blocking)."""
    E, N, Kh = q.shape
    S = Kh * 2 // kstage
    Np = -(-N // rows) * rows
    qp = np.zeros((E, Np, Kh), np.uint8); qp[:, :N] = q
    sp = np.zeros((E, Np, sf.shape[2]), np.uint8); sp[:, :N] = sf
    qp = qp.reshape(E, Np // rows, rows, S, kstage // 2).transpose(0, 1, 3, 2, 4)
    sp = sp.reshape(E, Np // rows, rows, S, kstage // 16).transpose(0, 1, 3, 2, 4)
    return qp.ravel(), sp.ravel()


@pytest.mark.parametrize("E,N,K", [(1, 512, 128), (3, 96, 256), (2, 1000, 384), (4, 4096, 7168)])
def test_pack_weights_layout(E, N, K):
    g = torch.Generator(device=DEV).manual_seed(E * N + K)
    q = torch.randint(0, 256, (E, N, K // 2), generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
    sf = torch.randint(0, 256, (E, N, K // 16), generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
    print(f"[case] pack E={E} N={N} K={K}", flush=True)
    pw = nv.pack_weights(q, sf)
    torch.cuda.synchronize()
    rq, rs = _pack_reference(host(q), host(sf))
    assert np.array_equal(host(pw.q), rq) and np.array_equal(host(pw.sf), rs)


def test_combine_rounding_exact_ties():
    # Every product and two-term sum below is exact in fp32 (powers-of-two
    # weights, addends within 2^-13 of each other's exponent), so the GPU's
    # fp32 accumulation and the oracle's fp64 one agree before rounding; the
    # second addend is a multiple of a quarter bf16 ulp of the first, so many
    # sums fall exactly halfway between two bf16 values and the output bits
    # pin round-to-nearest-even.
    rng = np.random.default_rng(11)
    T, H, k = 512, 64, 2
    sign = rng.choice([-1.0, 1.0], size=(T * k, H))
    mant = 1.0 + rng.integers(0, 128, size=(T * k, H)) / 128.0     # bf16 mantissas
    expo = rng.integers(-20, 20, size=(T * k, H))
    y = (sign * mant * np.exp2(expo)).astype(np.float32)
    # slot 1 rows: a quarter-ulp multiple of the slot 0 row of the same token
    base = y.reshape(T, k, H)[:, 0, :]
    ulp4 = np.exp2(np.floor(np.log2(np.abs(base))) - 9)
    y.reshape(T, k, H)[:, 1, :] = (rng.integers(-8, 9, size=(T, H)) * ulp4).astype(np.float32)
    y_bits = (y.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((y_bits.astype(np.uint32) << 16).view(np.float32), y)   # exact bf16
    w = np.ones((T, k), np.float32)
    inv_perm = np.arange(T * k, dtype=np.int32)
    out = nv.moe_combine(_bits_to_dev(y_bits), torch.from_numpy(inv_perm).to(DEV),
                         torch.from_numpy(w).to(DEV),
                         torch.tensor([0, T * k], dtype=torch.int32, device=DEV))
    from oracle import moe as O
    ref = O.combine(y_bits, inv_perm, w, T * k)
    exact = base.astype(np.float64) + y.reshape(T, k, H)[:, 1, :].astype(np.float64)
    r16 = (exact.astype(np.float32).view(np.uint32) & 0xFFFF)
    assert (r16 == 0x8000).sum() > 100                # many exact ties exercised
    assert np.array_equal(host(out).view(np.uint16), ref)


@pytest.mark.parametrize("H", [7296, 14336])
def test_combine_wide_rows_bit_exact(H):
    """Rows wider than one pass of the combine's block (896 vectors of 8 BF16):
    H = 7296 leaves a partial second vector per thread, H = 14336 two full
    ones.  Power-of-two weights and values within 2^7 of each other make every
    fp32 product and three-term sum exact, so the output bits must equal the
    oracle's; a quarter of the slots point past the valid rows and add
    nothing."""
    rng = np.random.default_rng(H)
    T, k, n_valid = 96, 3, 200                                 # rows >= 200 are never read
    mant = 1.0 + rng.integers(0, 128, size=(T * k, H)) / 128.0
    y = (rng.choice([-1.0, 1.0], size=(T * k, H)) * mant
         * np.exp2(rng.integers(-3, 4, size=(T * k, H)))).astype(np.float32)
    y_bits = (y.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((y_bits.astype(np.uint32) << 16).view(np.float32), y)
    inv_perm = rng.integers(0, n_valid, size=T * k).astype(np.int32)
    inv_perm[rng.random(T * k) < 0.25] = n_valid + 7            # invalid expert ids
    w = np.exp2(rng.integers(-3, 2, size=(T, k))).astype(np.float32)
    print(f"[case] combine wide rows T={T} H={H} k={k}", flush=True)
    out = nv.moe_combine(_bits_to_dev(y_bits), torch.from_numpy(inv_perm).to(DEV),
                         torch.from_numpy(w).to(DEV),
                         torch.tensor([0, n_valid], dtype=torch.int32, device=DEV))
    from oracle import moe as O
    ref = O.combine(y_bits, inv_perm, w, n_valid)
    assert np.array_equal(host(out).view(np.uint16), ref)


@pytest.mark.parametrize("T,H,E,k,invalid", [(37, 256, 8, 3, True), (2048, 7168, 256, 8, False),
                                             (0, 256, 4, 2, False), (5, 128, 1, 1, False)])
def test_quantize_scatter_bit_exact(T, H, E, k, invalid):
    """Quantise-and-scatter: every routed row d holds the oracle's NVFP4 of
    token perm[d] // k; rows of invalid ids are left untouched."""
    from oracle import quantize as Q, route as R
    print(f"[case] quantize_scatter T={T} H={H} E={E} k={k} invalid={invalid}", flush=True)
    rng = np.random.default_rng(T + H)
    ids = np.array([rng.permutation(E)[:k] for _ in range(T)], dtype=np.int32).reshape(T, k)
    if invalid and T > 4:
        ids[1, 0] = E + 3
        ids[4, k - 1] = -1
    g = torch.Generator(device=DEV).manual_seed(T * 7 + 1)
    x = torch.randn((T, H), generator=g, device=DEV).to(torch.bfloat16)
    off, perm, inv, bad = nv.moe_route(torch.from_numpy(ids).to(DEV), E)
    q = torch.full((T * k, H // 2), 0xAB, dtype=torch.uint8, device=DEV)
    sf = torch.full((T * k, H // 16), 0xAB, dtype=torch.uint8, device=DEV)
    gs = torch.zeros((1,), dtype=torch.float32, device=DEV)
    nv.quantize_scatter(x, inv, off, k, out=(q, sf, gs))
    torch.cuda.synchronize()
    roff, rperm, _, n_bad = R.route(ids, E)
    xb = host(x)
    rq, rsf, rgs = Q.quantize_nvfp4(xb) if T else (np.zeros((0, H // 2), np.uint8), None, [np.float32(1)])
    assert host(gs)[0] == rgs[0]
    n_valid = int(roff[E])
    gq, gsf = host(q), host(sf)
    if n_valid:
        src = rperm[:n_valid] // k
        assert np.array_equal(gq[:n_valid], rq[src])
        assert np.array_equal(gsf[:n_valid], rsf[src])
    assert np.all(gq[n_valid:] == 0xAB) and np.all(gsf[n_valid:] == 0xAB)
    assert n_bad == (2 if invalid and T > 4 else 0)


def test_l1_on_scattered_rows_equals_the_gather():
    """L1 on the quantise-and-scatter rows (no gather) gives the same bytes as
    L1 gathering the compact rows through perm."""
    from nvfp4_block_scaled_04_amd import inputs as I
    w = I.custom("scatter_l1", T=300, H=512, I=256, E=16, k=4, seed=13)
    print("[case] L1 scattered vs gathered", flush=True)
    pairs = [I.make_expert_weights(w, e, DEV) for e in range(w.E)]
    ew = nv.prepare_expert_weights([torch.stack([p[0] for p in pairs])],
                                   [torch.stack([p[1] for p in pairs])], DEV)
    x = I.make_x(w, DEV)
    ids, _ = I.make_routing(w)
    off, perm, inv, _ = nv.moe_route(torch.from_numpy(ids).to(DEV), w.E)
    M = w.T * w.k
    gs_h = torch.tensor([w.gs_h], dtype=torch.float32, device=DEV)
    a_q, a_sf, gs_a = nv.quantize(x)
    g_q, g_sf, _ = nv.grouped_gemm(nv.EPI_SWIGLU_NVFP4, a_q, a_sf, gs_a, off, ew.w1, ew.gs_w1, M,
                                   a_row_src=perm, a_row_div=w.k, gs_out=gs_h)
    s_q, s_sf, s_gs = nv.quantize_scatter(x, inv, off, w.k)
    h_q, h_sf, _ = nv.grouped_gemm(nv.EPI_SWIGLU_NVFP4, s_q, s_sf, s_gs, off, ew.w1, ew.gs_w1, M,
                                   gs_out=gs_h)
    torch.cuda.synchronize()
    n = int(host(off)[-1])
    assert host(s_gs)[0] == host(gs_a)[0]
    assert np.array_equal(host(h_q)[:n], host(g_q)[:n])
    assert np.array_equal(host(h_sf)[:n], host(g_sf)[:n])
