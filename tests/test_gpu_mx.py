"""GPU parity of the MX variant (NVFP4 re-encoded to E8M0-per-32 MXFP4, run
on the scaled FP4 MFMA) against its oracle (oracle/mx.py): the re-encoding
bit-exact, the grouped GEMM and the forward to the floating-point bar from
identical MX operands."""

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_04_amd as nv
from nvfp4_block_scaled_04_amd import inputs as I
from oracle import mx as X
from oracle import moe as O
from oracle import quantize as Q
from parity import assert_mx_requant_matches, host, bf16_values, assert_close, cosine

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _random_nvfp4_bytes(rows, cols, seed):
    """Seeded arbitrary NVFP4 bytes: every code (incl. -0) and every finite
    non-negative E4M3 scale byte, plus zero-scale and all-zero blocks."""
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    sf = rng.integers(0, 0x7F, size=(rows, cols // 16), dtype=np.uint8)
    sf[rng.random(sf.shape) < 0.05] = 0                       # zero-scale 16-blocks
    z = rng.random((rows, cols // 32)) < 0.05                 # all-zero 32-blocks
    q.reshape(rows, cols // 32, 16)[z] = 0
    q[0, :16] = 0x88                                          # a block of -0 codes only
    sf[0, :2] = 0x38
    return q, sf


def _expand(sc):
    """(R, C/32) E8M0 -> the GPU's (R, C/16) layout (each byte twice)."""
    return np.repeat(sc, 2, axis=1)


@pytest.mark.parametrize("rows,cols", [(1, 32), (37, 256), (512, 7168)])
def test_to_mx_bit_exact(rows, cols):
    print(f"[case] nvfp4_to_mx rows={rows} cols={cols}", flush=True)
    q, sf = _random_nvfp4_bytes(rows, cols, rows + cols)
    gq, gsf = torch.from_numpy(q).to(DEV), torch.from_numpy(sf).to(DEV)
    mq, msc = nv.to_mx(gq, gsf)
    torch.cuda.synchronize()
    rq, rsc = X.nvfp4_to_mx(q, sf)
    assert np.array_equal(host(mq), rq)
    assert np.array_equal(host(msc), _expand(rsc))
    # in place gives the same bytes
    nv.to_mx(gq, gsf, out=(gq, gsf))
    torch.cuda.synchronize()
    assert np.array_equal(host(gq), rq) and np.array_equal(host(gsf), _expand(rsc))


def _randn(shape, seed, std=1.0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV) * std).to(torch.bfloat16)


def _mx_case(counts, N, K, seed, epi, split=False):
    E, M = len(counts), int(sum(counts))
    print(f"[case] mx gemm epi={epi} counts={counts} N={N} K={K} split={split}", flush=True)
    x = _randn((M, K), seed)
    a_q, a_sf, gs_a = nv.quantize(x)
    a_mq, a_msc = nv.to_mx(a_q, a_sf)
    w = _randn((E * N, K), seed + 1, 0.02)
    b_q, b_sf, gs_b = nv.quantize(w, groups=E)
    b_mq, b_msc = nv.to_mx(b_q, b_sf)
    b = nv.pack_weights(b_mq.view(E, N, K // 2), b_msc.view(E, N, K // 16))
    off_h = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    off = torch.from_numpy(off_h).to(DEV)
    ws = None
    if split:
        ws = torch.empty(nv.gemm_splitk_workspace_bytes(epi, M, N, K, E), dtype=torch.uint8, device=DEV)
    res = nv.grouped_gemm(epi, a_mq, a_msc, gs_a, off, b, gs_b, M,
                          gs_out=torch.tensor([64.0], device=DEV), debug=True, workspace=ws, mx=True)
    torch.cuda.synchronize()
    aq, asf, ga = Q.quantize_nvfp4(host(x))
    bq, bsf, gb = Q.quantize_nvfp4(host(w), groups=E)
    amq, amsc = X.nvfp4_to_mx(aq, asf)
    bmq, bmsc = X.nvfp4_to_mx(bq, bsf)
    # operands identical on both sides
    assert np.array_equal(host(a_mq), amq) and np.array_equal(host(a_msc), _expand(amsc))
    bmq, bmsc = bmq.reshape(E, N, K // 2), bmsc.reshape(E, N, K // 32)
    return res, (amq, amsc, ga[0], bmq, bmsc, gb, off_h, aq, asf, bq.reshape(E, N, K // 2),
                 bsf.reshape(E, N, K // 16))


@pytest.mark.parametrize("counts,N,K,split", [
    ([5, 0, 130, 1, 64, 200], 96, 256, False),
    ([128, 128], 512, 1024, False),
    ([300], 256, 2048, True),
    ([0, 0, 3], 32, 384, False),
])
def test_mx_grouped_bf16(counts, N, K, split):
    res, (amq, amsc, ga, bmq, bmsc, gb, off, aq, asf, bq, bsf) = _mx_case(counts, N, K, 31,
                                                                         nv.EPI_BF16, split)
    got = bf16_values(host(res))
    cos_exact = []
    for e in range(len(counts)):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        ref = X.mx_matmul(amq[lo:hi], amsc[lo:hi], ga, bmq[e], bmsc[e], gb[e])
        assert_close(got[lo:hi], bf16_values(O.round_to_bf16(ref)), f"mx expert {e}", bf16=True)
        cos_exact.append(cosine(ref, O.nvfp4_matmul(aq[lo:hi], asf[lo:hi], ga, bq[e], bsf[e], gb[e])))
    print(f"[error study] mx vs exact nvfp4 product: cosine min {min(cos_exact):.5f}", flush=True)


def test_mx_grouped_swiglu():
    counts, N, K = [5, 0, 130, 64], 128, 512
    res, (amq, amsc, ga, bmq, bmsc, gb, off, *_rest) = _mx_case(counts, N, K, 41,
                                                                nv.EPI_SWIGLU_NVFP4)
    _, _, h_dbg = res
    gh = host(h_dbg)
    for e in range(len(counts)):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        acc = X.mx_matmul(amq[lo:hi], amsc[lo:hi], ga, bmq[e], bmsc[e], gb[e])
        from oracle.layout import deinterleave_cols
        g, u = deinterleave_cols(acc)
        assert_close(gh[lo:hi], (O.silu(g) * u).astype(np.float32), f"mx h expert {e}")


def test_mx_forward_tiny_workload():
    w = I.WORKLOADS["tiny"]
    pairs = [I.make_expert_weights(w, e, DEV) for e in range(w.E)]
    w1 = torch.stack([p[0] for p in pairs])
    w2 = torch.stack([p[1] for p in pairs])
    ew = nv.mx_expert_weights(nv.prepare_expert_weights([w1], [w2], DEV))
    x = I.make_x(w, DEV)
    ids, tw = I.make_routing(w)
    T, k, H, Iw = w.T, w.k, w.H, w.I
    M = T * k
    z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=DEV)
    taps = dict(a_q=z((T, H // 2), torch.uint8), a_sf=z((T, H // 16), torch.uint8),
                h_f32=z((M, Iw), torch.float32), h_q=z((M, Iw // 2), torch.uint8),
                h_sf=z((M, Iw // 16), torch.uint8), y_bf16=z((M, H), torch.bfloat16))
    print("[case] mx forward tiny", flush=True)
    out = nv.moe_expert_forward(x, torch.from_numpy(ids).to(DEV), torch.from_numpy(tw).to(DEV), ew,
                                torch.tensor([w.gs_h], dtype=torch.float32, device=DEV), taps=taps)
    torch.cuda.synchronize()
    wts = O.prepare_weights(host(w1), host(w2))
    ref = X.moe_forward_mx(host(x), ids, tw, X.prepare_weights_mx(wts), np.float32(w.gs_h), w.E)
    assert np.array_equal(host(taps["a_q"]), ref["a_q"])
    assert np.array_equal(host(taps["a_sf"]), _expand(ref["a_sc"]))
    assert_close(host(taps["h_f32"]), ref["h"], "mx forward h")
    # requantised + re-encoded h: 32-blocks equal except where the NVFP4
    # requant holds a certified near-tie
    nv_rows = int(ref["offsets"][-1])
    assert_mx_requant_matches(host(taps["h_q"])[:nv_rows], host(taps["h_sf"])[:nv_rows],
                              ref["h"][:nv_rows], w.gs_h, "mx forward requant")
    assert_close(bf16_values(host(out)), bf16_values(ref["out"]), "mx forward out", bf16=True)
    exact = O.moe_forward(host(x), ids, tw, wts, np.float32(w.gs_h), w.E)
    print(f"[error study] mx forward vs exact nvfp4 forward: cosine "
          f"{cosine(bf16_values(ref['out']), bf16_values(exact['out'])):.5f}", flush=True)


@pytest.mark.parametrize("split", [False, True])
def test_mx_dense_config2_sampled_rows(split):
    w = I.WORKLOADS["dense"]
    M, K, N = w.dense_mkn
    print(f"[case] mx dense M={M} K={K} N={N} split={split}", flush=True)
    a, b = I.make_dense(w, DEV)
    a_q, a_sf, gs_a = nv.quantize(a)
    a_mq, a_msc = nv.to_mx(a_q, a_sf)
    bk = nv.weight_layout(b.view(1, K, N), False)[0]
    b_q, b_sf, gs_b = nv.quantize(bk)
    b_mq, b_msc = nv.to_mx(b_q, b_sf)
    off = torch.tensor([0, M], dtype=torch.int32, device=DEV)
    ws = None
    if split:
        ws = torch.empty(nv.gemm_splitk_workspace_bytes(nv.EPI_BF16, M, N, K, 1), dtype=torch.uint8,
                         device=DEV)
    c = nv.grouped_gemm(nv.EPI_BF16, a_mq, a_msc, gs_a, off,
                        nv.pack_weights(b_mq.view(1, N, K // 2), b_msc.view(1, N, K // 16)), gs_b, M,
                        workspace=ws, mx=True)
    torch.cuda.synchronize()
    ab, bb = host(a), host(b)
    gsa = Q.global_scale(ab)
    rows = np.unique(np.concatenate([np.arange(0, M, 97), [M - 1]]))
    aq, asf = Q.quantize_blocks(ab[rows], gsa)
    amq, amsc = X.nvfp4_to_mx(Q.pack_codes(aq), asf)
    bq, bsf, gsb = Q.quantize_nvfp4(np.ascontiguousarray(bb.T))
    bmq, bmsc = X.nvfp4_to_mx(bq, bsf)
    ref = X.mx_matmul(amq, amsc, gsa, bmq, bmsc, gsb[0])
    assert_close(bf16_values(host(c))[rows], bf16_values(O.round_to_bf16(ref)), "mx dense (sampled rows)", bf16=True)
