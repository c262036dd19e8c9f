"""GPU parity of the expert-grouped NVFP4 GEMM (both epilogues) against the
oracle, from identical quantised operands."""

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_04_amd as nv
from nvfp4_block_scaled_04_amd import inputs as I
from oracle import quantize as Q
from oracle import moe as O
from oracle import route as R
from parity import host, bf16_values, assert_close, assert_requant_matches

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _randn(shape, seed, std=1.0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV) * std).to(torch.bfloat16)


def _grouped_case(counts, N, K, seed, epi, gather_k=None, T=0, split_ws=False):
    """Random grouped problem with the given rows per expert, or (gather_k)
    T tokens routed to gather_k distinct experts each, rows gathered by perm."""
    E = len(counts)
    M = T * gather_k if gather_k else int(sum(counts))
    print(f"[case] gemm epi={epi} counts={counts[:8]}.. E={E} M={M} N={N} K={K} gather={gather_k}",
          flush=True)
    if gather_k:
        rng = np.random.default_rng(seed)
        ids = np.stack([rng.permutation(E)[:gather_k] for _ in range(T)]).astype(np.int32)
        off_h, perm_h, _, _ = R.route(ids, E)
        x = _randn((T, K), seed)
        a_q, a_sf, gs_a = nv.quantize(x)
        off = torch.from_numpy(off_h).to(DEV)
        src = torch.from_numpy(perm_h).to(DEV)
        a_rows = perm_h // gather_k
    else:
        x = _randn((M, K), seed)
        a_q, a_sf, gs_a = nv.quantize(x)
        off_h = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        off = torch.from_numpy(off_h).to(DEV)
        src = None
        a_rows = np.arange(M)
    w = _randn((E * N, K), seed + 1, 0.02)
    b_q, b_sf, gs_b = nv.quantize(w, groups=E)
    b = nv.pack_weights(b_q.view(E, N, K // 2), b_sf.view(E, N, K // 16))
    gs_out = torch.tensor([64.0], device=DEV)
    ws = None
    if split_ws:
        nbytes = nv.gemm_splitk_workspace_bytes(epi, M, N, K, E)
        print(f"[case] split-K workspace {nbytes} bytes", flush=True)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    res = nv.grouped_gemm(epi, a_q, a_sf, gs_a, off, b, gs_b, M, a_row_src=src,
                          a_row_div=gather_k or 1, gs_out=gs_out, debug=True, workspace=ws)
    torch.cuda.synchronize()
    # oracle from the same bf16 inputs
    aq, asf, ga = Q.quantize_nvfp4(host(x))
    bq, bsf, gb = Q.quantize_nvfp4(host(w), groups=E)
    bq, bsf = bq.reshape(E, N, K // 2), bsf.reshape(E, N, K // 16)
    return res, (aq, asf, ga[0], bq, bsf, gb, off_h, a_rows)


@pytest.mark.parametrize("counts,N,K", [
    ([5, 0, 130, 1, 64, 200], 96, 256),
    ([128, 128], 128, 128),
    ([0, 0, 3], 32, 384),
    ([300], 256, 1024),
])
def test_grouped_bf16_epilogue(counts, N, K):
    res, (aq, asf, ga, bq, bsf, gb, off, rows) = _grouped_case(counts, N, K, 11, nv.EPI_BF16)
    got = bf16_values(host(res))
    for e in range(len(counts)):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        ref = bf16_values(O.round_to_bf16(
            O.nvfp4_matmul(aq[rows[lo:hi]], asf[rows[lo:hi]], ga, bq[e], bsf[e], gb[e])))
        assert_close(got[lo:hi], ref, f"expert {e}", bf16=True)


@pytest.mark.parametrize("counts,N,K", [
    ([5, 0, 130, 1, 64, 200], 96, 1024),      # 8 K stages: 2 parts
    ([5, 0, 130, 1, 64, 200], 96, 1152),      # 9 stages: parts of 4 and 5
    ([300], 512, 2048),                       # 16 stages: 4 parts
    ([0, 1], 32, 512),                        # one row, 4 stages: no split
    ([1024], 2048, 7168),                     # a dense linear of 1024 rows: 64 tiles of 64 x 512
])
def test_grouped_bf16_split_k(counts, N, K):
    """Launches with few tiles split K when the workspace allows it; each
    part's fp32 partials are summed in order by a second kernel."""
    res, (aq, asf, ga, bq, bsf, gb, off, rows) = _grouped_case(counts, N, K, 13, nv.EPI_BF16,
                                                               split_ws=True)
    nbytes = nv.gemm_splitk_workspace_bytes(nv.EPI_BF16, int(sum(counts)), N, K, len(counts))
    if K // 128 >= 8:
        assert nbytes > nv.gemm_workspace_bytes(), "this launch is expected to split K"
    got = bf16_values(host(res))
    for e in range(len(counts)):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        ref = bf16_values(O.round_to_bf16(
            O.nvfp4_matmul(aq[rows[lo:hi]], asf[rows[lo:hi]], ga, bq[e], bsf[e], gb[e])))
        assert_close(got[lo:hi], ref, f"expert {e}", bf16=True)


@pytest.mark.parametrize("counts,N,K,gk,T", [
    ([5, 0, 130, 1, 64, 200], 64, 256, None, 0),
    ([0, 37, 0, 91], 256, 512, None, 0),
    ([0] * 8, 128, 256, 3, 45),
])
def test_grouped_swiglu_epilogue(counts, N, K, gk, T):
    res, (aq, asf, ga, bq, bsf, gb, off, rows) = _grouped_case(
        counts, N, K, 21, nv.EPI_SWIGLU_NVFP4, gather_k=gk, T=T)
    c_q, c_sf, h_dbg = res
    gq, gsf, gh = host(c_q), host(c_sf), host(h_dbg)
    E = bq.shape[0]
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        ref_h = O.l1_swiglu(aq[rows[lo:hi]], asf[rows[lo:hi]], ga, bq[e], bsf[e], gb[e])
        assert_close(gh[lo:hi], ref_h, f"h expert {e}")
        assert_requant_matches(gq[lo:hi], gsf[lo:hi], ref_h, 64.0, f"requant expert {e}")


@pytest.mark.parametrize("split", [False, True])
def test_dense_linear_config2_sampled_rows(split):
    w = I.WORKLOADS["dense"]
    M, K, N = w.dense_mkn
    print(f"[case] dense M={M} K={K} N={N}", flush=True)
    a, b = I.make_dense(w, DEV)
    a_q, a_sf, gs_a = nv.quantize(a)
    bk = nv.weight_layout(b.view(1, K, N), False)[0]              # (N, K)
    b_q, b_sf, gs_b = nv.quantize(bk)
    off = torch.tensor([0, M], dtype=torch.int32, device=DEV)
    ws = None
    if split:
        nbytes = nv.gemm_splitk_workspace_bytes(nv.EPI_BF16, M, N, K, 1)
        print(f"[case] dense split-K workspace {nbytes} bytes", flush=True)
        # 64-token tiles (256 of them) cover 256 CUs: K is not split even
        # when the workspace would allow it
        assert nbytes == nv.gemm_workspace_bytes(), "the dense shape runs unsplit 64-token tiles"
        nbytes = nv.gemm_splitk_workspace_bytes(nv.EPI_BF16, 1024, N, K, 1)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    c = nv.grouped_gemm(nv.EPI_BF16, a_q, a_sf, gs_a, off,
                        nv.pack_weights(b_q.view(1, N, K // 2), b_sf.view(1, N, K // 16)), gs_b, M,
                        workspace=ws)
    torch.cuda.synchronize()
    ab, bb = host(a), host(b)
    gsa = Q.global_scale(ab)
    # all of A and B bit-exact on the GPU
    aq_all = np.empty((M, K // 2), np.uint8)
    asf_all = np.empty((M, K // 16), np.uint8)
    for r0 in range(0, M, 1024):
        cq, cs = Q.quantize_blocks(ab[r0:r0 + 1024], gsa)
        aq_all[r0:r0 + 1024], asf_all[r0:r0 + 1024] = Q.pack_codes(cq), cs
    assert np.array_equal(host(a_q), aq_all) and np.array_equal(host(a_sf), asf_all)
    bq, bsf, gsb = Q.quantize_nvfp4(np.ascontiguousarray(bb.T))
    assert np.array_equal(host(b_q), bq) and np.array_equal(host(b_sf), bsf)
    assert host(gs_a)[0] == gsa and host(gs_b)[0] == gsb[0]
    # rows of every 128-row m tile (its first, last and a middle row) and
    # every 61st row, all N columns (all n tiles)
    mt = np.arange(0, M, 128)
    rows = np.unique(np.concatenate([mt, mt + 127, mt + 53, np.arange(0, M, 61)]))
    ref = bf16_values(O.dense_linear(aq_all[rows], asf_all[rows], gsa, bq, bsf, gsb[0]))
    assert_close(bf16_values(host(c))[rows], ref, f"dense linear ({rows.size} rows, every m tile)", bf16=True)


# 315 rows over 16 experts (<= 32 per expert on average: the 32-token tile
# configuration); experts of 0, 1, 31-33 and up to 70 rows
SMALL_COUNTS = [0, 1, 31, 32, 33, 70, 5, 0, 2, 9, 17, 64, 3, 0, 8, 40]


@pytest.mark.parametrize("K", [128, 256, 384, 512, 640, 1152])
@pytest.mark.parametrize("epi", ["bf16", "swiglu"])
def test_small_expert_tiles(epi, K):
    """Launches whose experts average at most 32 rows run 32-token tiles
    with loads three stages ahead: K of 1 to 9 stages covers every way the
    last stages are peeled; experts above 32 rows span several tiles."""
    if epi == "bf16":
        res, (aq, asf, ga, bq, bsf, gb, off, rows) = _grouped_case(SMALL_COUNTS, 96, K, 31,
                                                                   nv.EPI_BF16)
        got = bf16_values(host(res))
    else:
        res, (aq, asf, ga, bq, bsf, gb, off, rows) = _grouped_case(SMALL_COUNTS, 128, K, 33,
                                                                   nv.EPI_SWIGLU_NVFP4)
        gq, gsf, gh = (host(t) for t in res)
    for e in range(len(SMALL_COUNTS)):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        if epi == "bf16":
            ref = bf16_values(O.round_to_bf16(
                O.nvfp4_matmul(aq[rows[lo:hi]], asf[rows[lo:hi]], ga, bq[e], bsf[e], gb[e])))
            assert_close(got[lo:hi], ref, f"expert {e}", bf16=True)
        else:
            ref_h = O.l1_swiglu(aq[rows[lo:hi]], asf[rows[lo:hi]], ga, bq[e], bsf[e], gb[e])
            assert_close(gh[lo:hi], ref_h, f"h expert {e}")
            assert_requant_matches(gq[lo:hi], gsf[lo:hi], ref_h, 64.0, f"requant expert {e}")


@pytest.mark.parametrize("E,rows_per_expert", [
    (1024, 32),     # the largest expert count of 32-token tiles, at its row limit
    (1025, 4),      # one expert more: 128-token tiles
    (4096, 33),     # the largest expert count of the API, 128-token tiles
])
def test_tile_configuration_limits(E, rows_per_expert):
    """Expert counts at the edges of each tile configuration (the expert
    prefix lives in LDS beside the stage buffers); sampled experts against
    the oracle."""
    rng = np.random.default_rng(E)
    counts = rng.integers(0, 2 * rows_per_expert + 1, size=E)
    counts[-1] = 0
    counts[0] = rows_per_expert + 7
    res, (aq, asf, ga, bq, bsf, gb, off, rows) = _grouped_case(list(counts), 32, 128, 41, nv.EPI_BF16)
    got = bf16_values(host(res))
    for e in sorted({0, 1, E // 2, E - 2, E - 1, *rng.integers(0, E, size=12).tolist()}):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        ref = bf16_values(O.round_to_bf16(
            O.nvfp4_matmul(aq[rows[lo:hi]], asf[rows[lo:hi]], ga, bq[e], bsf[e], gb[e])))
        assert_close(got[lo:hi], ref, f"expert {e}", bf16=True)
