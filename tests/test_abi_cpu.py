"""The C ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments on the host before touching HIP (no compute calls)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4moe.h")


@pytest.fixture(scope="module")
def L():
    from nvfp4_block_scaled_04_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from nvfp4_block_scaled_04_amd import build
        build.build(verbose=False)
    return binding.lib()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_0-9]+)\s*\(", text)
    skip = {"sizeof", "defined"}
    return sorted({n for n in names if n not in skip and (n.startswith("nvfp4_") or n.startswith("moe_"))})


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n


def test_binding_signatures_cover_header():
    from nvfp4_block_scaled_04_amd import binding
    assert set(_declared()) == set(binding.SIGNATURES)


def test_status_strings_and_version(L):
    assert L.nvfp4_status_string(0) == b"ok"
    for s in (-1, -2, -3, -4, -5):
        assert L.nvfp4_status_string(s) != b"unknown status"
    assert L.nvfp4_version() >= 100


def test_workspace_sizes(L):
    assert L.nvfp4_quantize_workspace_size(1, 8192, 7168) > 0
    assert L.nvfp4_quantize_workspace_size(0, 8, 16) == 0
    assert L.nvfp4_moe_route_workspace_size(8192, 8, 256) >= 257 * 4
    small = L.moe_expert_forward_workspace_size(64, 256, 128, 4, 2)
    big = L.moe_expert_forward_workspace_size(8192, 7168, 2048, 256, 8)
    assert 0 < small < big
    # y (M x H bf16) dominates the forward workspace
    assert big >= 65536 * 7168 * 2


FAKE = 0x1000  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("args,status", [
    ((FAKE, 1, 4, 15, 16, None, FAKE, FAKE, FAKE, FAKE, 1 << 20, None), -2),   # cols % 16
    ((FAKE, -1, 4, 16, 16, None, FAKE, FAKE, FAKE, FAKE, 1 << 20, None), -2),
    ((FAKE, 1, 4, 32, 16, None, FAKE, FAKE, FAKE, FAKE, 1 << 20, None), -2),   # ld_x < cols
    ((FAKE, 1, 4, 32, 36, None, FAKE, FAKE, FAKE, FAKE, 1 << 20, None), -2),   # ld_x % 8
    ((None, 1, 4, 16, 16, None, FAKE, FAKE, FAKE, FAKE, 1 << 20, None), -1),   # null x
    ((FAKE, 1, 4, 16, 16, None, FAKE, FAKE, FAKE, None, 0, None), -3),         # no workspace
    ((FAKE + 8, 1, 4, 16, 16, None, FAKE, FAKE, FAKE, FAKE, 1 << 20, None), -1),  # misaligned x
])
def test_quantize_rejects(L, args, status):
    assert L.nvfp4_quantize(*args) == status
    assert L.nvfp4_last_error() != b""


def test_route_rejects(L):
    assert L.nvfp4_moe_route(FAKE, 4, 0, 8, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, None) == -2
    assert L.nvfp4_moe_route(FAKE, 4, 2, 0, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, None) == -2
    assert L.nvfp4_moe_route(FAKE, 4, 2, 8, None, FAKE, FAKE, None, FAKE, 1 << 20, None) == -1
    assert L.nvfp4_moe_route(FAKE, 4, 2, 8, FAKE, FAKE, FAKE, None, FAKE, 4, None) == -3


def _gemm(L, **kw):
    a = dict(epi=0, a_q=FAKE, a_sf=FAKE, gs_a=FAKE, src=None, div=1, off=FAKE, E=4, M=64, N=256,
             K=256, b_q=FAKE, b_sf=FAKE, gs_b=FAKE, gs_out=FAKE, c=FAKE, cq=FAKE, csf=FAKE,
             dbg=None, ws=FAKE, wsb=256)
    a.update(kw)
    return L.nvfp4_grouped_gemm(a["epi"], a["a_q"], a["a_sf"], a["gs_a"], a["src"], a["div"],
                                a["off"], a["E"], a["M"], a["N"], a["K"], a["b_q"], a["b_sf"],
                                a["gs_b"], a["gs_out"], a["c"], a["cq"], a["csf"], a["dbg"],
                                a["ws"], a["wsb"], None)


def test_gemm_rejects(L):
    assert _gemm(L, epi=7) == -1
    assert _gemm(L, K=200) == -2
    assert _gemm(L, K=64) == -2
    assert _gemm(L, N=48) == -2
    assert _gemm(L, E=0) == -2
    assert _gemm(L, c=None) == -1
    assert _gemm(L, epi=1, cq=None) == -1
    assert _gemm(L, src=FAKE, div=0) == -2
    assert _gemm(L, off=None) == -1
    assert _gemm(L, M=1 << 30, N=1 << 29) == -2          # tile indices would overflow 32 bits
    # A codes of 4 GiB or more would wrap the kernels' 32-bit row offsets
    assert _gemm(L, M=1_200_000, N=2048, K=7168) == -2    # 4.3 GB without a gather
    assert _gemm(L, M=300_000, N=256, K=28672) == -2
    assert _gemm(L, M=1_198_373, N=256, K=7168) == -2     # the first M with M*K/2 >= 2^32
    assert _gemm(L, K=1 << 24) == -2                      # K stage offsets of a weight tile


def test_gemm_workspace(L):
    need = L.nvfp4_grouped_gemm_workspace_size()
    assert need >= 32                                     # eight 32-bit counters
    # the split-K size is never below the minimum (and is the minimum for
    # invalid shapes or when no device can be queried)
    assert L.nvfp4_grouped_gemm_splitk_workspace_size(0, 4096, 2048, 7168, 1) >= need
    assert L.nvfp4_grouped_gemm_splitk_workspace_size(0, -1, 2048, 7168, 1) == need
    assert L.nvfp4_grouped_gemm_splitk_workspace_size(1, 4096, 2048, 7168, 1) == need  # SwiGLU
    assert _gemm(L, ws=None, wsb=0) == -3
    assert _gemm(L, wsb=need - 1) == -3
    assert _gemm(L, ws=FAKE + 2) == -3                    # not 4-byte aligned
    assert _gemm(L, M=0, ws=None, wsb=0) == 0             # nothing to do, nothing launched


def test_router_rejects(L):
    assert L.nvfp4_router_topk(FAKE, 4, 0, 1, FAKE, FAKE, None) == -2          # E < 1
    assert L.nvfp4_router_topk(FAKE, 4, 1025, 1, FAKE, FAKE, None) == -2       # E > 1024
    assert L.nvfp4_router_topk(FAKE, 4, 8, 9, FAKE, FAKE, None) == -2          # k > E
    assert L.nvfp4_router_topk(FAKE, 4, 256, 65, FAKE, FAKE, None) == -2       # k > 64
    assert L.nvfp4_router_topk(None, 4, 8, 2, FAKE, FAKE, None) == -1
    assert L.nvfp4_router_topk(FAKE + 2, 4, 8, 2, FAKE, FAKE, None) == -1      # misaligned
    assert L.nvfp4_router_topk(None, 0, 8, 2, None, None, None) == 0           # nothing to do


def test_combine_and_forward_reject(L):
    assert L.nvfp4_moe_combine(FAKE, FAKE, FAKE, FAKE, 4, 2, 4, 12, FAKE, None) == -2
    assert L.nvfp4_moe_combine(None, FAKE, FAKE, FAKE, 4, 2, 4, 16, FAKE, None) == -1
    f = lambda **kw: L.moe_expert_forward(
        FAKE, kw.get("T", 4), kw.get("H", 256), kw.get("I", 128), kw.get("E", 4), kw.get("k", 2),
        FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, kw.get("gs_h", FAKE), FAKE, None,
        kw.get("ws", FAKE), kw.get("wsb", 1 << 30), None)
    assert f(H=200) == -2
    assert f(I=64) == -2
    assert f(k=0) == -2
    assert f(gs_h=None) == -1
    assert f(wsb=16) == -3
    assert f(ws=FAKE + 16) == -3
    # quantised x or h of 4 GiB or more would wrap the GEMMs' 32-bit row offsets
    assert f(T=1_200_000, H=7168, I=128, k=1) == -2       # x codes 4.3 GB
    assert f(T=524_288, H=1024, I=2048, k=8) == -2        # h codes 4.3 GB
    assert L.nvfp4_weight_layout(FAKE, 2, 4, 24, 1, FAKE, None) == -2
    assert L.nvfp4_weight_layout(FAKE, 2, 4, 32, 1, None, None) == -1


def test_packed_weight_sizes_and_rejects(L):
    sf = ctypes.c_size_t(0)
    assert L.nvfp4_packed_weight_bytes(2, 1000, 384, ctypes.byref(sf)) == 2 * 1024 * 192
    assert sf.value == 2 * 1024 * 24
    assert L.nvfp4_packed_weight_bytes(2, 1000, 100, ctypes.byref(sf)) == 0
    assert L.nvfp4_pack_weights(FAKE, FAKE, 2, 100, 200, FAKE, FAKE, None) == -2
    assert L.nvfp4_pack_weights(None, FAKE, 2, 100, 256, FAKE, FAKE, None) == -1
    assert L.nvfp4_pack_weights(FAKE, FAKE, 2, 100, 256, FAKE, FAKE + 8, None) == -1


def test_mx_entry_points_reject(L):
    B = 1 << 20
    assert L.nvfp4_to_mx(FAKE, FAKE, 4, 48, FAKE + B, FAKE + B, None) == -2     # cols % 32
    assert L.nvfp4_to_mx(FAKE, FAKE, -1, 64, FAKE + B, FAKE + B, None) == -2
    assert L.nvfp4_to_mx(None, FAKE, 4, 64, FAKE + B, FAKE + B, None) == -1
    assert L.nvfp4_to_mx(FAKE + 8, FAKE, 4, 64, FAKE + B, FAKE + B, None) == -1  # misaligned codes
    assert L.nvfp4_to_mx(FAKE, FAKE, 4, 64, FAKE + 16, FAKE + B, None) == -1     # partial overlap
    assert L.nvfp4_to_mx(None, None, 0, 64, None, None, None) == 0               # nothing to do
    # the MX GEMM validates like the NVFP4 one
    args = lambda **kw: (kw.get("epi", 0), FAKE, FAKE, FAKE, None, 1, FAKE, 4, 64,
                         kw.get("N", 64), kw.get("K", 256), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                         FAKE, None, FAKE, 1 << 20, None)
    assert L.nvfp4_mx_grouped_gemm(*args(K=200)) == -2
    assert L.nvfp4_mx_grouped_gemm(*args(N=48)) == -2
    assert L.nvfp4_mx_grouped_gemm(*args(epi=7)) == -1
    f = lambda **kw: L.moe_expert_forward_mx(
        FAKE, 4, kw.get("H", 256), 128, 4, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
        FAKE, FAKE, None, FAKE, kw.get("wsb", 1 << 30), None)
    assert f(H=200) == -2
    assert f(wsb=16) == -3


def test_shared_forward_rejects(L):
    f = lambda **kw: L.moe_expert_forward_shared(
        FAKE, kw.get("T", 4), kw.get("H", 256), 128, kw.get("E", 4), kw.get("k", 2), FAKE, FAKE,
        FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, kw.get("ws", FAKE),
        kw.get("wsb", 1 << 30), None)
    assert f(k=64) == -2                      # k + 1 slots must fit 64
    assert f(E=4096) == -2                    # E + 1 experts must fit 4096
    assert f(H=200) == -2                     # checked by the routed forward before anything runs
    assert f(wsb=16) == -3
    assert f(ws=FAKE + 16) == -3
    need = L.moe_expert_forward_shared_workspace_size(64, 256, 128, 4, 2)
    assert need > L.moe_expert_forward_workspace_size(64, 256, 128, 5, 3)


def test_quantize_scatter_rejects(L):
    f = lambda **kw: L.nvfp4_quantize_scatter(FAKE, kw.get("T", 4), kw.get("H", 256), kw.get("k", 2),
                                              FAKE, FAKE, kw.get("E", 8), FAKE, FAKE,
                                              kw.get("gs", FAKE), kw.get("ws", FAKE),
                                              kw.get("wsb", 1 << 20), None)
    assert f(H=24) == -2
    assert f(k=0) == -2
    assert f(E=0) == -2
    assert f(gs=None) == -1
    assert f(wsb=0) == -3
    assert L.nvfp4_quantize_scatter_workspace_size(0, 256) == 0
    assert L.nvfp4_quantize_scatter_workspace_size(8192, 7168) >= 4


def test_noalloc_forward_rejects_before_touching_the_device(L):
    f = lambda **kw: L.moe_expert_forward_noalloc(
        FAKE, kw.get("T", 4), kw.get("H", 256), kw.get("I", 128), 4, kw.get("k", 2), FAKE, FAKE,
        FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, kw.get("gs_h", FAKE), FAKE, None, None)
    # a shape whose workspace exceeds the static scratch
    assert L.moe_expert_forward_workspace_size(600, 7168, 2048, 4, 8) > (64 << 20)
    assert f(T=600, H=7168, I=2048, k=8) == -3
    assert b"static scratch" in L.nvfp4_last_error()
    assert f(H=200) == -2
    assert f(gs_h=None) == -1
