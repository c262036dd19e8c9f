"""moe_expert_forward_noalloc (the forward on the library's static scratch,
for callers that cannot allocate) against moe_expert_forward with a
workspace: bit-identical outputs and taps on two calls in a row, the second
with a smaller input."""

import pytest
import torch

import nvfp4_block_scaled_04_amd as nv
from nvfp4_block_scaled_04_amd import inputs as I

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bits(t):
    return t.contiguous().view(torch.int16) if t.dtype == torch.bfloat16 else t


def test_noalloc_forward_matches_workspace_forward_twice():
    w = I.custom("noalloc", T=256, H=7168, I=2048, E=8, k=2, seed=21, gs_h=32.0)
    pairs = [I.make_expert_weights(w, e, DEV) for e in range(w.E)]
    ew = nv.prepare_expert_weights([torch.stack([p[0] for p in pairs])],
                                   [torch.stack([p[1] for p in pairs])], DEV)
    gs_h = torch.tensor([w.gs_h], dtype=torch.float32, device=DEV)
    x_all = I.make_x(w, DEV)
    ids_all, tw_all = I.make_routing(w)
    for T in (256, 40):                      # the second call is smaller
        x = x_all[:T].contiguous()
        ids = torch.from_numpy(ids_all[:T].copy()).to(DEV)
        tw = torch.from_numpy(tw_all[:T].copy()).to(DEV)
        M = T * w.k
        mk = lambda: dict(h_q=torch.zeros((M, w.I // 2), dtype=torch.uint8, device=DEV),
                          h_sf=torch.zeros((M, w.I // 16), dtype=torch.uint8, device=DEV),
                          y_bf16=torch.zeros((M, w.H), dtype=torch.bfloat16, device=DEV))
        t_ref, t_na = mk(), mk()
        print(f"[case] noalloc forward T={T} H={w.H} I={w.I} E={w.E} k={w.k}", flush=True)
        ref = nv.moe_expert_forward(x, ids, tw, ew, gs_h, taps=t_ref)
        out = torch.full((T, w.H), float("nan"), dtype=torch.bfloat16, device=DEV)
        got = nv.moe_expert_forward_noalloc(x, ids, tw, ew, gs_h, out=out, taps=t_na)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(_bits(got), _bits(ref)), f"T={T}: outputs differ"
        for n in t_ref:
            assert torch.equal(_bits(t_na[n]), _bits(t_ref[n])), f"T={T}: tap {n} differs"
        # and without taps, straight after
        out2 = torch.full((T, w.H), float("nan"), dtype=torch.bfloat16, device=DEV)
        nv.moe_expert_forward_noalloc(x, ids, tw, ew, gs_h, out=out2)
        torch.cuda.synchronize()
        assert torch.equal(_bits(out2), _bits(ref)), f"T={T}: outputs differ (no taps)"
