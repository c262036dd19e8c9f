"""The forward is graph-capturable and deterministic.

README "NVFP4 MegaMoE Kernel", "What We Have" (grouped GEMM): the kernel is
safe under graph capture because its workspace is allocated up front and it
allocates nothing at run time; "File Structure" lists a graph-capture test.  Here: capture moe_expert_forward in a hipGraph (through
torch.cuda.graph), replay it several times with eager work and
synchronisation in between, and require every replay to equal the eager
result bit for bit; and two eager runs must be bitwise identical."""

import pytest
import torch

import nvfp4_block_scaled_04_amd as nv
from nvfp4_block_scaled_04_amd import inputs as I

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _setup(w):
    pairs = [I.make_expert_weights(w, e, DEV) for e in range(w.E)]
    ew = nv.prepare_expert_weights([torch.stack([p[0] for p in pairs])],
                                   [torch.stack([p[1] for p in pairs])], DEV)
    x = I.make_x(w, DEV)
    ids, tw = I.make_routing(w)
    return (x, torch.from_numpy(ids).to(DEV), torch.from_numpy(tw).to(DEV), ew,
            torch.tensor([w.gs_h], dtype=torch.float32, device=DEV))


@pytest.mark.parametrize("w", [I.WORKLOADS["tiny"],
                               I.custom("graph_mid", T=300, H=512, I=256, E=16, k=4, seed=9)],
                         ids=lambda w: w.name)
def test_graph_capture_replays_match_eager(w):
    print(f"[case] graph {w.name}", flush=True)
    x, ids, tw, ew, gs_h = _setup(w)
    ws = nv.forward_workspace(w.T, w.H, w.I, w.E, w.k, DEV)
    out = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=DEV)
    nv.moe_expert_forward(x, ids, tw, ew, gs_h, out=out, workspace=ws)   # eager (also warms up)
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out.zero_()
        with torch.cuda.graph(g, stream=s):
            nv.moe_expert_forward(x, ids, tw, ew, gs_h, out=out, workspace=ws)
    torch.cuda.synchronize()
    for r in range(4):
        out.fill_(0)                                  # eager work between replays
        ws.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {r}"


@pytest.mark.parametrize("variant", ["mx", "shared"])
def test_graph_capture_variants(variant):
    """The MX variant and the shared-expert forward replay from a graph bit
    for bit like the eager call."""
    w = I.custom("graph_var", T=300, H=512, I=256, E=16, k=4, seed=9)
    print(f"[case] graph {variant}", flush=True)
    nexp = w.E + 1 if variant == "shared" else w.E
    pairs = [I.make_expert_weights(w, e, DEV) for e in range(nexp)]
    ew = nv.prepare_expert_weights([torch.stack([p[0] for p in pairs])],
                                   [torch.stack([p[1] for p in pairs])], DEV)
    if variant == "mx":
        ew = nv.mx_expert_weights(ew)
    x = I.make_x(w, DEV)
    ids_h, tw_h = I.make_routing(w)
    ids, tw = torch.from_numpy(ids_h).to(DEV), torch.from_numpy(tw_h).to(DEV)
    gs_h = torch.tensor([w.gs_h], dtype=torch.float32, device=DEV)
    out = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=DEV)
    if variant == "shared":
        ws = nv.forward_shared_workspace(w.T, w.H, w.I, w.E, w.k, DEV)
        call = lambda: nv.moe_expert_forward_shared(x, ids, tw, ew, gs_h, out=out, workspace=ws)
    else:
        ws = nv.forward_workspace(w.T, w.H, w.I, w.E, w.k, DEV)
        call = lambda: nv.moe_expert_forward(x, ids, tw, ew, gs_h, out=out, workspace=ws)
    call()
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.synchronize()
    for r in range(3):
        out.fill_(0)
        ws.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"{variant} replay {r}"


def test_forward_is_deterministic():
    w = I.custom("determinism", T=500, H=384, I=256, E=32, k=6, routing="zipf", seed=10)
    print(f"[case] determinism {w.name}", flush=True)
    x, ids, tw, ew, gs_h = _setup(w)
    a = nv.moe_expert_forward(x, ids, tw, ew, gs_h)
    b = nv.moe_expert_forward(x, ids, tw, ew, gs_h)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
