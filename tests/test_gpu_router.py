"""GPU parity of the router (top-k of the logits + softmax over the k
chosen): ids bit-exact against the oracle, weights to fp32 rounding."""

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_04_amd as nv
from nvfp4_block_scaled_04_amd import inputs as I
from oracle import route as R
from parity import host

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _check(lg, k, what):
    print(f"[case] router {what} T={lg.shape[0]} E={lg.shape[1]} k={k}", flush=True)
    ids, w = nv.router_topk(torch.from_numpy(lg).to(DEV), k)
    torch.cuda.synchronize()
    rid, rw = R.router_topk(lg, k)
    assert np.array_equal(host(ids), rid), what
    np.testing.assert_allclose(host(w), rw, rtol=2e-6, atol=1e-7, err_msg=what)


@pytest.mark.parametrize("T,E,k,seed", [(1, 4, 1, 0), (37, 256, 8, 1), (1000, 384, 6, 2),
                                        (64, 100, 7, 3), (5, 1024, 64, 4), (3, 64, 64, 5)])
def test_router_random_logits(T, E, k, seed):
    lg = np.random.default_rng(seed).standard_normal((T, E)).astype(np.float32)
    _check(lg, k, "random")


def test_router_ties_resolve_to_lower_id():
    rng = np.random.default_rng(7)
    lg = np.round(rng.standard_normal((200, 256)), 1).astype(np.float32)   # many equal logits
    lg[0] = 0.5                                                              # a row of equal logits
    _check(lg, 8, "ties")


def test_router_reproduces_tiny_workload_routing():
    w = I.WORKLOADS["tiny"]
    ids, tw = nv.router_topk(torch.from_numpy(I.make_router_logits(w)).to(DEV), w.k)
    rid, rtw = I.make_routing(w)
    assert np.array_equal(host(ids), rid)
    np.testing.assert_allclose(host(tw), rtw, rtol=2e-6, atol=1e-7)


def test_router_prefill_shape_and_empty():
    lg = np.random.default_rng(9).standard_normal((8192, 256)).astype(np.float32)
    _check(lg, 8, "prefill shape")
    ids, w = nv.router_topk(torch.zeros((0, 16), dtype=torch.float32, device=DEV), 2)
    assert ids.shape == (0, 2) and w.shape == (0, 2)


def test_router_feeds_the_forward():
    """Router -> expert forward on the device, end to end, against the oracle
    router -> oracle forward (ids bit-exact, output to the floating-point bar).
    The oracle forward takes the GPU's fp32 routing weights only after they
    have been checked against its own to fp32 rounding."""
    from oracle import moe as O
    from parity import bf16_values, assert_close
    w = I.custom("router_fwd", T=96, H=256, I=128, E=8, k=2, seed=21)
    print("[case] router -> forward", flush=True)
    lg = np.random.default_rng(22).standard_normal((w.T, w.E)).astype(np.float32)
    pairs = [I.make_expert_weights(w, e, DEV) for e in range(w.E)]
    w1 = torch.stack([p[0] for p in pairs])
    w2 = torch.stack([p[1] for p in pairs])
    ew = nv.prepare_expert_weights([w1], [w2], DEV)
    x = I.make_x(w, DEV)
    ids, tw = nv.router_topk(torch.from_numpy(lg).to(DEV), w.k)
    out = nv.moe_expert_forward(x, ids, tw, ew, torch.tensor([w.gs_h], dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    rid, rw = R.router_topk(lg, w.k)
    assert np.array_equal(host(ids), rid)
    np.testing.assert_allclose(host(tw), rw, rtol=2e-6, atol=1e-7)
    ref = O.moe_forward(host(x), rid, rw.astype(np.float32), O.prepare_weights(host(w1), host(w2)),
                        np.float32(w.gs_h), w.E)
    assert_close(bf16_values(host(out)), bf16_values(ref["out"]), "router -> forward out", bf16=True)
