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
