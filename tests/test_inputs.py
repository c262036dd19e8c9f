"""The seeded workload generators: stated structure, and traceability of the
stored gs_h constants to tests/golden/calibrate_gs_h.py."""

import json
import os

import numpy as np
import pytest
import torch

from nvfp4_block_scaled_04_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gs_h.json")


def test_gs_h_constants_match_calibration_file():
    cal = json.load(open(GOLDEN))
    for name in ("tiny", "decode", "prefill", "skewed", "moe384"):
        assert I.WORKLOADS[name].gs_h == cal[name]["gs_h"], name


def test_tiny_calibration_reproduces():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "calibrate_gs_h", os.path.join(os.path.dirname(__file__), "golden", "calibrate_gs_h.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert mod.calibrate(I.WORKLOADS["tiny"])["gs_h"] == json.load(open(GOLDEN))["tiny"]["gs_h"]


def test_deterministic_generation():
    w = I.WORKLOADS["tiny"]
    assert torch.equal(I.make_x(w), I.make_x(w))
    a, b = I.make_routing(w), I.make_routing(w)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert torch.equal(I.make_expert_weights(w, 2)[0], I.make_expert_weights(w, 2)[0])
    assert not torch.equal(I.make_expert_weights(w, 2)[0], I.make_expert_weights(w, 3)[0])


def test_tiny_special_blocks():
    w = I.WORKLOADS["tiny"]
    x = I.make_x(w).float().view(w.T, w.H // 16, 16)
    amax = x.abs().amax(-1)
    assert int((amax == 0).sum()) == 1
    assert int(((amax > 0) & (amax < 2e-4)).sum()) == 1
    ids, wts = I.make_routing(w)
    assert ids.shape == (64, 2) and np.allclose(wts.sum(1), 1, atol=1e-6)
    assert all(len(set(r)) == 2 for r in ids)


@pytest.mark.parametrize("name", ["decode", "skewed"])
def test_routing_structure(name):
    w = I.WORKLOADS[name]
    ids, wts = I.make_routing(w)
    assert ids.shape == (w.T, w.k) and ids.dtype == np.int32
    assert all(len(set(r)) == w.k for r in ids[:500])          # distinct experts per token
    assert np.allclose(wts.sum(1), 1, atol=1e-5)
    counts = np.bincount(ids.ravel(), minlength=w.E)
    if name == "skewed":
        empty = np.mean(counts == 0)
        share = np.sort(counts)[::-1] / counts.sum()
        assert 0.25 <= empty <= 0.35                             # roughly 30% empty
        assert (share > 0.05).sum() >= 2                         # a few experts above 5%
        assert share[0] <= 1.0 / w.k + 1e-9                      # at most one row per token
    else:
        assert counts.sum() == w.T * w.k


def test_skewed_special_blocks():
    w = I.WORKLOADS["skewed"]
    x = I.make_x(w).float().view(-1, 16)
    amax = x.abs().amax(-1)
    n = x.shape[0]
    assert abs(int((amax == 0).sum()) - n // 100) <= 2
    tiny = (amax > 0) & (amax < 2e-6)
    assert abs(int(tiny.sum()) - n // 100) <= 2


def test_router_logits_are_the_router_workloads_draw():
    # the tiny workload's routing is the oracle router applied to these logits
    from oracle import route as R
    w = I.WORKLOADS["tiny"]
    ids, tw = I.make_routing(w)
    rid, rtw = R.router_topk(I.make_router_logits(w), w.k)
    assert np.array_equal(ids, rid)
    np.testing.assert_allclose(tw, rtw, rtol=1e-6)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus N > 1 exits with status 2 and says so,
    before touching a device."""
    import subprocess
    import sys
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
