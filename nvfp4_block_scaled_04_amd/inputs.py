"""Seeded synthetic inputs for the NVFP4 MoE expert forward.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no quantisation, routing offsets, GEMM or combine).  Both
the HIP path and the CPU oracle take their inputs from here.  Large tensors are
drawn on the requested device with a seeded ``torch.Generator``; a check that
compares the two sides copies the device tensors to the host, so both see the
same bytes.

Workloads (names used by the tests and the benchmark):
  tiny     T=64 H=256 I=128 E=4 k=2; router logits N(0,1) -> top-2 -> softmax
           over the two; x N(0,1) with one all-zero 16-block and one 16-block
           rescaled to amax 1e-4; W1, W2 N(0, 0.02).
  dense    one NVFP4 linear: A (4096, 7168) N(0,1), B (7168, 2048) N(0, 0.02).
  decode   T=256 H=7168 I=2048 E=256 k=8; 8 distinct uniform experts per
           token, weights softmax of 8 N(0,1) logits.
  prefill  as decode with T=8192 (65536 expert rows).
  skewed   T=16384; expert choice Zipf(1.2) over the first 179 experts of a
           seeded permutation (the other 77 = 30% are never chosen), 8
           distinct experts per token by Gumbel-top-8; 1% of x's 16-blocks
           zeroed and 1% rescaled to amax 1e-6.
  moe384   the pages' own MoE shape: T=8192 H=7168 I=3072 E=384 k=6 (49152
           expert rows), routing and distributions as prefill.
decode/prefill/skewed share one weight seed (identical weights).
BF16 values are float32 draws rounded to nearest even by torch.
"""

from dataclasses import dataclass, field
import numpy as np
import torch

WEIGHT_STD = 0.02


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    T: int = 0
    H: int = 0
    I: int = 0
    E: int = 0
    k: int = 0
    routing: str = "uniform"      # "router" | "uniform" | "zipf"
    special: str = ""             # "tiny" | "blocks" | ""
    weight_seed: int = 0
    gs_h: float = 1.0             # global scale of the requantised L2 input
    dense_mkn: tuple = field(default=())

    @property
    def M(self):
        return self.T * self.k


# gs_h values are powers of two written by tests/golden/calibrate_gs_h.py,
# which runs the CPU oracle on a row sample of each workload.
WORKLOADS = {
    "tiny": Workload("tiny", 1, T=64, H=256, I=128, E=4, k=2, routing="router",
                     special="tiny", weight_seed=0x5EED0001, gs_h=1024.0),
    "dense": Workload("dense", 2, dense_mkn=(4096, 7168, 2048), weight_seed=0x5EED0002),
    "decode": Workload("decode", 3, T=256, H=7168, I=2048, E=256, k=8,
                       weight_seed=0x5EED0003, gs_h=32.0),
    "prefill": Workload("prefill", 4, T=8192, H=7168, I=2048, E=256, k=8,
                        weight_seed=0x5EED0003, gs_h=32.0),
    "skewed": Workload("skewed", 5, T=16384, H=7168, I=2048, E=256, k=8, routing="zipf",
                       special="blocks", weight_seed=0x5EED0003, gs_h=32.0),
    "moe384": Workload("moe384", 6, T=8192, H=7168, I=3072, E=384, k=6,
                       weight_seed=0x5EED0006, gs_h=32.0),
}


def custom(name, T, H, I, E, k, routing="uniform", special="", seed=1, gs_h=64.0):
    """A workload of any shape (for edge-case tests)."""
    return Workload(name, 100 + seed, T=T, H=H, I=I, E=E, k=k, routing=routing,
                    special=special, weight_seed=0x5EED1000 + seed, gs_h=gs_h)


def _seed(*parts):
    return int(np.random.SeedSequence([int(p) & 0xFFFFFFFF for p in parts]).generate_state(1)[0])


def _gen(device, *parts):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def _randn(shape, std, device, *seed_parts):
    g = _gen(device, *seed_parts)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def make_x(w: Workload, device="cpu"):
    """Activations x (T, H) bfloat16."""
    x = _randn((w.T, w.H), 1.0, device, 0x5EED0000 + w.wid, 1)
    nb = w.H // 16
    xb = x.view(w.T, nb, 16)
    rng = np.random.default_rng(_seed(0x5EED0000 + w.wid, 2))
    if w.special == "tiny":
        flat = rng.choice(w.T * nb, size=2, replace=False)
        (t0, b0), (t1, b1) = divmod(int(flat[0]), nb), divmod(int(flat[1]), nb)
        xb[t0, b0] = 0.0
        blk = xb[t1, b1]
        xb[t1, b1] = blk * (1e-4 / blk.abs().max())
    elif w.special == "blocks":
        n = w.T * nb
        pick = rng.permutation(n)
        nz = n // 100
        zero = torch.from_numpy(pick[:nz]).to(device)
        tiny = torch.from_numpy(pick[nz:2 * nz]).to(device)
        xf = xb.view(n, 16)
        xf[zero] = 0.0
        sub = xf[tiny]
        xf[tiny] = sub * (1e-6 / sub.abs().amax(dim=1, keepdim=True))
    return x.to(torch.bfloat16)


def make_router_logits(w: Workload):
    """Router logits (T, E) float32 N(0,1): the draw the router workloads'
    routing starts from (same seed and stream as make_routing)."""
    rng = np.random.default_rng(_seed(0x5EED0000 + w.wid, 3))
    return rng.standard_normal((w.T, w.E)).astype(np.float32)


def make_routing(w: Workload):
    """(topk_ids int32 (T, k), topk_w float32 (T, k)) as numpy arrays."""
    rng = np.random.default_rng(_seed(0x5EED0000 + w.wid, 3))
    T, E, k = w.T, w.E, w.k
    if w.routing == "router":
        logits = rng.standard_normal((T, E)).astype(np.float32)
        ids = np.argsort(-logits, axis=1, kind="stable")[:, :k]     # ties -> lower id
        sel = np.take_along_axis(logits, ids, axis=1).astype(np.float64)
    else:
        if w.routing == "uniform":
            keys = rng.random((T, E))
        elif w.routing == "zipf":
            order = rng.permutation(E)
            n_live = int(round(0.70 * E))
            p = np.zeros(E)
            p[order[:n_live]] = 1.0 / np.arange(1, n_live + 1) ** 1.2
            with np.errstate(divide="ignore"):
                keys = np.log(p)[None, :] + rng.gumbel(size=(T, E))
        else:
            raise ValueError(w.routing)
        ids = np.argsort(-keys, axis=1, kind="stable")[:, :k]
        sel = rng.standard_normal((T, k))
    ex = np.exp(sel - sel.max(axis=1, keepdims=True))
    wts = (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids.astype(np.int32), wts


def make_expert_weights(w: Workload, e: int, device="cpu"):
    """Expert e's logical weights: W1 (H, 2I) = [gate | up], W2 (I, H), bf16."""
    w1 = _randn((w.H, 2 * w.I), WEIGHT_STD, device, w.weight_seed, 10, e)
    w2 = _randn((w.I, w.H), WEIGHT_STD, device, w.weight_seed, 11, e)
    return w1.to(torch.bfloat16), w2.to(torch.bfloat16)


def make_dense(w: Workload, device="cpu"):
    """Dense linear operands: A (M, K) bf16 N(0,1), B (K, N) bf16 N(0, 0.02)."""
    M, K, N = w.dense_mkn
    a = _randn((M, K), 1.0, device, 0x5EED0000 + w.wid, 1).to(torch.bfloat16)
    b = _randn((K, N), WEIGHT_STD, device, w.weight_seed, 12).to(torch.bfloat16)
    return a, b


def bf16_to_bits(t):
    """bfloat16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
