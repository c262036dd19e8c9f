"""Oracle work for sampled rows of a full-size workload, run in worker
processes (spawned; they import only NumPy and the oracle, never the GPU)."""

import numpy as np

from oracle import moe as O
from oracle import quantize as Q


def init_worker():
    """Keep each worker's BLAS to a couple of threads: the pool itself is the
    parallelism (16 workers fill a GPU machine's CPU share)."""
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(2)
    except Exception:
        pass


def expert_rows(w1_bits, w2_bits, a_q, a_sf, gs_a, gs_h):
    """Prepare one expert's weights and run L1 -> SwiGLU -> requant -> L2 for
    the given quantised activation rows."""
    p = O.prepare_expert_weights(w1_bits, w2_bits)
    h = O.l1_swiglu(a_q, a_sf, gs_a, p["w1_q"], p["w1_sf"], p["gs_w1"])
    codes, h_sf = Q.quantize_blocks(h, np.float32(gs_h))
    h_q = Q.pack_codes(codes)
    y = O.l2(h_q, h_sf, np.float32(gs_h), p["w2_q"], p["w2_sf"], p["gs_w2"])
    p.update(h=h, h_q=h_q, h_sf=h_sf, y=y)
    return p


def expert_rows_mx(w1_bits, w2_bits, a_q_mx, a_sc_mx, gs_a, gs_h):
    """The MX variant for one expert's rows: weights prepared as NVFP4 and
    re-encoded; L1 on MX operands -> SwiGLU -> NVFP4 requant -> re-encode ->
    L2 on MX operands (a_q_mx / a_sc_mx: the rows' MX activations, scales
    one per 32).  Also returns the NVFP4 requant (h_q_nv, h_sf_nv) before the
    re-encoding."""
    from oracle import mx as X
    from oracle.layout import deinterleave_cols
    p = O.prepare_expert_weights(w1_bits, w2_bits)
    w1q, w1s = X.nvfp4_to_mx(p["w1_q"], p["w1_sf"])
    w2q, w2s = X.nvfp4_to_mx(p["w2_q"], p["w2_sf"])
    acc = X.mx_matmul(a_q_mx, a_sc_mx, gs_a, w1q, w1s, p["gs_w1"])
    g, u = deinterleave_cols(acc)
    h = (O.silu(g) * u).astype(np.float32)
    codes, h_sf = Q.quantize_blocks(h, np.float32(gs_h))
    h_q_nv = Q.pack_codes(codes)
    h_q, h_sc = X.nvfp4_to_mx(h_q_nv, h_sf)
    y = O.round_to_bf16(X.mx_matmul(h_q, h_sc, np.float32(gs_h), w2q, w2s, p["gs_w2"]))
    return dict(w1_q=w1q, w1_sc=w1s, w2_q=w2q, w2_sc=w2s, h=h, h_q_nv=h_q_nv, h_sf_nv=h_sf,
                h_q=h_q, h_sc=h_sc, y=y)
