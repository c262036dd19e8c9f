"""Oracle work for sampled rows of a full-size workload, run in worker
processes (spawned; they import only NumPy and the oracle, never the GPU)."""

import numpy as np

from oracle import moe as O
from oracle import quantize as Q


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
