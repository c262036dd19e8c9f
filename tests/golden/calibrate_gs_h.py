"""Calibrate gs_h, the pre-computed global scale of the requantised L2 input.

The fused SwiGLU epilogue cannot see a per-call amax of h, so the method uses
the quantiser's pre-computed-scale mode for h (README "NVFP4 MegaMoE Kernel",
"What We Have", bridge layer: a quantiser with a pre-computed global scale).
For each MoE workload this script draws the workload's inputs on the CPU,
runs the CPU oracle's L1 + SwiGLU on a row sample (the rows of the first
experts, at most ROWS rows), and sets

    gs_h = 2 ** floor(log2(2688 / amax(h_sample))) / 2

(a power of two, so a_s = amax * gs_h is exact; one binade of headroom for
rows outside the sample).  Output: tests/golden/gs_h.json.  Calls only the
oracle and the input generators.

    python tests/golden/calibrate_gs_h.py
"""

import json
import math
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from nvfp4_block_scaled_04_amd import inputs as I  # noqa: E402
from oracle import moe as O, quantize as Q, route as R  # noqa: E402

ROWS = 512
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gs_h.json")


def calibrate(w):
    x = I.bf16_to_bits(I.make_x(w, "cpu"))
    ids, _ = I.make_routing(w)
    offsets, perm, _, _ = R.route(ids, w.E)
    gs_a = Q.global_scale(x)
    amax, rows = 0.0, 0
    for e in range(w.E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        hi = min(hi, lo + ROWS - rows)
        w1, w2 = (I.bf16_to_bits(t) for t in I.make_expert_weights(w, e, "cpu"))
        p = O.prepare_expert_weights(w1, w2)
        tok = perm[lo:hi] // w.k
        codes, a_sf = Q.quantize_blocks(x[tok], gs_a)
        h = O.l1_swiglu(Q.pack_codes(codes), a_sf, gs_a, p["w1_q"], p["w1_sf"], p["gs_w1"])
        amax = max(amax, float(np.abs(h).max()))
        rows += hi - lo
        if rows >= ROWS:
            break
    gs_h = 2.0 ** math.floor(math.log2(2688.0 / amax)) / 2
    return {"gs_h": gs_h, "sample_rows": rows, "sample_amax": amax}


def main():
    res = {}
    for name in ("tiny", "decode", "prefill", "skewed", "moe384"):
        res[name] = calibrate(I.WORKLOADS[name])
        print(name, res[name], flush=True)
    res["_recipe"] = ("gs_h = 2**floor(log2(2688/amax(h over a row sample)))/2; sample = rows of the "
                      "first experts (<= %d rows), inputs drawn on the CPU, oracle L1 + SwiGLU" % ROWS)
    with open(OUT, "w") as f:
        json.dump(res, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main()
