"""Expert offsets and the expert-order permutation of routed token rows.

README ("NVFP4 MegaMoE Kernel"), section "Correctness Bugs Fixed", bug 5:
experts are counted with a histogram (``torch.bincount``) instead of an
O(n x E) comparison mask.  The grouped GEMM of section "What We Have"
consumes rows grouped by expert; README "Key Lessons" 4: quantise the compact
rows, then place them.

Readings: the flat index of routed pair (token t, slot j) is f = t*k + j; rows
are ordered by expert and, inside an expert, by increasing f (a stable sort),
with no padding between experts.  Expert ids outside [0, E) are counted as
invalid and placed after all valid rows, in increasing f; they contribute
nothing to the combine.
"""

import numpy as np


def route(topk_ids, E):
    """topk_ids (T, k) int -> (offsets (E+1,), perm (M,), inv_perm (M,),
    invalid_count) with M = T*k, all int32 except the count.

    offsets[e] .. offsets[e+1] are the rows of expert e; perm[d] is the flat
    index f of row d; inv_perm[f] = d.
    """
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    valid = (ids >= 0) & (ids < E)
    counts = np.bincount(ids[valid], minlength=E)[:E]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    key = np.where(valid, ids, E)                 # invalid rows sort last
    perm = np.argsort(key, kind="stable").astype(np.int32)
    inv_perm = np.empty_like(perm)
    inv_perm[perm] = np.arange(perm.size, dtype=np.int32)
    return offsets, perm, inv_perm, int(np.count_nonzero(~valid))
