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


def router_topk(logits, k):
    """Router: logits (T, E) float32 -> (topk_ids (T, k) int32, topk_w (T, k)
    float64).

    The pages take the expert ids and routing weights as given (the runner
    scatters "with routing weights"); the tiny workload's description fixes
    the router as top-k of the logits followed by a softmax over the k chosen
    ones.  Reading: the k largest logits in decreasing order, equal logits in
    increasing expert id; w_j = exp(l_j - l_max) / sum_i exp(l_i - l_max) over
    the chosen logits, in float64.
    """
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        # descending by value; a stable sort of the negated values keeps
        # equal logits in increasing id
        order = np.argsort(-lg[t].astype(np.float64), kind="stable")[:k]
        sel = lg[t, order].astype(np.float64)
        ex = np.exp(sel - sel[0])
        ids[t] = order
        w[t] = ex / ex.sum()
    return ids, w
