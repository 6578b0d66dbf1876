"""Top-k softmax routing (oracle).

Source: FreeToken PR #676, "Known limits" (a chunk's copies wait on the
router) and gdevenyi's PR #68 commit message (route, then fetch the missing
routed experts, then the slot GEMM): each token is routed to its top-k
experts before any expert is loaded.  The tiny workload defines the weights
as a softmax over the top-k logits, renormalised.

Reading taken where the pages are silent:
  * order: logit descending, ties broken by the lower expert id;
  * weights: softmax over the k selected logits, computed in fp64
    (exp of the difference to the largest selected logit, summed in rank
    order) and rounded once to fp32.  A softmax over all E logits
    renormalised over the top-k is the same quantity in exact arithmetic.

Parity: pinned (brute force over all k-subsets, scipy softmax special case,
k=1 and k=2 closed forms).
"""
import math

import numpy as np


def route_topk_softmax(logits: np.ndarray, k: int):
    """logits float32 [T, E] -> (ids int32 [T, k], weights float32 [T, k])."""
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    for t in range(T):
        row = logits[t]
        # descending by value, ascending id on ties: a stable sort of the
        # negated values keeps equal values in id order
        order = sorted(range(E), key=lambda e: (-float(row[e]), e))[:k]
        ids[t] = order
        top = [float(row[e]) for e in order]          # exact float32 values as fp64
        ex = [math.exp(v - top[0]) for v in top]
        s = 0.0
        for v in ex:                                   # rank order
            s += v
        w[t] = [np.float32(v / s) for v in ex]
    return ids, w
