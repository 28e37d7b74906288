"""Top-k router with renormalized softmax weights (test infrastructure).

The layer's inputs topk_ids / topk_weights are what the last stage of the
NVFP4 MegaMoE Debug Log's "NVFP4 MoE Pipeline" (the routing-weighted scatter
of the L2 rows) consumes. The pages
do not define how they are produced; the reading taken (the plainest one, and
the one the synthetic workloads use) is the usual MoE router on per-token
logits over the E local experts:

1. ids: the k largest logits of the token, in descending order of value; equal
   values are taken in ascending expert order (so the result is unique);
2. weights: the softmax over the k selected logits only (a renormalized
   softmax), w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0), l_0 the largest.

Written here with pure NumPy: a stable sort on the negated logits for step 1,
float64 arithmetic for step 2 (exact selection, weights with float64 rounding
only).

Parity pins (tests/test_oracle_ext.py): brute force over all k-subsets on tiny
inputs (the chosen set maximizes the sum of logits, lexicographically smallest
ids among equal sums when there are ties); k = 1 gives weight 1 exactly; equal
logits give weights 1/k and ids 0..k-1; shift invariance of the weights; the
library routine torch.topk + torch.softmax on distinct logits.
"""
import numpy as np


def route_topk(logits, k):
    """logits (T, E) float32 -> (ids int32 (T, k), weights float64 (T, k))."""
    lg = np.asarray(logits, dtype=np.float32)
    if lg.ndim != 2 or not 1 <= k <= lg.shape[1]:
        raise ValueError("logits must be (T, E) with 1 <= k <= E")
    # stable sort of -l: descending values, ascending index among equal values
    order = np.argsort(-lg.astype(np.float64), axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(lg, order, axis=1).astype(np.float64)
    ex = np.exp(sel - sel[:, :1])
    w = ex / ex.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w


__all__ = ["route_topk"]
