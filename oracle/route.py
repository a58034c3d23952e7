"""Router top-k (oracle).

The pages leave router design out of scope (snackonai, "The Promise"); the
tiny workload names a softmax router with top-2.  Reading used here:
  * selection on the fp32 logits both sides receive: order experts by
    descending logit, equal logits by ascending expert index, keep the first k;
  * weights: softmax over the k selected logits (renormalised), in fp64.
"""
from __future__ import annotations

import numpy as np


def route_topk(logits: np.ndarray, k: int):
    """logits: float32 [T, E].  Returns (ids int64 [T, k], w float64 [T, k])."""
    lg = np.asarray(logits)
    assert lg.dtype == np.float32 and lg.ndim == 2
    T, E = lg.shape
    assert 1 <= k <= E
    neg = -lg.astype(np.float64)
    idx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((idx, neg), axis=-1)        # primary: -logit, then index
    ids = order[:, :k].astype(np.int64)
    sel = np.take_along_axis(lg.astype(np.float64), ids, axis=-1)
    z = np.exp(sel - sel[:, :1])                   # first column is the max
    w = z / z.sum(axis=-1, keepdims=True)
    return ids, w
