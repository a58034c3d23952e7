"""MoE-layer output, its dense equivalent, the merge and grouped prefill
evaluation (oracle, fp64).

Plain definition (the result the method reaches whatever the placement:
snackonai, "What It Actually Does"; satyajit, "Decode: the one equation"):

    y[t] = sum_j w[t,j] * FFN_{l*E + ids[t,j]}(x[t])

`weights_of(u)` returns the decoded (W_gate, W_up, W_down) of flat id u.
"""
from __future__ import annotations

import numpy as np

from .expert import ffn


def expert_rows(x, ids, layer: int, E: int, weights_of):
    """Partial rows P[t, j] = FFN_{l*E+ids[t,j]}(x[t]), fp64 [T, k, H]."""
    x = np.asarray(x, np.float64)
    ids = np.asarray(ids)
    T, k = ids.shape
    P = np.zeros((T, k, x.shape[1]))
    for e in sorted(set(ids.ravel().tolist())):
        tj = np.argwhere(ids == e)
        rows = ffn(x[tj[:, 0]], weights_of(layer * E + int(e)))
        P[tj[:, 0], tj[:, 1]] = rows
    return P


def merge(P, w):
    """y[t] = sum over ranks j of w[t,j] * P[t,j]."""
    return np.einsum("tj,tjh->th", np.asarray(w, np.float64), np.asarray(P, np.float64))


def moe_layer(x, ids, w, layer: int, E: int, weights_of):
    """Sparse sum over each token's k routed experts."""
    return merge(expert_rows(x, ids, layer, E, weights_of), w)


def dense_layer(x, ids, w, layer: int, E: int, weights_of):
    """Every expert of the layer evaluated on every token, with weight zero
    for experts a token did not select: must equal moe_layer."""
    x = np.asarray(x, np.float64)
    ids = np.asarray(ids)
    T = x.shape[0]
    wfull = np.zeros((T, E))
    for t in range(T):
        for j in range(ids.shape[1]):
            wfull[t, int(ids[t, j])] += float(w[t, j])
    y = np.zeros_like(x)
    for e in range(E):
        y += wfull[:, e:e + 1] * ffn(x, weights_of(layer * E + e))
    return y


def merge_placed(P_gpu, P_cpu, slot_map, w):
    """Merge of GPU and host partial rows: rank j of token t comes from the
    host rows when its slot-map entry is the CPU flag (-1), else from the GPU
    rows; summed over ascending j."""
    sm = np.asarray(slot_map)
    P = np.where((sm >= 0)[..., None], np.asarray(P_gpu, np.float64),
                 np.asarray(P_cpu, np.float64))
    return merge(P, w)


def group_by_expert(ids, E: int):
    """Per-expert token counts and the stable permutation of the T*k routed
    (token, rank) pairs sorted by expert: entry i of `perm` is the flattened
    index t*k + j."""
    flat = np.asarray(ids).reshape(-1)
    counts = np.bincount(flat, minlength=E)
    perm = np.argsort(flat, kind="stable")
    offsets = np.concatenate([[0], np.cumsum(counts)])
    return counts, offsets, perm


def prefill_grouped(x, ids, w, layer: int, E: int, weights_of):
    """Prefill layer evaluated expert by expert on its gathered tokens
    (satyajit, "Prefill: hide the pool behind the wire": every expert of the
    layer is resident).  Returns (y, P, counts)."""
    x = np.asarray(x, np.float64)
    ids = np.asarray(ids)
    T, k = ids.shape
    counts, offsets, perm = group_by_expert(ids, E)
    P = np.zeros((T * k, x.shape[1]))
    for e in range(E):
        sel = perm[offsets[e]:offsets[e + 1]]
        if sel.size == 0:
            continue
        P[sel] = ffn(x[sel // k], weights_of(layer * E + e))
    P = P.reshape(T, k, -1)
    return merge(P, w), P, counts
