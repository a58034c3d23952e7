"""Pins of the MoE-layer output (CPU only): the sparse sum equals the dense
all-experts sum, the grouped prefill evaluation equals the per-token one, and
the merge of GPU/host rows is placement-independent."""
import numpy as np
import pytest

import workload as W
from oracle import expert as X, layer as Y, plan as P
from oracle.route import route_topk


def _weights_of(wl):
    cache = {}

    def f(u):
        if u not in cache:
            cache[u] = X.expert_weights(W.bank(wl, u), wl.w_dtype, wl.H, wl.I)
        return cache[u]
    return f


@pytest.mark.parametrize("w_dtype", ["f32", "bf16", "mxfp4"])
def test_sparse_equals_dense(w_dtype):
    wl = W.Workload(name="t", L=3, E=8, k=3, H=64, I=32, w_dtype=w_dtype, act_dtype="f32",
                    n_slots=4, bw_pcie_mbps=1, bw_host_mbps=2, steps=1, T=5, seed=31)
    wf = _weights_of(wl)
    rng = np.random.default_rng(1)
    for layer in range(wl.L):
        x = rng.normal(size=(wl.T, wl.H))
        lg = rng.normal(size=(wl.T, wl.E)).astype(np.float32)
        ids, w = route_topk(lg, wl.k)
        ys = Y.moe_layer(x, ids, w, layer, wl.E, wf)
        yd = Y.dense_layer(x, ids, w, layer, wl.E, wf)
        scale = np.abs(yd).max()
        assert np.abs(ys - yd).max() <= 1e-12 * scale


def test_tiny_workload_dense_invariant():
    wl = W.TINY
    wf = _weights_of(wl)
    lg = W.router_logits(wl)
    for s in range(wl.steps):
        for layer in range(wl.L):
            x = W.hidden(wl, s, layer).astype(np.float64)
            ids, w = route_topk(lg[s, layer], wl.k)
            ys = Y.moe_layer(x, ids, w, layer, wl.E, wf)
            yd = Y.dense_layer(x, ids, w, layer, wl.E, wf)
            assert np.abs(ys - yd).max() <= 1e-12 * np.abs(yd).max()


def test_prefill_grouped_equals_per_token():
    wl = W.Workload(name="t", L=2, E=16, k=4, H=64, I=32, w_dtype="mxfp4", act_dtype="bf16",
                    n_slots=32, bw_pcie_mbps=1, bw_host_mbps=2, steps=1, T=97, seed=4,
                    zipf_s=1.0, prefill=True)
    wf = _weights_of(wl)
    for layer in range(wl.L):
        x = W.bf16_bits_to_f32(W.hidden(wl, 0, layer)).astype(np.float64)
        ids, w = route_topk(W.prefill_logits(wl, layer), wl.k)
        yg, Pg, counts = Y.prefill_grouped(x, ids, w, layer, wl.E, wf)
        yt = Y.moe_layer(x, ids, w, layer, wl.E, wf)
        assert counts.sum() == wl.T * wl.k
        assert np.abs(yg - yt).max() <= 1e-12 * np.abs(yt).max()
        assert np.abs(Pg - Y.expert_rows(x, ids, layer, wl.E, wf)).max() == 0.0


def test_group_permutation_is_stable():
    ids = np.array([[3, 1], [1, 0], [3, 2], [0, 1]])
    counts, off, perm = Y.group_by_expert(ids, 4)
    assert counts.tolist() == [2, 3, 1, 2]
    assert perm.tolist() == [3, 6, 1, 2, 7, 5, 0, 4]


def test_merge_placement_independent():
    """Any CPU/GPU split of the same exact rows gives the same output."""
    rng = np.random.default_rng(3)
    T, k, H = 6, 4, 16
    Pr = rng.normal(size=(T, k, H))
    w = rng.random(size=(T, k))
    y0 = Y.merge(Pr, w)
    junk = rng.normal(size=(T, k, H))
    for trial in range(10):
        sm = rng.integers(-1, 5, size=(T, k))
        Pg = np.where((sm >= 0)[..., None], Pr, junk)
        Pc = np.where((sm < 0)[..., None], Pr, junk)
        assert np.array_equal(Y.merge_placed(Pg, Pc, sm, w), y0)


def test_plan_then_layer_tiny_end_to_end():
    """The tiny workload driven through plan + placement-split rows: merged
    output equals the sparse definition whatever the plan decided."""
    wl = W.TINY
    wf = _weights_of(wl)
    lg = W.router_logits(wl)
    st = P.Residency(wl.n_ids, wl.n_slots)
    K = P.victim_bound(wl.T, wl.k, wl.E, wl.n_slots)
    cpu_rows = 0
    for s in range(wl.steps):
        for layer in range(wl.L):
            x = W.hidden(wl, s, layer).astype(np.float64)
            ids, w = route_topk(lg[s, layer], wl.k)
            pl = P.plan(st, layer, ids.tolist(), wl.E, K, wl.bw_pcie_mbps, wl.bw_host_mbps)
            rows = Y.expert_rows(x, ids, layer, wl.E, wf)
            y = Y.merge_placed(rows, rows, pl.slot_map, w)
            cpu_rows += sum(v < 0 for r in pl.slot_map for v in r)
            assert np.array_equal(y, Y.moe_layer(x, ids, w, layer, wl.E, wf))
    assert cpu_rows > 0
