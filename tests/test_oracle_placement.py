"""Pins of the locality statements (CPU only): routing-blind placement misses
at 1 - capacity, a whole-layer split misses exactly the unplaced layers'
share, and the global LRU misses less than either at every capacity short of
the full pool, on the synthetic Zipf workload with step-to-step reuse."""
import json
import math
import os

import numpy as np
import pytest

import workload as W
from oracle import placement as S, plan as P
from oracle.route import route_topk

WL = W.Workload(name="locality", L=8, E=64, k=4, H=8, I=8, w_dtype="bf16", act_dtype="bf16",
                n_slots=0, bw_pcie_mbps=1, bw_host_mbps=1, steps=200, T=1, seed=2024,
                zipf_s=1.1, beta=1.0)


@pytest.fixture(scope="module")
def calls():
    lg = W.decode_logits(WL)
    out = []
    for s in range(WL.steps):
        for l in range(WL.L):
            ids, _ = route_topk(lg[s, l], WL.k)
            out.append((l, ids))
    return out


def lru_miss_rate(calls, n, warm=0):
    """Miss rate of the global LRU (offload: every miss admitted) over
    calls[warm:], after running calls[:warm] to warm it."""
    st = P.Residency(WL.n_ids, n)
    K = P.victim_bound(WL.T, WL.k, WL.E, n)
    miss = acc = 0
    for i, (l, ids) in enumerate(calls):
        pl = P.plan(st, l, ids.tolist(), WL.E, K, 1, 1, P.OFFLOAD)
        if i >= warm:
            miss += len(pl.misses)
            acc += len(pl.uniq)
    return miss / acc


def uniq_calls(calls):
    return [(l, sorted({l * WL.E + int(e) for e in ids.ravel()})) for l, ids in calls]


def test_blind_placement_misses_one_minus_capacity(calls, golden_dir):
    with open(os.path.join(golden_dir, "locality.json")) as f:
        g = json.load(f)
    uc = uniq_calls(calls)
    N = WL.n_ids
    for row in g["rows"]:
        c = row["capacity"]
        rates = []
        for r in range(60):
            u = W.uniform(99, 7, r, int(c * 1000), N)
            res = S.random_set(N, c, u)
            m, a = S.static_misses(uc, res)
            rates.append(m / a)
        expect = 1.0 - math.floor(c * N) / N
        se = np.std(rates, ddof=1) / math.sqrt(len(rates))
        assert abs(np.mean(rates) - expect) <= 4 * se + 1e-12, (c, np.mean(rates), expect)
        # the pages' own arithmetic: 1 - c predicts the routing-blind rate
        assert round(1 - c, 2) == row["predicted_blind_miss"]


def test_whole_layer_split_exact(calls):
    uc = uniq_calls(calls)
    for c in (0.11, 0.37, 0.5, 0.9):
        res = S.whole_layers(WL.L, WL.E, c)
        n_layers = len(res) // WL.E
        m, a = S.static_misses(uc, res)
        assert m / a == pytest.approx((WL.L - n_layers) / WL.L, abs=1e-15)


def test_lru_beats_static_below_full_pool(calls):
    uc = uniq_calls(calls)
    N = WL.n_ids
    # Capacities at least one decode step's working set (L * k ids): below
    # that a recency policy thrashes on the cyclic layer order.
    # Static placements are made at load time, so the LRU is compared on the
    # second half of the trace after warming on the first half.
    warm = len(calls) // 2
    for c in (0.11, 0.2, 0.37, 0.5, 0.75, 0.95):
        n = math.floor(c * N)
        assert n >= WL.L * WL.k
        lru = lru_miss_rate(calls, n, warm)
        res = S.random_set(N, c, W.uniform(5, 5, 5, int(c * 100), N))
        blind = S.static_misses(uc[warm:], res)
        layers = S.static_misses(uc[warm:], S.whole_layers(WL.L, WL.E, c))
        assert lru < blind[0] / blind[1], c
        assert lru < layers[0] / layers[1], c
    # the full pool: only compulsory misses remain
    distinct = len({u for _, uq in uc for u in uq})
    acc = sum(len(uq) for _, uq in uc)
    assert lru_miss_rate(calls, N) == pytest.approx(distinct / acc)
