"""Pins of the q split and the two-branch cost model against the numbers the
pages print and against exact arithmetic (CPU only)."""
import json
import os
import random
from fractions import Fraction

import pytest

from oracle import costmodel, plan as P


def _mbps(gbps):
    return int(round(gbps * 1000))


def load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_worked_q_values(golden_dir):
    g = load(golden_dir, "split_policy.json")
    for row in g["worked_q"]:
        q = P.split_q(row["m"], _mbps(row["bp_gbps"]), _mbps(row["bh_gbps"]), P.HYBRID)
        assert q == row["q"], row
        assert row["m"] - q == row["cpu"]


def test_bw_table_derived_columns(golden_dir):
    """Ratio, backend (hybrid iff B_H > 2 B_P) and CPU share = 1 - B_P/B_H, the
    continuous q*/m complement, for all six machines."""
    g = load(golden_dir, "split_policy.json")
    for row in g["bw_table"]:
        bp, bh = row["bp"], row["bh"]
        assert round(bh / bp, 2) == pytest.approx(row["ratio"], abs=1e-9), row
        hybrid = costmodel.recommend_hybrid(bp, bh, g["threshold"])
        assert ("hybrid" if hybrid else "offload") == row["backend"], row
        share = 1.0 - costmodel.q_star(1.0, bp, bh)
        assert round(100 * share) == row["cpu_share_pct"], row


def test_laptop_cost_model(golden_dir):
    g = load(golden_dir, "laptop_step.json")
    m, bp, bh, q = g["m"], g["bp"], g["bh"], g["q"]
    assert round(costmodel.t_fill(q, bp), 4) == g["t_fill"]
    assert round(costmodel.t_cpu(m, q, bp, bh), 4) == g["t_cpu"]
    assert round(costmodel.exposed(m, q, bp, bh), 4) == g["exposed"]
    assert round(costmodel.all_pcie(m, bp), 4) == g["all_pcie"]
    assert round(costmodel.all_pcie(m, bp) / costmodel.exposed(m, q, bp, bh), 1) == \
        g["all_pcie_vs_exposed"]
    assert round(costmodel.pure_cpu(m, bh), 4) == g["pure_cpu"]
    slower = costmodel.exposed(m, q, bp, bh) / costmodel.pure_cpu(m, bh) - 1.0
    assert round(100 * slower, 1) == g["hybrid_slower_pct"]


def test_prefill_transfer_arithmetic(golden_dir):
    g = load(golden_dir, "prefill_transfer.json")
    s = g["pool_gb"] / g["pcie_gbps"]
    assert round(s, 3) == g["stream_s"]
    lo, hi = g["measured_s"]
    assert lo <= round(s, 2) <= hi


def test_balance_closed_form():
    """At the real-valued q* the two branch times are equal and equal m/B_H
    (S cancels)."""
    rng = random.Random(7)
    for _ in range(200):
        bp = rng.uniform(5, 100)
        bh = bp * rng.uniform(1.05, 6)
        m = rng.randint(1, 64)
        S = rng.uniform(0.1, 20)
        qs = costmodel.q_star(m, bp, bh)
        tf = costmodel.t_fill(qs, bp, S)
        tc = costmodel.t_cpu(m, qs, bp, bh, S)
        assert tf == pytest.approx(tc, rel=1e-12)
        assert tf == pytest.approx(m * S / bh, rel=1e-12)


def test_rne_matches_python_round():
    """Half-to-even on exact rationals, as Python's round() on a Fraction."""
    rng = random.Random(3)
    for _ in range(20000):
        b = rng.randint(1, 10**6)
        a = rng.randint(0, 10**7)
        assert P.rne_div(a, b) == round(Fraction(a, b))
    for a in range(0, 40):
        assert P.rne_div(a, 2) == round(Fraction(a, 2))


def test_q_table_at_half_ratio():
    """B_P/B_H = 1/2: q = clamp(rne(m/2), 1, m); ties at m = 1, 5, 9, 13 go to
    the even neighbour."""
    exp = {1: 1, 2: 1, 3: 2, 4: 2, 5: 2, 6: 3, 7: 4, 8: 4, 9: 4, 10: 5, 11: 6, 12: 6, 13: 6}
    for m, q in exp.items():
        assert P.split_q(m, 25_000, 50_000, P.HYBRID) == q


def test_degenerate_and_modes():
    for m in range(0, 30):
        # B_H -> B_P: every miss is filled
        assert P.split_q(m, 52_700, 52_700, P.HYBRID) == m
        assert P.split_q(m, 1, 10**9, P.OFFLOAD) == m
        assert P.split_q(m, 10**9, 1, P.CPU) == 0
        q = P.split_q(m, 11_800, 47_500, P.HYBRID)
        if m == 0:
            assert q == 0
        else:
            assert 1 <= q <= m
            assert q == min(max(1, round(Fraction(m * 11_800, 47_500))), m)
