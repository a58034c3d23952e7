"""Bandwidth calibration on the GPU: both rates are measured on the context's
expert shape, the measurement leaves the slot pool and the residency tables
as they were, and decode steps run with the measured split (and the backend
the pages' rule picks for it) keep every plan bit-exact against the oracle
given the same two numbers, with outputs within tolerance."""
import dataclasses

import numpy as np
import pytest

import workload as W
from tests.harness import DeviceRun, OracleRun, compare_plan, log, rel_err, x_f64

pytestmark = pytest.mark.gpu


def test_measure_then_decode_with_measured_split():
    wl = dataclasses.replace(W.QWEN_BF16, L=4, steps=8, n_slots=189)
    g = DeviceRun(wl)
    try:
        B = g.B
        logits = W.router_logits(wl)
        o0 = OracleRun(wl, g.bank)
        # two steps with the configured split first, so the cache holds experts
        for s in range(2):
            for l in range(wl.L):
                ids_g, _ = g.decode_call(l, logits[s, l], W.hidden(wl, s, l))
                ids_o, _ = o0.route(logits[s, l])
                assert np.array_equal(ids_g, ids_o)
                compare_plan(g.plan_view(wl.T), o0.plan(l, ids_o), wl.T)
        before = g.tables()
        slots_before = [g.slot_bytes(s)[:4096].copy() for s in (0, 1, 2)]
        bp, bh = B.moe_measure_bandwidth(g.ctx, 8, 3)
        log(f"  measured B_P {bp} MB/s, B_H {bh} MB/s (expert {W.expert_bytes(wl)} B)")
        # PCIe 4/5 x16 and a host DRAM expert kernel: loose physical bounds
        assert 2_000 <= bp <= 80_000, bp
        assert 500 <= bh <= 2_000_000, bh
        assert g.tables() == before
        for s, sb in zip((0, 1, 2), slots_before):
            assert np.array_equal(g.slot_bytes(s)[:4096], sb)
        mode = B.moe_recommend_mode(bp, bh, 2.0)
        B.moe_set_split(g.ctx, bp, bh, mode)
        # the oracle continues from the same state with the same two numbers
        o0.wl = dataclasses.replace(wl, bw_pcie_mbps=bp, bw_host_mbps=bh)
        o0.mode = mode
        worst = 0.0
        for s in range(2, wl.steps):
            for l in range(wl.L):
                x = W.hidden(wl, s, l)
                ids_g, w_g = g.decode_call(l, logits[s, l], x)
                ids_o, w_o = o0.route(logits[s, l])
                assert np.array_equal(ids_g, ids_o), (s, l)
                op = o0.plan(l, ids_o)
                compare_plan(g.plan_view(wl.T), op, wl.T)
                err, _ = rel_err(g.y_f64(), o0.output(l, x_f64(wl, x), ids_o, w_o))
                worst = max(worst, err)
                assert err <= 2e-2, (s, l, err)
        i2s, s2i, ts, tick = g.tables()
        assert i2s == o0.st.id2slot and s2i == o0.st.slot2id and ts == o0.st.slot_ts
        log(f"  mode {'hybrid' if mode == 0 else 'offload'} with the measured split: "
            f"worst rel err {worst:.3e}")
    finally:
        g.close()
