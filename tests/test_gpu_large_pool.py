"""GPU parity of the control kernel on large slot pools and across 2^32 LRU
ticks.

The control kernel holds the slot table in registers of one 1,024-thread
workgroup, more slots per thread as the pool grows (the variants for more
than 4,096, 8,192 and 16,384 slots).  Small fp32 experts (H = I = 64) let a
pool of up to 20,000 slots fill quickly: 160 layers of 128 experts, 32 tokens
per call, offload mode (every miss fills), the pool grown 5,000 -> 12,000 ->
20,000 slots between steps.  Every plan (victim list of 128 slots included)
and the tables are compared bit for bit with the oracle.

Then the LRU clock is moved close to 2^32: the same constant is added to the
tick and to every occupied slot's tick, on the device (a table write) and in
the oracle's state, which leaves the oracle's LRU order unchanged.  The next
calls cross 2^32 in hybrid mode (q = m / 2, host work every call) and must
stay bit-exact."""
import dataclasses

import numpy as np
import pytest

import workload as W
from oracle import plan as OP
from tests.harness import DeviceRun, OracleRun, compare_plan, d2h, h2d, log, rel_err, x_f64

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(600)
def test_large_pools_and_tick_crossing_2_32():
    wl = dataclasses.replace(W.TINY, name="tiny-f32-large-pool", L=160, E=128, k=8, H=64, I=64,
                             n_slots=5000, T=32, steps=6, seed=1777, router="zipf", zipf_s=0.5,
                             beta=0.0, bw_pcie_mbps=1000, bw_host_mbps=2000)
    schedule = {1: 12_000, 2: 20_000}
    log("large pools: 160 layers x 128 experts (f32, H=I=64), T=32, slots 5000 -> 12000 -> 20000")
    g = DeviceRun(wl, mode=OP.OFFLOAD, n_slots=wl.n_slots, max_slots=20_000, max_tokens=wl.T)
    try:
        o = OracleRun(wl, g.bank, mode=OP.OFFLOAD, n_slots=wl.n_slots, max_tokens=wl.T)
        logits = W.router_logits(wl)
        calls = worst = 0
        evictions = 0
        for s in range(wl.steps):
            if s in schedule:
                g.B.moe_cache_resize(g.ctx, schedule[s], 60_000)
                o.resize(schedule[s])
            if s == 4:
                # move the clock to just below 2^32 on both sides, then hybrid
                v = g.B.moe_plan_view_get(g.ctx)
                n = v.n_slots
                ts = d2h(v.slot_ts, n, np.int64)
                tick = int(d2h(v.tick, 1, np.int64)[0])
                assert tick == o.st.tick
                off = 2**32 - tick - 80
                ts[ts >= 0] += off
                h2d(v.slot_ts, ts)
                h2d(v.tick, np.array([tick + off], np.int64))
                o.st.slot_ts = [t + off if t >= 0 else t for t in o.st.slot_ts]
                o.st.tick += off
                g.B.moe_set_split(g.ctx, wl.bw_pcie_mbps, wl.bw_host_mbps, OP.HYBRID)
                o.mode = OP.HYBRID
                log(f"  clock moved from {tick} to {tick + off} (2^32 - 80); hybrid from here")
            for l in range(wl.L):
                x = W.hidden(wl, s, l)
                ids_g, w_g = g.decode_call(l, logits[s, l], x)
                ids_o, w_o = o.route(logits[s, l])
                assert np.array_equal(ids_g, ids_o), (s, l)
                op = o.plan(l, ids_o)
                compare_plan(g.plan_view(wl.T), op, wl.T)
                evictions += sum(1 for f in op.fills if f[2] >= 0)
                calls += 1
                if calls % 16 == 0:
                    err, _ = rel_err(g.y_f64(), o.output(l, x_f64(wl, x), ids_o, w_o))
                    worst = max(worst, err)
                    assert err <= 1e-4, (s, l, err)
                    for (u, sl, _) in op.fills[:4]:
                        assert np.array_equal(g.slot_bytes(sl), g.bank(u)), (s, l, u)
            i2s, s2i, ts, tick = g.tables()
            assert i2s == o.st.id2slot and s2i == o.st.slot2id and ts == o.st.slot_ts, s
            assert tick == o.st.tick, s
            occ = sum(1 for u in s2i if u >= 0)
            log(f"  step {s}: {len(s2i)} slots, {occ} occupied, tick {tick}, evictions so far "
                f"{evictions}, worst rel err {worst:.2e}")
        assert o.st.tick > 2**32 and evictions > 0
    finally:
        g.close()


@pytest.mark.timeout(600)
def test_maximum_shapes():
    """The largest shapes the configuration accepts, on small fp32 experts
    (H = I = 64): 1,024 experts per layer, top-32, 64 tokens per call (2,048
    routed pairs, the most the plan buffers take at this k is 4,096), so K =
    1,024 victims: the radix select and the rank sort at their largest.  Every
    plan and table bit-exact, outputs within tolerance."""
    wl = dataclasses.replace(W.TINY, name="tiny-f32-max-shapes", L=3, E=1024, k=32, H=64, I=64,
                             n_slots=2500, T=64, steps=4, seed=1779, router="zipf", zipf_s=0.8,
                             beta=0.0, bw_pcie_mbps=1000, bw_host_mbps=2000)
    log("maximum shapes: E=1024, k=32, T=64 (2,048 pairs), 2,500 slots")
    g = DeviceRun(wl, mode=OP.HYBRID, n_slots=wl.n_slots, max_tokens=wl.T)
    try:
        o = OracleRun(wl, g.bank, mode=OP.HYBRID, n_slots=wl.n_slots, max_tokens=wl.T)
        assert o.K == 1024
        logits = W.router_logits(wl)
        worst = 0.0
        for s in range(wl.steps):
            for l in range(wl.L):
                x = W.hidden(wl, s, l)
                ids_g, w_g = g.decode_call(l, logits[s, l], x)
                ids_o, w_o = o.route(logits[s, l])
                assert np.array_equal(ids_g, ids_o), (s, l)
                op = o.plan(l, ids_o)
                compare_plan(g.plan_view(wl.T), op, wl.T)
                err, _ = rel_err(g.y_f64(), o.output(l, x_f64(wl, x), ids_o, w_o))
                worst = max(worst, err)
                assert err <= 1e-4, (s, l, err)
            i2s, s2i, ts, tick = g.tables()
            assert i2s == o.st.id2slot and s2i == o.st.slot2id and ts == o.st.slot_ts, s
            log(f"  step {s}: {len(op.uniq)} unique, {len(op.hits)} hits, q {op.q}, "
                f"worst rel err {worst:.2e}")
    finally:
        g.close()
