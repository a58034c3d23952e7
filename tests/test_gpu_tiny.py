"""GPU parity on the tiny fp32 workload (2 layers, 8 experts, top-2, H=64,
I=128, 6 slots, 25/50 GB/s, 16 steps): route, plan (bit-exact on every call),
fills (slot bytes equal host banks), outputs within 1e-4 x RMS of the fp64
oracle, in all three miss modes."""
import numpy as np
import pytest

import workload as W
from tests.harness import DeviceRun, OracleRun, compare_plan, log, rel_err, x_f64

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_tiny_end_to_end(mode):
    wl = W.TINY
    log(f"tiny mode={mode}")
    g = DeviceRun(wl, mode=mode)
    try:
        o = OracleRun(wl, g.bank, mode=mode)
        logits = W.router_logits(wl)
        worst = 0.0
        for s in range(wl.steps):
            for l in range(wl.L):
                x = W.hidden(wl, s, l)
                ids_g, w_g = g.decode_call(l, logits[s, l], x)
                ids_o, w_o = o.route(logits[s, l])
                assert np.array_equal(ids_g, ids_o), (s, l)
                assert np.allclose(w_g, w_o, rtol=2e-6, atol=1e-7)
                op = o.plan(l, ids_o)
                compare_plan(g.plan_view(wl.T), op, wl.T)
                i2s, s2i, ts, tick = g.tables()
                assert i2s == o.st.id2slot and s2i == o.st.slot2id
                assert ts == o.st.slot_ts and tick == o.st.tick
                for (u, sl, old) in op.fills:
                    assert np.array_equal(g.slot_bytes(sl), g.bank(u))
                y_ref = o.output(l, x_f64(wl, x), ids_o, w_o)
                err, rms = rel_err(g.y_f64(), y_ref)
                worst = max(worst, err)
                assert err <= TOL_F32, (s, l, err)
        log(f"tiny mode={mode}: worst max|dy|/rms = {worst:.3e}")
    finally:
        g.close()


def test_prefill_refusals():
    """The grouped GEMM takes MXFP4 experts with bf16 activations
    (MOE_EUNSUPPORTED otherwise); a pool too small for the full-layer buffers
    falls back to on-demand loading, and only an empty pool is refused
    (MOE_ENOSPC)."""
    import dataclasses

    import torch
    import routed_expert_execution_moe_amd as B

    def call(wl):
        g = DeviceRun(wl, max_prefill_tokens=16)
        try:
            dt = torch.float32 if wl.act_dtype == "f32" else torch.bfloat16
            x = torch.zeros((4, wl.H), dtype=dt, device="cuda")
            ids = torch.zeros((4, wl.k), dtype=torch.int32, device="cuda")
            w = torch.zeros((4, wl.k), dtype=torch.float32, device="cuda")
            y = torch.zeros((4, wl.H), dtype=dt, device="cuda")
            with pytest.raises(B.MoertError) as e:
                B.moe_prefill_layer(g.ctx, 0, x, 4, ids, w, y)
            return e.value.status
        finally:
            g.close()

    assert call(W.TINY) == -7
    empty = dataclasses.replace(W.DSV4_PREFILL, L=2, E=16, k=2, H=512, I=512, T=16, n_slots=0)
    assert call(empty) == -3


def test_call_order_enforced():
    import torch
    import routed_expert_execution_moe_amd as B
    wl = W.TINY
    g = DeviceRun(wl)
    try:
        x = torch.zeros((1, wl.H), dtype=torch.float32, device="cuda")
        w = torch.zeros((1, wl.k), dtype=torch.float32, device="cuda")
        with pytest.raises(B.MoertError):
            B.moe_expert_ffn(g.ctx, 0, x, 1)
        with pytest.raises(B.MoertError):
            B.moe_merge(g.ctx, w, 1, g.y)
        with pytest.raises(B.MoertError):
            B.moe_cache_plan(g.ctx, 5, g.ids, 1, x)
    finally:
        g.close()
