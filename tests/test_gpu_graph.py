"""GPU parity of whole decode steps replayed from a captured HIP graph.

The decode calls enqueue only kernels, and every per-call value they depend
on (tick, plan count used as the host branch's sequence number, counts, slot
lists) lives on the device, so one step of all layers (route, control kernel,
fill, expert FFN, merge per layer) can be captured once and replayed with new
inputs copied into the captured buffers.  Each replay is checked against the
oracle stepped through the same calls: residency tables and the last layer's
plan bit-exact, router ids exact, every layer's output within the dtype's
tolerance.  Eager steps on the same context are interleaved with the replays
(the plan count must stay consistent between the two), and the host does its
own copies and synchronisations between replays."""
import dataclasses

import numpy as np
import pytest

import workload as W
from tests.harness import DeviceRun, OracleRun, compare_plan, log, rel_err, x_f64

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "mxfp4": 2e-2}


def _graph_steps(wl, eager_steps):
    import torch
    g = DeviceRun(wl)
    try:
        B = g.B
        o = OracleRun(wl, g.bank)
        logits = W.router_logits(wl)
        L, T, k = wl.L, wl.T, wl.k
        # captured buffers: inputs are copied in before every replay
        lg_s = torch.empty((L, T, wl.E), dtype=torch.float32, device=g.dev)
        x_s = torch.empty((L, T, wl.H), dtype=g.act, device=g.dev)
        ids_s = torch.empty((L, T, k), dtype=torch.int32, device=g.dev)
        w_s = torch.empty((L, T, k), dtype=torch.float32, device=g.dev)
        y_s = torch.empty((L, T, wl.H), dtype=g.act, device=g.dev)

        def layer_calls():
            for l in range(L):
                B.moe_route_topk(g.ctx, lg_s[l], T, ids_s[l], w_s[l])
                B.moe_cache_plan(g.ctx, l, ids_s[l], T, x_s[l])
                B.moe_expert_ffn(g.ctx, l, x_s[l], T)
                B.moe_merge(g.ctx, w_s[l], T, y_s[l])

        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            layer_calls()
        torch.cuda.synchronize()

        worst, replays = 0.0, 0
        for s in range(wl.steps):
            xs = [W.hidden(wl, s, l) for l in range(L)]
            lg_s.copy_(torch.from_numpy(np.ascontiguousarray(logits[s])).to(g.dev))
            x_s.copy_(torch.stack([g.to_dev_x(x) for x in xs]))
            torch.cuda.synchronize()
            eager = s in eager_steps
            if eager:
                layer_calls()
            else:
                graph.replay()
                replays += 1
            torch.cuda.synchronize()
            ids_all = ids_s.cpu().numpy()
            w_all = w_s.cpu().numpy().astype(np.float64)
            y_all = y_s.float().cpu().numpy().astype(np.float64)
            for l in range(L):
                ids_o, w_o = o.route(logits[s, l])
                assert np.array_equal(ids_all[l], ids_o), (s, l)
                assert np.allclose(w_all[l], w_o, rtol=2e-6, atol=1e-7), (s, l)
                op = o.plan(l, ids_o)
                y_ref = o.output(l, x_f64(wl, xs[l]), ids_o, w_o)
                err, _ = rel_err(y_all[l], y_ref)
                worst = max(worst, err)
                assert err <= TOL[wl.w_dtype], (s, l, err, "eager" if eager else "replay")
            compare_plan(g.plan_view(T), op, T)  # the step's last layer
            i2s, s2i, ts, tick = g.tables()
            assert i2s == o.st.id2slot and s2i == o.st.slot2id, s
            assert ts == o.st.slot_ts and tick == o.st.tick, s
            log(f"  step {s} ({'eager' if eager else 'replay'}): worst rel err {worst:.3e}")
        st = B.moe_ctx_stats(g.ctx)
        assert st.plans == wl.steps * L
        return worst, replays
    finally:
        g.close()


def test_graph_replay_bf16():
    """Qwen-shaped bf16 experts, 4 layers, 189 slots: hits, fills and host
    work in the replayed steps."""
    wl = dataclasses.replace(W.QWEN_BF16, L=4, steps=10, n_slots=189)
    worst, replays = _graph_steps(wl, eager_steps={0, 4})
    assert replays == 8
    log(f"bf16 graph replay: worst rel err {worst:.3e} over {replays} replays")


def test_graph_replay_tiny_f32():
    """The small fp32 workload (2 layers, 8 experts, 6 slots) at fp32 tolerance."""
    worst, replays = _graph_steps(W.TINY, eager_steps={1, 2, 9})
    assert replays == W.TINY.steps - 3
    log(f"fp32 graph replay: worst rel err {worst:.3e} over {replays} replays")
