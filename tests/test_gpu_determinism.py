"""Bitwise determinism of the hot path on the GPU.

The pages claim the GPU and host partial sums merge exactly (snackonai, "What
It Actually Does"): the result must not depend on timing.  Here the same
decode steps run on two fresh contexts, and every layer call's output, plan
and tables must be bit-identical between the two (the host branch races the
GPU path differently on each run; the fill and FFN kernels run on different
workgroup schedules).  The same prefill chunk run twice must give a
bit-identical output although the order of pairs inside an expert (LDS
atomics in the grouping scatter) may differ from run to run."""
import dataclasses

import numpy as np
import pytest

import workload as W
from tests.harness import DeviceRun, log

pytestmark = pytest.mark.gpu


def record_decode(wl, resize=None):
    """Every call's output bits, plan view and tables, in call order."""
    resize = resize or {}
    g = DeviceRun(wl)
    out = []
    try:
        logits = W.router_logits(wl)
        for s in range(wl.steps):
            if s in resize:
                g.B.moe_cache_resize(g.ctx, resize[s], 60_000)
            for l in range(wl.L):
                x = W.hidden(wl, s, l)
                g.decode_call(l, logits[s, l], x)
                y = g.y[:wl.T].view(g.torch.int16 if wl.act_dtype == "bf16" else g.torch.int32)
                out.append((y.cpu().numpy().copy(), g.plan_view(wl.T), g.tables()))
        return out
    finally:
        g.close()


def compare_runs(a, b, what):
    assert len(a) == len(b)
    for i, ((ya, pa, ta), (yb, pb, tb)) in enumerate(zip(a, b)):
        assert np.array_equal(ya, yb), (what, "output", i)
        assert pa == pb, (what, "plan", i)
        assert ta == tb, (what, "tables", i)


@pytest.mark.parametrize("case", ["bf16_hybrid", "streams_resize"])
def test_decode_runs_bit_identical(case):
    if case == "bf16_hybrid":
        wl = dataclasses.replace(W.QWEN_BF16, L=4, steps=16, n_slots=120)
        resize = None
    else:
        wl = dataclasses.replace(W.QWEN_ELASTIC, L=3, steps=16, n_slots=141,
                                 resize={5: 57, 10: 115})
        resize = wl.resize
    a = record_decode(wl, resize)
    b = record_decode(wl, resize)
    compare_runs(a, b, case)
    cpu_calls = sum(1 for _, p, _ in a if p["counts"]["n_cpu"] > 0)
    fills = sum(p["counts"]["q"] for _, p, _ in a)
    log(f"  {case}: {len(a)} layer calls bit-identical across two contexts "
        f"({cpu_calls} with host work, {fills} fills)")
    assert cpu_calls > 0 and fills > 0


def test_prefill_chunk_bit_identical():
    import torch
    wl = dataclasses.replace(W.DSV4_PREFILL, L=3, E=16, k=4, H=512, I=512, T=777, n_slots=40)
    g = DeviceRun(wl, n_slots=wl.n_slots, max_tokens=8, max_prefill_tokens=wl.T)
    try:
        dev = g.dev
        ids = torch.empty((wl.T, wl.k), dtype=torch.int32, device=dev)
        w = torch.empty((wl.T, wl.k), dtype=torch.float32, device=dev)
        y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=dev)
        runs = []
        for rep in range(3):
            ys = []
            for l in range(wl.L):
                lg = W.prefill_logits(wl, l)
                g.B.moe_route_topk(g.ctx, torch.from_numpy(lg).to(dev), wl.T, ids, w)
                g.B.moe_prefill_layer(g.ctx, l, g.to_dev_x(W.hidden(wl, 0, l)), wl.T, ids, w, y)
                torch.cuda.synchronize()
                ys.append(y.view(torch.int16).cpu().numpy().copy())
            runs.append(ys)
        for rep in (1, 2):
            for l in range(wl.L):
                assert np.array_equal(runs[0][l], runs[rep][l]), (rep, l)
        log(f"  prefill chunk (T={wl.T}, {wl.L} layers) three times: bit-identical outputs")
    finally:
        g.close()
