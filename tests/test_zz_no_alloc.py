"""moe_prefill_layer_noalloc (the prefill call for callers that cannot
allocate: its intermediates live in the library's fixed device scratch)
against moe_prefill_layer on the same inputs, through the C ABI.

Two contexts share one host pool: A calls moe_prefill_layer, B the
no-allocation variant.  Each case runs two prefill calls in a row per layer
schedule, the second with a smaller chunk, so anything the first call left in
the shared scratch that the second reads without rewriting would show.
Outputs must be bit-identical (the same kernels on the same inputs), and so
must the residency tables and the grouping each call leaves; the mini case is
also checked against the fp64 oracle.  Then a chunk over the scratch limit is
refused with MOE_EINVAL and changes nothing."""
import dataclasses

import numpy as np
import pytest

import workload as W
from oracle import layer as OY
from tests.harness import DeviceRun, OracleRun, d2h, log, rel_err, x_f64

pytestmark = pytest.mark.gpu
TOL = 2e-2


def grouping(B, ctx, E, Tk):
    v = B.moe_prefill_view_get(ctx)
    off = d2h(v.offsets, E + 2, np.int32)
    perm = d2h(v.perm, Tk, np.int32)
    # the order inside an expert is free (LDS atomics): compare the sets
    segs = [np.sort(perm[off[e]:off[e + 1]]) for e in range(E)]
    return d2h(v.counts, E, np.int32), off, np.concatenate(segs), d2h(v.tiles, int(off[E + 1]), np.int32)


def run_case(wl, n_slots, Ts, max_T, with_oracle):
    import torch
    g = DeviceRun(wl, n_slots=n_slots, max_tokens=8, max_prefill_tokens=max_T)
    B = g.B
    ctx_b = None
    try:
        ctx_b = B.moe_create(g.cfg, g.pool, g.pool_bytes)
        o = OracleRun(wl, g.bank, n_slots=n_slots, max_tokens=8) if with_oracle else None
        dev = g.dev
        for call, T in enumerate(Ts):
            ids = torch.empty((T, wl.k), dtype=torch.int32, device=dev)
            w = torch.empty((T, wl.k), dtype=torch.float32, device=dev)
            ya = torch.empty((T, wl.H), dtype=torch.bfloat16, device=dev)
            yb = torch.full((T, wl.H), 7.0, dtype=torch.bfloat16, device=dev)
            for l in range(wl.L):
                lg = np.ascontiguousarray(W.prefill_logits(dataclasses.replace(wl, T=max_T), l)[:T])
                x = W.hidden(dataclasses.replace(wl, T=max_T), call, l)[:T]
                xd = g.to_dev_x(x)
                B.moe_route_topk(g.ctx, torch.from_numpy(lg).to(dev), T, ids, w)
                B.moe_prefill_layer(g.ctx, l, xd, T, ids, w, ya)
                B.moe_prefill_layer_noalloc(ctx_b, l, xd, T, ids, w, yb)
                torch.cuda.synchronize()
                assert torch.equal(ya.view(torch.int16), yb.view(torch.int16)), (call, T, l)
                ga = grouping(B, g.ctx, wl.E, T * wl.k)
                gb = grouping(B, ctx_b, wl.E, T * wl.k)
                for a, b in zip(ga, gb):
                    assert np.array_equal(a, b), (call, T, l)
                va, vb = B.moe_plan_view_get(g.ctx), B.moe_plan_view_get(ctx_b)
                n = va.n_slots
                for name, cnt, dt in (("id2slot", wl.n_ids, np.int32), ("slot2id", n, np.int32),
                                      ("slot_ts", n, np.int64), ("tick", 1, np.int64)):
                    assert np.array_equal(d2h(getattr(va, name), cnt, dt), d2h(getattr(vb, name), cnt, dt)), name
                if o is not None:
                    ids_o, w_o = o.route(lg)
                    ref = OY.moe_layer(x_f64(wl, x), ids_o, w_o, l, wl.E, o.weights)
                    err, _ = rel_err(yb.float().cpu().numpy().astype(np.float64), ref)
                    assert err <= TOL, (call, T, l, err)
            log(f"  call {call}: T={T}, {wl.L} layers, n={n_slots}: no-allocation output, tables and "
                f"grouping bit-identical to moe_prefill_layer")
        return g, ctx_b
    except BaseException:
        if ctx_b:
            B.moe_destroy(ctx_b)
        g.close()
        raise


def close(g, ctx_b):
    g.B.moe_destroy(ctx_b)
    g.close()


@pytest.mark.parametrize("n_slots", [40, 9])  # two full-layer buffers; on-demand passes
def test_noalloc_prefill_mini(n_slots):
    wl = dataclasses.replace(W.DSV4_PREFILL, L=3, E=16, k=4, H=512, I=512, T=333, n_slots=n_slots)
    log(f"no-allocation prefill, mini: L=3 E=16 k=4 H=512 I=512, n={n_slots}")
    close(*run_case(wl, n_slots, [333, 77], 333, with_oracle=True))


def test_noalloc_prefill_deepseek_shape_limit():
    """The DeepSeek-V4-Flash expert shape (E 256, H 4096, I 2048, k 8): the
    largest chunk that fits the scratch (409 tokens), then a smaller one;
    then 410 tokens are refused and leave outputs and tables alone."""
    import torch
    wl = dataclasses.replace(W.DSV4_PREFILL, L=2, T=409, n_slots=512)
    log("no-allocation prefill, DeepSeek shape: L=2 E=256 H=4096 I=2048 k=8, T=409 then 120")
    g, ctx_b = run_case(wl, 512, [409, 120], 410, with_oracle=False)
    try:
        B = g.B
        T = 410
        dev = g.dev
        ids = torch.zeros((T, wl.k), dtype=torch.int32, device=dev)
        w = torch.zeros((T, wl.k), dtype=torch.float32, device=dev)
        x = torch.zeros((T, wl.H), dtype=torch.bfloat16, device=dev)
        y = torch.full((T, wl.H), 3.0, dtype=torch.bfloat16, device=dev)
        tick0 = int(d2h(B.moe_plan_view_get(ctx_b).tick, 1, np.int64)[0])
        with pytest.raises(B.MoertError) as ei:
            B.moe_prefill_layer_noalloc(ctx_b, 0, x, T, ids, w, y)
        assert ei.value.status == -1 and "scratch" in str(ei.value)
        torch.cuda.synchronize()
        assert bool((y == 3.0).all())
        assert int(d2h(B.moe_plan_view_get(ctx_b).tick, 1, np.int64)[0]) == tick0
        log(f"  T={T}: refused ({ei.value}); nothing enqueued")
    finally:
        close(g, ctx_b)
