"""GPU parity of the prefill path: full-layer buffers streamed by the copy
stream, grouped MFMA GEMM over uneven per-expert token counts, merge.

Mid-size: every token of every layer against the fp64 oracle, ragged T
(not a multiple of the 128-row tile), tables after every layer against the
oracle's buffer admission, the GPU's grouping of pairs by expert against the
oracle's, buffer bytes against the host banks, and a decode call that follows
(what survives prefill seeds decode).  Full size (8 layers, 8,192 tokens, 256
experts, H 4096, I 2048): every token of the first layer and 256 sampled
tokens of each other layer against the oracle, the grouping, tables and
buffer bytes of every layer, a repeated layer bit-identical, then the same
chunk through the on-demand fallback after shrinking the pool, bit-identical
to the two-buffer outputs.
Tolerance: max |y - y_oracle| <= 2e-2 x RMS(y_oracle) per token."""
import dataclasses

import numpy as np
import pytest

import workload as W
from oracle import layer as OY, plan as OP
from tests.harness import (DeviceRun, OracleRun, bf16_round_err, check_grouping, compare_plan, log,
                           rel_err, x_f64)

pytestmark = pytest.mark.gpu
TOL = 2e-2


def run_prefill(wl, sample_tokens=None, check_bytes=True, decode_after=False, buffers=2):
    """buffers x E > n_slots runs the on-demand fallback (checked against the
    oracle's on-demand admission, pass by pass through the final tables)."""
    import torch
    g = DeviceRun(wl, n_slots=wl.n_slots, max_tokens=8, max_prefill_tokens=wl.T)
    try:
        if buffers != 2:
            g.B.moe_prefill_set_buffers(g.ctx, buffers)
        o = OracleRun(wl, g.bank, n_slots=wl.n_slots, max_tokens=8)
        dev = g.dev
        ids = torch.empty((wl.T, wl.k), dtype=torch.int32, device=dev)
        w = torch.empty((wl.T, wl.k), dtype=torch.float32, device=dev)
        y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=dev)
        worst = 0.0
        rng = np.random.default_rng(7)
        for l in range(wl.L):
            lg = W.prefill_logits(wl, l)
            x = W.hidden(wl, 0, l)
            xd = g.to_dev_x(x)
            g.B.moe_route_topk(g.ctx, torch.from_numpy(lg).to(dev), wl.T, ids, w)
            g.B.moe_prefill_layer(g.ctx, l, xd, wl.T, ids, w, y)
            torch.cuda.synchronize()
            ids_o, w_o = o.route(lg)
            assert np.array_equal(ids.cpu().numpy(), ids_o), l
            on_demand = wl.n_slots < buffers * wl.E
            if on_demand:
                passes = OP.prefill_on_demand(o.st, l, ids_o.ravel(), wl.E)
            else:
                b = OP.prefill_admit(o.st, l, wl.E, buffers)
            i2s, s2i, ts, tick = g.tables()
            assert i2s == o.st.id2slot and s2i == o.st.slot2id and ts == o.st.slot_ts, l
            assert tick == o.st.tick
            counts = check_grouping(g, ids_o, wl.E, wl.T)
            assert counts.sum() == wl.T * wl.k
            if check_bytes and on_demand:
                for i, e in enumerate(passes[-1]):
                    assert np.array_equal(g.slot_bytes(i), g.bank(l * wl.E + e)), (l, e)
            elif check_bytes:
                for e in (0, wl.E // 2, wl.E - 1):
                    assert np.array_equal(g.slot_bytes(b * wl.E + e), g.bank(l * wl.E + e)), (l, e)
            yg = y.float().cpu().numpy().astype(np.float64)
            xf = x_f64(wl, x)
            if sample_tokens is None:
                rows = np.arange(wl.T)
            else:
                rows = np.sort(rng.choice(wl.T, size=sample_tokens, replace=False))
            ref = OY.moe_layer(xf[rows], ids_o[rows], w_o[rows], l, wl.E, o.weights)
            err, _ = rel_err(yg[rows], ref)
            worst = max(worst, err)
            log(f"  layer {l}: tokens checked {len(rows)}, max rel err {err:.3e} "
                f"(bf16 rounding alone {bf16_round_err(ref):.3e}); experts used "
                f"{int((counts > 0).sum())}, max n_e {int(counts.max())}, min n_e {int(counts.min())}"
                + (f"; on-demand passes {len(passes)}" if on_demand else ""))
            assert err <= TOL, (l, err)
        if decode_after:
            # decode continues from what prefill left resident
            dl = dataclasses.replace(wl, T=1, steps=2, prefill=False)
            logits = W.decode_logits(dl)
            for s in range(2):
                for l in range(wl.L):
                    xdec = W.hidden(dl, 100 + s, l)
                    ids_g, w_g = g.decode_call(l, logits[s, l], xdec)
                    ids_o, w_o = o.route(logits[s, l])
                    assert np.array_equal(ids_g, ids_o)
                    op = o.plan(l, ids_o)
                    compare_plan(g.plan_view(1), op, 1)
                    ref = o.output(l, x_f64(dl, xdec), ids_o, w_o)
                    y1 = g.y[:1].float().cpu().numpy().astype(np.float64)
                    assert rel_err(y1, ref)[0] <= TOL
            log("  decode after prefill: plans bit-exact, outputs within tolerance")
        return worst
    finally:
        g.close()


def test_prefill_mini_every_token():
    wl = dataclasses.replace(W.DSV4_PREFILL, L=3, E=16, k=4, H=512, I=512, T=333, n_slots=40)
    log("prefill mini: L=3 E=16 k=4 H=512 I=512 T=333 n=40")
    run_prefill(wl, decode_after=True)


def test_prefill_mini_single_buffer():
    """The second buffer disabled: every layer in slots [0, E), n < 2E, and
    decode continuing from what is left."""
    wl = dataclasses.replace(W.DSV4_PREFILL, L=3, E=16, k=4, H=512, I=512, T=333, n_slots=24)
    log("prefill mini, one buffer: L=3 E=16 k=4 H=512 I=512 T=333 n=24")
    run_prefill(wl, decode_after=True, buffers=1)


def test_prefill_mini_on_demand_passes():
    """n < E: the on-demand fallback loads the routed experts in passes of at
    most n (4 passes of 5, 5, 5, 1 when all 16 are routed); every token, the
    tables after each layer, the last pass's slot bytes, decode after."""
    wl = dataclasses.replace(W.DSV4_PREFILL, L=3, E=16, k=4, H=512, I=512, T=333, n_slots=5)
    log("prefill mini, on demand: L=3 E=16 k=4 H=512 I=512 T=333 n=5")
    run_prefill(wl, decode_after=True)


def test_prefill_mini_on_demand_one_pass():
    """E <= n < 2E with two buffers configured: one on-demand pass over the
    routed experts; T small enough that some experts are not routed."""
    wl = dataclasses.replace(W.DSV4_PREFILL, L=3, E=16, k=2, H=512, I=512, T=5, n_slots=20)
    log("prefill mini, on demand one pass: L=3 E=16 k=2 H=512 I=512 T=5 n=20")
    run_prefill(wl, decode_after=True)


def test_prefill_mini_large_tiles():
    # several 128-row tiles per expert, ragged tails, every token
    wl = dataclasses.replace(W.DSV4_PREFILL, L=2, E=8, k=2, H=1024, I=512, T=1111, n_slots=16)
    log("prefill mini 2: L=2 E=8 k=2 H=1024 I=512 T=1111 n=16")
    run_prefill(wl)


def _bits_to_f64(bits):
    return W.bf16_bits_to_f32(bits.view(np.uint16)).astype(np.float64)


@pytest.mark.timeout(900)
def test_prefill_full():
    """The full chunk: 8 layers x 8,192 tokens through two full-layer buffers
    (512 slots), then the last layer once more, then the pool shrunk to the
    DeepSeek-shaped decode budget (225 slots, fewer than two full layers) and
    the same chunk through on-demand loading, then decode."""
    import torch
    wl = W.DSV4_PREFILL
    n_od = W.DSV4_MXFP4.n_slots
    log("prefill full: 8 layers x 8192 tokens, E=256, H=4096, I=2048, n=512, then n=225 on demand")
    g = DeviceRun(wl, n_slots=wl.n_slots, max_tokens=8, max_prefill_tokens=wl.T)
    try:
        o = OracleRun(wl, g.bank, n_slots=wl.n_slots, max_tokens=8)
        dev = g.dev
        ids = torch.empty((wl.T, wl.k), dtype=torch.int32, device=dev)
        w = torch.empty((wl.T, wl.k), dtype=torch.float32, device=dev)
        y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=dev)
        rng = np.random.default_rng(7)

        def layer_call(l):
            lg = W.prefill_logits(wl, l)
            x = W.hidden(wl, 0, l)
            g.B.moe_route_topk(g.ctx, torch.from_numpy(lg).to(dev), wl.T, ids, w)
            g.B.moe_prefill_layer(g.ctx, l, g.to_dev_x(x), wl.T, ids, w, y)
            torch.cuda.synchronize()
            ids_o, w_o = o.route(lg)
            assert np.array_equal(ids.cpu().numpy(), ids_o), l
            return x, ids_o, w_o, y.view(torch.int16).cpu().numpy().copy()

        def tables_match(where):
            i2s, s2i, ts, tick = g.tables()
            assert i2s == o.st.id2slot and s2i == o.st.slot2id and ts == o.st.slot_ts, where
            assert tick == o.st.tick, where

        ys = []
        for l in range(wl.L):
            x, ids_o, w_o, yb = layer_call(l)
            b = OP.prefill_admit(o.st, l, wl.E, 2)
            tables_match(l)
            counts = check_grouping(g, ids_o, wl.E, wl.T)
            top = int(np.argmax(counts))
            for e in sorted({0, wl.E // 2, wl.E - 1, top}):
                assert np.array_equal(g.slot_bytes(b * wl.E + e), g.bank(l * wl.E + e)), (l, e)
            ys.append(yb)
            if l == 0:
                rows = np.arange(wl.T)
            else:
                rows = np.union1d(rng.choice(wl.T, size=256, replace=False), [0, wl.T - 1])
            xf = x_f64(wl, x)
            ref = o.output(l, xf[rows], ids_o[rows], w_o[rows])
            err, _ = rel_err(_bits_to_f64(yb)[rows], ref)
            log(f"  layer {l}: {len(rows)} tokens, max rel err {err:.3e} (bf16 rounding alone "
                f"{bf16_round_err(ref):.3e}); experts routed {int((counts > 0).sum())}, n_e "
                f"{int(counts.min())}..{int(counts.max())}, M-tiles {int(((counts + 127) // 128).sum())}")
            assert err <= TOL, (l, err)

        # the last layer once more: its buffer already holds it; one more tick,
        # and the output bit for bit the same (grouping order is free, rows are not)
        last = wl.L - 1
        _, ids_o, _, yb = layer_call(last)
        OP.prefill_admit(o.st, last, wl.E, 2)
        tables_match("repeat")
        check_grouping(g, ids_o, wl.E, wl.T)
        assert np.array_equal(yb, ys[last]), "repeated layer differs"
        log("  last layer repeated: bit-identical output, tables as the oracle's")

        # shrink to the decode budget: prefill now loads on demand
        g.B.moe_cache_resize(g.ctx, n_od, 60_000)
        o.resize(n_od)
        tables_match("resize")
        for l in range(wl.L):
            _, ids_o, _, yb = layer_call(l)
            passes = OP.prefill_on_demand(o.st, l, ids_o.ravel(), wl.E)
            tables_match(("on demand", l))
            check_grouping(g, ids_o, wl.E, wl.T)
            lp = passes[-1]
            for i in sorted({0, len(lp) // 2, len(lp) - 1}):
                assert np.array_equal(g.slot_bytes(i), g.bank(l * wl.E + lp[i])), (l, i)
            assert np.array_equal(yb, ys[l]), ("on-demand output differs from two buffers", l)
            log(f"  on demand, layer {l}: {len(passes)} passes, output bit-identical to two buffers")

        # decode continues from what the chunk left resident
        dl = dataclasses.replace(wl, T=1, steps=2, prefill=False)
        logits = W.decode_logits(dl)
        for s_ in range(2):
            for l in range(wl.L):
                xdec = W.hidden(dl, 100 + s_, l)
                ids_g, _ = g.decode_call(l, logits[s_, l], xdec)
                ids_o, w_o = o.route(logits[s_, l])
                assert np.array_equal(ids_g, ids_o)
                compare_plan(g.plan_view(1), o.plan(l, ids_o), 1)
                ref = o.output(l, x_f64(dl, xdec), ids_o, w_o)
                assert rel_err(g.y[:1].float().cpu().numpy().astype(np.float64), ref)[0] <= TOL
        log("  decode after the chunk: plans bit-exact, outputs within tolerance")
    finally:
        g.close()


def test_prefill_then_resize_with_pending_slab():
    """Prefill layers 0..2 of 4 with two buffers: layer 2's call streams layer
    3 into the other buffer ahead of time.  A resize at that point admits the
    pending slab first (as decode would), then keeps the most recent experts;
    tables bit-exact against the oracle (admit layer 3, then resize), every
    survivor's slot holds its bank's bytes, and decode continues with plans
    bit-exact and outputs within tolerance.  Then a grow and the same again."""
    import torch
    wl = dataclasses.replace(W.DSV4_PREFILL, L=4, E=16, k=4, H=512, I=512, T=200, n_slots=40)
    log("prefill then resize with a pending slab: L=4 E=16 k=4 H=512 I=512 T=200 n=40")
    g = DeviceRun(wl, n_slots=wl.n_slots, max_slots=64, max_tokens=8, max_prefill_tokens=wl.T)
    try:
        o = OracleRun(wl, g.bank, n_slots=wl.n_slots, max_tokens=8)
        dev = g.dev
        ids = torch.empty((wl.T, wl.k), dtype=torch.int32, device=dev)
        w = torch.empty((wl.T, wl.k), dtype=torch.float32, device=dev)
        y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=dev)
        dl = dataclasses.replace(wl, T=1, steps=6, prefill=False)
        logits = W.decode_logits(dl)

        def tables_match(where):
            i2s, s2i, ts, tick = g.tables()
            assert i2s == o.st.id2slot and s2i == o.st.slot2id and ts == o.st.slot_ts, where
            assert tick == o.st.tick, where
            for sl, u in enumerate(s2i):
                if u >= 0:
                    assert np.array_equal(g.slot_bytes(sl), g.bank(u)), (where, sl, u)

        for rnd, n_new in enumerate((17, 64)):
            for l in range(3):
                lg = W.prefill_logits(wl, l)
                x = W.hidden(wl, rnd, l)
                g.B.moe_route_topk(g.ctx, torch.from_numpy(lg).to(dev), wl.T, ids, w)
                g.B.moe_prefill_layer(g.ctx, l, g.to_dev_x(x), wl.T, ids, w, y)
                torch.cuda.synchronize()
                ids_o, w_o = o.route(lg)
                if o.st.n_slots >= 2 * wl.E:
                    OP.prefill_admit(o.st, l, wl.E, 2)
                else:
                    OP.prefill_on_demand(o.st, l, ids_o.ravel(), wl.E)
                ref = OY.moe_layer(x_f64(wl, x), ids_o, w_o, l, wl.E, o.weights)
                assert rel_err(y.float().cpu().numpy().astype(np.float64), ref)[0] <= TOL
            if o.st.n_slots >= 2 * wl.E:
                OP.prefill_admit(o.st, 3, wl.E, 2)  # the slab streamed ahead, admitted by the resize
            g.B.moe_cache_resize(g.ctx, n_new, 60_000)
            o.resize(n_new)
            tables_match(("resize", n_new))
            for s_ in range(3 * rnd, 3 * rnd + 3):
                for l in range(wl.L):
                    xdec = W.hidden(dl, 50 + s_, l)
                    ids_g, _ = g.decode_call(l, logits[s_, l], xdec)
                    ids_o, w_o = o.route(logits[s_, l])
                    assert np.array_equal(ids_g, ids_o)
                    compare_plan(g.plan_view(1), o.plan(l, ids_o), 1)
                    ref = o.output(l, x_f64(dl, xdec), ids_o, w_o)
                    assert rel_err(g.y[:1].float().cpu().numpy().astype(np.float64), ref)[0] <= TOL
            tables_match(("decode after resize", n_new))
            log(f"  resized to {n_new} with a pending slab: tables, slot bytes and decode as the oracle's")
    finally:
        g.close()


def test_prefill_two_buffers_cache_hits():
    """Decode first, in a pool of 2E + 16 slots: experts of every layer end up
    in slots outside the two full-layer buffers [0, 2E).  A two-buffer prefill
    of every layer then copies those experts device to device into the
    buffers and brings only the others over PCIe.  Tables follow the oracle's
    buffer admission, every buffer slot holds its bank's bytes, every token is
    within tolerance, the copy counts match the residency the chunk found, and
    decode continues.  A second chunk right after finds no expert outside the
    buffers (the first chunk's admissions emptied them): it copies from the
    host, except the layer whose slab is still in its buffer."""
    import torch
    wl = dataclasses.replace(W.DSV4_PREFILL, L=3, E=16, k=4, H=512, I=512, T=333, n_slots=48)
    log("two-buffer prefill after decode: L=3 E=16 k=4 H=512 I=512 T=333 n=48")
    g = DeviceRun(wl, n_slots=wl.n_slots, max_tokens=8, max_prefill_tokens=wl.T)
    try:
        o = OracleRun(wl, g.bank, n_slots=wl.n_slots, max_tokens=8)
        dl = dataclasses.replace(wl, T=1, steps=16, prefill=False)
        logits = W.decode_logits(dl)

        def decode_steps(steps):
            for s_ in steps:
                for l in range(wl.L):
                    xdec = W.hidden(dl, 300 + s_, l)
                    ids_g, _ = g.decode_call(l, logits[s_, l], xdec)
                    ids_o, w_o = o.route(logits[s_, l])
                    assert np.array_equal(ids_g, ids_o)
                    compare_plan(g.plan_view(1), o.plan(l, ids_o), 1)
                    ref = o.output(l, x_f64(dl, xdec), ids_o, w_o)
                    assert rel_err(g.y[:1].float().cpu().numpy().astype(np.float64), ref)[0] <= TOL

        decode_steps(range(12))
        i2s = g.tables()[0]
        outside = {l: [e for e in range(wl.E) if i2s[l * wl.E + e] >= 2 * wl.E] for l in range(wl.L)}
        n_out = sum(len(v) for v in outside.values())
        log(f"  after decode: experts outside the buffers per layer {[len(outside[l]) for l in range(wl.L)]}")
        assert n_out > 0, "the scenario must leave experts outside the full-layer buffers"
        dev = g.dev
        ids = torch.empty((wl.T, wl.k), dtype=torch.int32, device=dev)
        w = torch.empty((wl.T, wl.k), dtype=torch.float32, device=dev)
        y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=dev)
        st0 = g.B.moe_ctx_stats(g.ctx)
        for chunk in range(2):
            for l in range(wl.L):
                lg = W.prefill_logits(wl, l)
                x = W.hidden(wl, chunk, l)
                g.B.moe_route_topk(g.ctx, torch.from_numpy(lg).to(dev), wl.T, ids, w)
                g.B.moe_prefill_layer(g.ctx, l, g.to_dev_x(x), wl.T, ids, w, y)
                torch.cuda.synchronize()
                ids_o, w_o = o.route(lg)
                b = OP.prefill_admit(o.st, l, wl.E, 2)
                i2s_g, s2i, ts, tick = g.tables()
                assert i2s_g == o.st.id2slot and s2i == o.st.slot2id and ts == o.st.slot_ts, (chunk, l)
                assert tick == o.st.tick
                for e in range(wl.E):
                    assert np.array_equal(g.slot_bytes(b * wl.E + e), g.bank(l * wl.E + e)), (chunk, l, e)
                ref = OY.moe_layer(x_f64(wl, x), ids_o, w_o, l, wl.E, o.weights)
                err, _ = rel_err(y.float().cpu().numpy().astype(np.float64), ref)
                assert err <= TOL, (chunk, l, err)
            st1 = g.B.moe_ctx_stats(g.ctx)
            d2d = st1.prefill_d2d_experts - st0.prefill_d2d_experts
            h2d = st1.prefill_h2d_experts - st0.prefill_h2d_experts
            # chunk 0 copies every layer; chunk 1 finds layer 1 still in buffer 1
            # (layer 2 went to buffer 0 last) and reuses it, copying layers 0 and 2
            want_d2d = n_out if chunk == 0 else 0
            want_total = wl.L * wl.E if chunk == 0 else (wl.L - 1) * wl.E
            log(f"  chunk {chunk}: {d2d} experts device to device, {h2d} over PCIe")
            assert d2d == want_d2d and h2d == want_total - want_d2d, (chunk, d2d, h2d)
            st0 = st1
        decode_steps(range(12, 16))
        log("  decode after: plans bit-exact, outputs within tolerance")
    finally:
        g.close()


def test_prefill_on_demand_cache_hits():
    """Decode first: two layers of 16 experts through 24 slots leave some of
    layer 1's experts in slots 16..23.  An on-demand prefill of layer 1 (one
    pass of at most 16) then copies those device to device and brings the
    rest over PCIe; the same chunk once more finds every expert in its pass
    slot and copies nothing.  The tables
    follow the oracle's on-demand admission, every pass slot holds its bank's
    bytes, every token is within tolerance, and decode continues."""
    import torch
    wl = dataclasses.replace(W.DSV4_PREFILL, L=2, E=16, k=4, H=512, I=512, T=333, n_slots=24)
    log("prefill on demand after decode: L=2 E=16 k=4 H=512 I=512 T=333 n=24")
    g = DeviceRun(wl, n_slots=wl.n_slots, max_tokens=8, max_prefill_tokens=wl.T)
    try:
        o = OracleRun(wl, g.bank, n_slots=wl.n_slots, max_tokens=8)
        dl = dataclasses.replace(wl, T=1, steps=12, prefill=False)
        logits = W.decode_logits(dl)

        def decode_steps(steps):
            for s in steps:
                for l in range(wl.L):
                    xdec = W.hidden(dl, 200 + s, l)
                    ids_g, _ = g.decode_call(l, logits[s, l], xdec)
                    ids_o, w_o = o.route(logits[s, l])
                    assert np.array_equal(ids_g, ids_o)
                    compare_plan(g.plan_view(1), o.plan(l, ids_o), 1)
                    ref = o.output(l, x_f64(dl, xdec), ids_o, w_o)
                    assert rel_err(g.y[:1].float().cpu().numpy().astype(np.float64), ref)[0] <= TOL

        decode_steps(range(10))
        layer = 1
        lg = W.prefill_logits(wl, layer)
        ids_o, w_o = o.route(lg)
        routed = sorted(set(ids_o.ravel().tolist()))
        P = min(len(routed), wl.n_slots)
        i2s = g.tables()[0]
        beyond = [e for e in routed if i2s[layer * wl.E + e] >= P]
        in_place = [e for i, e in enumerate(routed) if i2s[layer * wl.E + e] == i]
        log(f"  before prefill: {len(routed)} routed, resident beyond the pass {beyond}, in place {in_place}")
        assert beyond, "the scenario must leave a routed expert beyond the pass's slots"
        dev = g.dev
        ids = torch.empty((wl.T, wl.k), dtype=torch.int32, device=dev)
        w = torch.empty((wl.T, wl.k), dtype=torch.float32, device=dev)
        y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=dev)
        x = W.hidden(wl, 0, layer)
        st0 = g.B.moe_ctx_stats(g.ctx)
        g.B.moe_route_topk(g.ctx, torch.from_numpy(lg).to(dev), wl.T, ids, w)
        g.B.moe_prefill_layer(g.ctx, layer, g.to_dev_x(x), wl.T, ids, w, y)
        torch.cuda.synchronize()
        assert np.array_equal(ids.cpu().numpy(), ids_o)
        passes = OP.prefill_on_demand(o.st, layer, ids_o.ravel(), wl.E)
        assert len(passes) == 1
        st1 = g.B.moe_ctx_stats(g.ctx)
        assert st1.prefill_d2d_experts - st0.prefill_d2d_experts == len(beyond)
        assert st1.prefill_h2d_experts - st0.prefill_h2d_experts == P - len(beyond) - len(in_place)
        i2s, s2i, ts, tick = g.tables()
        assert i2s == o.st.id2slot and s2i == o.st.slot2id and ts == o.st.slot_ts and tick == o.st.tick
        for i, e in enumerate(passes[0]):
            assert np.array_equal(g.slot_bytes(i), g.bank(layer * wl.E + e)), (i, e)
        ref = OY.moe_layer(x_f64(wl, x), ids_o, w_o, layer, wl.E, o.weights)
        err, _ = rel_err(y.float().cpu().numpy().astype(np.float64), ref)
        log(f"  prefill: max rel err {err:.3e}")
        assert err <= TOL
        # the same chunk again: every expert is already in its pass slot, so
        # nothing is copied; tables, bytes and outputs as before
        y.zero_()
        g.B.moe_prefill_layer(g.ctx, layer, g.to_dev_x(x), wl.T, ids, w, y)
        torch.cuda.synchronize()
        st2 = g.B.moe_ctx_stats(g.ctx)
        assert (st2.prefill_d2d_experts, st2.prefill_h2d_experts) == (st1.prefill_d2d_experts,
                                                                     st1.prefill_h2d_experts)
        assert OP.prefill_on_demand(o.st, layer, ids_o.ravel(), wl.E) == passes
        i2s, s2i, ts, tick = g.tables()
        assert i2s == o.st.id2slot and s2i == o.st.slot2id and ts == o.st.slot_ts and tick == o.st.tick
        for i, e in enumerate(passes[0]):
            assert np.array_equal(g.slot_bytes(i), g.bank(layer * wl.E + e)), (i, e)
        err2, _ = rel_err(y.float().cpu().numpy().astype(np.float64), ref)
        log(f"  prefill again (all in place): max rel err {err2:.3e}")
        assert err2 <= TOL
        decode_steps(range(10, 12))
    finally:
        g.close()
