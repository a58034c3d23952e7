"""GPU parity of the decode path at the real expert shapes.

Mid-size cases use the Qwen-shaped bf16 and DeepSeek-shaped MXFP4 experts
with fewer layers and steps (every plan, table and output checked).  Full
cases run the stated workloads end to end: every plan and table bit-exact on
every call; outputs compared with the fp64 oracle on sampled calls (the
oracle's dequantised fp64 expert evaluation is the slow part).
Tolerance for bf16 / MXFP4: max |y - y_oracle| <= 2e-2 x RMS(y_oracle)."""
import dataclasses

import numpy as np
import pytest

import workload as W
from tests.harness import (DeviceRun, OracleRun, bf16_round_err, compare_plan, d2h, h2d, log, rel_err,
                           x_f64)

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "mxfp4": 2e-2}


def run_decode(wl, mode=0, check_output=lambda s, l: True, check_fill=lambda s, l: False,
               resize=None, n_slots=None, max_fetch=0):
    resize = wl.resize if resize is None else resize
    g = DeviceRun(wl, mode=mode, n_slots=n_slots, max_fetch=max_fetch)
    try:
        o = OracleRun(wl, g.bank, mode=mode, n_slots=n_slots, max_fetch=max_fetch)
        logits = W.router_logits(wl)
        worst, worst_round, checked, stats = 0.0, 0.0, 0, dict(hit=0, q=0, cpu=0)
        for s in range(wl.steps):
            if s in resize:
                g.B.moe_cache_resize(g.ctx, resize[s], 60_000)
                moves = o.resize(resize[s])
                i2s, s2i, ts, tick = g.tables()
                assert i2s == o.st.id2slot and s2i == o.st.slot2id and ts == o.st.slot_ts, s
                # moved survivors (and a few that stayed) hold their banks' bytes
                stayed = [j for j, u in enumerate(s2i) if u >= 0 and j not in {d for _, d in moves}]
                for j in [d for _, d in moves][:24] + stayed[:4]:
                    assert np.array_equal(g.slot_bytes(j), g.bank(s2i[j])), (s, j)
                log(f"  resized to {resize[s]} before step {s}: {len(moves)} survivors moved")
            for l in range(wl.L):
                x = W.hidden(wl, s, l)
                ids_g, w_g = g.decode_call(l, logits[s, l], x)
                ids_o, w_o = o.route(logits[s, l])
                assert np.array_equal(ids_g, ids_o), (s, l)
                assert np.allclose(w_g, w_o, rtol=2e-6, atol=1e-7)
                op = o.plan(l, ids_o)
                gp = g.plan_view(wl.T)
                compare_plan(gp, op, wl.T)
                stats["hit"] += len(op.hits)
                stats["q"] += op.q
                stats["cpu"] += len(op.cpu)
                if check_fill(s, l):
                    for (u, sl, old) in op.fills:
                        assert np.array_equal(g.slot_bytes(sl), g.bank(u)), (s, l, u, sl)
                if check_output(s, l):
                    y_ref = o.output(l, x_f64(wl, x), ids_o, w_o)
                    err, rms = rel_err(g.y_f64(), y_ref)
                    if err > worst:
                        worst = err
                        worst_round = bf16_round_err(y_ref) if wl.act_dtype == "bf16" else 0.0
                    checked += 1
                    assert err <= TOL[wl.w_dtype], (s, l, err)
            if s % 32 == 0 or s == wl.steps - 1:
                i2s, s2i, ts, tick = g.tables()
                assert i2s == o.st.id2slot and s2i == o.st.slot2id, s
                assert ts == o.st.slot_ts and tick == o.st.tick, s
                log(f"  step {s}: worst rel err {worst:.3e} (bf16 output rounding alone: "
                    f"{worst_round:.3e}) over {checked} outputs; {stats}")
        st = g.B.moe_ctx_stats(g.ctx)
        assert st.hits == stats["hit"] and st.fills == stats["q"] and st.cpu == stats["cpu"]
        return worst, checked, stats
    finally:
        g.close()


def mini(wl, **kw):
    return dataclasses.replace(wl, **kw)


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_bf16_mini_every_call(mode):
    wl = mini(W.QWEN_BF16, L=4, steps=20, n_slots=189)
    log(f"bf16 mini mode={mode}")
    worst, n, st = run_decode(wl, mode=mode, check_fill=lambda s, l: True)
    log(f"bf16 mini mode={mode}: worst {worst:.3e} over {n} outputs {st}")


@pytest.mark.parametrize("mode", [0, 1])
def test_mxfp4_mini_every_call(mode):
    wl = mini(W.DSV4_MXFP4, L=2, steps=12, n_slots=56)
    log(f"mxfp4 mini mode={mode}")
    worst, n, st = run_decode(wl, mode=mode, check_fill=lambda s, l: True)
    log(f"mxfp4 mini mode={mode}: worst {worst:.3e} over {n} outputs {st}")


@pytest.mark.parametrize("T", [1, 3])
def test_bf16_partial_chunk_columns(T):
    """bf16 experts whose rows leave the last 64-lane column of 16-byte
    chunks partly empty in both halves of the FFN: H = 576 (72 chunks of a
    W_gate / W_up row, two per lane, gate/up items of two rows) and I = 320
    (40 chunks of a W_down row, one per lane, lanes 40-63 idle, down items of
    eight rows), at one and three tokens per call.  Every plan bit-exact,
    every output within tolerance, filled slots byte-equal to their banks."""
    wl = mini(W.QWEN_BF16, L=2, steps=8, n_slots=60, H=576, I=320, T=T)
    log(f"bf16 H=576 I=320 T={T}")
    worst, n, st = run_decode(wl, check_fill=lambda s, l: True)
    log(f"bf16 H=576 I=320 T={T}: worst {worst:.3e} over {n} outputs {st}")


def test_bf16_streams_mini_with_resizes():
    wl = mini(W.QWEN_ELASTIC, L=3, steps=24, n_slots=141, resize={6: 57, 12: 115, 18: 115})
    log("bf16 8-stream mini")
    worst, n, st = run_decode(wl, check_fill=lambda s, l: True)
    log(f"bf16 8-stream mini: worst {worst:.3e} over {n} outputs {st}")


def test_tiny_pool_and_max_fetch_edges():
    # empty pool: everything on the host; then a fetch cap of 1
    wl = mini(W.QWEN_BF16, L=2, steps=6, n_slots=0)
    run_decode(wl, n_slots=0)
    wl = mini(W.QWEN_BF16, L=2, steps=6, n_slots=40)
    run_decode(wl, n_slots=40, max_fetch=1, mode=1)


# ------------------------------------------------------------------ full workloads
@pytest.mark.timeout(900)
def test_qwen_bf16_full():
    wl = W.QWEN_BF16
    log("qwen bf16 full: 48 layers x 256 steps, n=2273")
    # every layer on the first step, the first timed step of the bench (32),
    # a middle step and the last; four layers every 16th step
    worst, n, st = run_decode(
        wl, check_output=lambda s, l: s in (0, 32, 128, wl.steps - 1) or (s % 16 == 0 and l < 4),
        check_fill=lambda s, l: s % 64 == 1)
    log(f"qwen bf16 full: worst {worst:.3e} over {n} outputs {st}")


@pytest.mark.timeout(900)
def test_dsv4_mxfp4_full():
    wl = W.DSV4_MXFP4
    log("dsv4 mxfp4 full: 8 layers x 128 steps, n=225")
    worst, n, st = run_decode(
        wl, check_output=lambda s, l: s % 16 == 0 or s == wl.steps - 1,
        check_fill=lambda s, l: s % 32 == 1)
    log(f"dsv4 mxfp4 full: worst {worst:.3e} over {n} outputs {st}")


@pytest.mark.timeout(1200)
def test_qwen_elastic_full():
    wl = W.QWEN_ELASTIC
    log("qwen elastic 8 streams full: 48 layers x 512 steps, resizes " + str(wl.resize))
    # every layer on the steps on each side of every resize and on the last
    # step; two layers every 64th step
    worst, n, st = run_decode(
        wl, check_output=lambda s, l: s in (127, 128, 255, 256, 383, 384, wl.steps - 1)
        or (s % 64 == 0 and l < 2))
    log(f"qwen elastic full: worst {worst:.3e} over {n} outputs {st}")


def test_cpu_layers_bf16():
    """Layers 1 and 3 decode on the host (mode CPU for their calls), the others
    hybrid: every plan bit-exact against the oracle run with the same
    per-layer modes, outputs within tolerance, and no expert of a host layer
    ever admitted.  Switching the flags off mid-run lets those layers fill."""
    wl = mini(W.QWEN_BF16, L=4, steps=12, n_slots=189)
    g = DeviceRun(wl)
    try:
        o = OracleRun(wl, g.bank)
        logits = W.router_logits(wl)
        cpu = [False, True, False, True]
        g.B.moe_set_cpu_layers(g.ctx, cpu)
        worst = 0.0
        for s in range(wl.steps):
            if s == 8:
                g.B.moe_set_cpu_layers(g.ctx, None)
                cpu = [False] * wl.L
            for l in range(wl.L):
                x = W.hidden(wl, s, l)
                ids_g, w_g = g.decode_call(l, logits[s, l], x)
                ids_o, w_o = o.route(logits[s, l])
                assert np.array_equal(ids_g, ids_o), (s, l)
                o.mode = 2 if cpu[l] else 0
                op = o.plan(l, ids_o)
                compare_plan(g.plan_view(wl.T), op, wl.T)
                if cpu[l]:
                    assert op.q == 0 and not op.hits, (s, l)
                err, _ = rel_err(g.y_f64(), o.output(l, x_f64(wl, x), ids_o, w_o))
                worst = max(worst, err)
                assert err <= TOL[wl.w_dtype], (s, l, err)
            if s == 7:
                i2s, _, _, _ = g.tables()
                for l in (1, 3):
                    assert all(i2s[l * wl.E + e] == -1 for e in range(wl.E)), l
        i2s, s2i, ts, tick = g.tables()
        assert i2s == o.st.id2slot and s2i == o.st.slot2id and ts == o.st.slot_ts
        assert any(i2s[1 * wl.E + e] >= 0 for e in range(wl.E))  # filled once released
        log(f"  host layers 1, 3 then none: worst rel err {worst:.3e}")
    finally:
        g.close()


@pytest.mark.parametrize("T", [1, 3])
def test_repeated_expert_in_a_token(T):
    """ids given directly, with an expert listed two or three times by one
    token (the layer sums w[t][j] * FFN_e(x_t) over every j, repeats
    included): plans bit-exact, outputs within tolerance, and a repeated
    pair's partial rows equal to its first occurrence's.  T = 1 runs the
    single-pair FFN kernel, T = 3 the token loop."""
    wl = mini(W.QWEN_BF16, L=2, steps=6, n_slots=40, T=T)
    g = DeviceRun(wl)
    torch = g.torch
    try:
        o = OracleRun(wl, g.bank)
        rng = np.random.default_rng(7)
        worst = 0.0
        for s in range(wl.steps):
            for l in range(wl.L):
                ids = np.empty((T, wl.k), np.int32)
                for t in range(T):
                    pick = rng.choice(wl.E, 5, replace=False)
                    ids[t] = [pick[0], pick[0], pick[1], pick[2], pick[2], pick[2], pick[3], pick[4]]
                    if (s + t) % 2:
                        ids[t] = ids[t][::-1]
                w = rng.random((T, wl.k)).astype(np.float32)
                w /= w.sum(axis=1, keepdims=True)
                x = W.hidden(wl, s, l)
                xd = g.to_dev_x(x)
                idd = torch.from_numpy(ids).to(g.dev)
                wd = torch.from_numpy(w).to(g.dev)
                g.B.moe_cache_plan(g.ctx, l, idd, T, xd)
                g.B.moe_expert_ffn(g.ctx, l, xd, T)
                g.B.moe_merge(g.ctx, wd, T, g.y[:T])
                torch.cuda.synchronize()
                op = o.plan(l, ids)
                gp = g.plan_view(T)
                compare_plan(gp, op, T)
                pg = g.p_gpu_rows(T)
                for t in range(T):
                    for j in range(wl.k):
                        first = int(np.flatnonzero(ids[t] == ids[t][j])[0])
                        if gp["slot_map"][t][j] >= 0 and first != j:
                            assert np.array_equal(pg[t, j], pg[t, first]), (s, l, t, j)
                err, _ = rel_err(g.y_f64()[:T], o.output(l, x_f64(wl, x), ids, w.astype(np.float64)))
                worst = max(worst, err)
                assert err <= TOL[wl.w_dtype], (s, l, err)
        log(f"  repeated experts, T={T}: worst rel err {worst:.3e}")
    finally:
        g.close()


def test_intermediate_marks_across_tick_jumps():
    """The expert FFN hands silu(gate) * up from its gate/up waves to its down
    workgroups as 64-bit entries {fp32 value, low 32 bits of the call's tick}.
    Before every step the clock moves on by 2^32 - 1 (the tick and every
    occupied slot's tick, on the device and in the oracle, which keeps the
    LRU order), so the first call of the step has the same low word as the
    call before it: only the control kernel's rewrite of every mark at a new
    2^30-tick epoch keeps that call's entries from passing for this one's.
    After each call: the GPU pairs' entries carry this call's mark and hold
    silu(W_g x) * (W_u x) of the oracle's weights; every other entry carries
    another mark (the rewritten one after a jump); plans and outputs match
    the oracle."""
    from oracle import expert as OX
    wl = mini(W.QWEN_BF16, L=2, steps=6, n_slots=189)
    g = DeviceRun(wl)
    try:
        o = OracleRun(wl, g.bank)
        logits = W.router_logits(wl)
        Tk, I = wl.T * wl.k, wl.I
        checked = 0
        for s in range(wl.steps):
            jumped = s > 0
            if jumped:
                v = g.B.moe_plan_view_get(g.ctx)
                ts = d2h(v.slot_ts, v.n_slots, np.int64)
                tick = int(d2h(v.tick, 1, np.int64)[0])
                assert tick == o.st.tick
                off = 2**32 - 1
                ts[ts >= 0] += off
                h2d(v.slot_ts, ts)
                h2d(v.tick, np.array([tick + off], np.int64))
                o.st.slot_ts = [t + off if t >= 0 else t for t in o.st.slot_ts]
                o.st.tick += off
            for l in range(wl.L):
                x = W.hidden(wl, s, l)
                ids_g, w_g = g.decode_call(l, logits[s, l], x)
                ids_o, w_o = o.route(logits[s, l])
                assert np.array_equal(ids_g, ids_o), (s, l)
                op = o.plan(l, ids_o)
                gp = g.plan_view(wl.T)
                compare_plan(gp, op, wl.T)
                v = g.B.moe_plan_view_get(g.ctx)
                tick = int(d2h(v.tick, 1, np.int64)[0])
                cur = tick & 0xFFFFFFFF
                hm = d2h(v.h_marked, Tk * I, np.uint64).reshape(Tk, I)
                marks = (hm >> np.uint64(32)).astype(np.int64)
                vals = (hm & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32)
                sm = np.asarray(gp["slot_map"]).ravel()
                xf = x_f64(wl, x)
                for p in range(Tk):
                    if sm[p] >= 0:
                        assert (marks[p] == cur).all(), (s, l, p)
                        wg, wu, _ = o.weights(l * wl.E + int(ids_o.ravel()[p]))
                        xt = xf[p // wl.k]
                        h_ref = OX.silu(wg @ xt) * (wu @ xt)
                        rms = np.sqrt(np.mean(h_ref ** 2))
                        assert np.max(np.abs(vals[p] - h_ref)) <= 2e-3 * rms, (s, l, p)
                        checked += 1
                    else:
                        assert (marks[p] != cur).all(), (s, l, p)
                        if jumped and l == 0:
                            assert (marks[p] == cur ^ 0x80000000).all(), (s, l, p)
                err, _ = rel_err(g.y_f64(), o.output(l, xf, ids_o, w_o))
                assert err <= TOL[wl.w_dtype], (s, l, err)
        assert o.st.tick > 5 * 2**32
        log(f"  marks checked on {checked} GPU pairs over {wl.steps - 1} clock jumps")
    finally:
        g.close()


@pytest.mark.parametrize("name,T", [("mxfp4", 4), ("f32", 3)])
def test_token_loop_other_formats(name, T):
    """Several tokens per call with MXFP4 (DeepSeek-shaped) and fp32 (tiny)
    experts: the FFN kernels evaluate every routed pair of an expert from one
    register-resident copy of its rows; every plan bit-exact, every output
    within tolerance, filled slots byte-equal to their banks."""
    if name == "mxfp4":
        wl = mini(W.DSV4_MXFP4, L=2, steps=6, n_slots=56, T=T)
    else:
        wl = mini(W.TINY, steps=12, T=T)
    log(f"{name} T={T}")
    worst, n, st = run_decode(wl, check_fill=lambda s, l: True)
    log(f"{name} T={T}: worst {worst:.3e} over {n} outputs {st}")
