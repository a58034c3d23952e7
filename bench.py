"""Benchmark of the routed-expert MoE decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one decode pass over every MoE layer of the workload: per layer
router top-k, the control kernel, the PCIe fill of admitted experts, the host
branch, the grouped expert GEMV and the merge.  The default workload is the
Qwen3.6-35B-A3B-shaped bf16 decode (48 layers, 128 experts, top-8, H 2048,
I 768, 2,273 slots = 37% of the pool, 256 steps, bandwidths 52.7 / 77.3 GB/s):
steps [0, W) run untimed on the cold cache, steps [W, W+K) are timed; all
router logits and hidden states are resident in HBM before timing starts.

Prints one JSON line: value = MoE-layer decode time in microseconds per layer
(wall clock over the timed steps, bracketed by device synchronisation), plus
the roofline of the expert FFN (HBM bytes of the unique GPU-resident experts
per launch over its duration, from HIP events the launch binds to its own
dispatch), a per-phase breakdown and the CPU
oracle timed on a bounded sample of the same calls.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Kernel sources whose counters profiles/traffic.json holds: a recorded
# figure is used only while these files are unchanged.
TRAFFIC_SOURCES = {
    "decode_ffn": ["routed_expert_execution_moe_amd/csrc/ffn.h",
                   "routed_expert_execution_moe_amd/csrc/ffn_bf16.hip"],
    "prefill_gemm": ["routed_expert_execution_moe_amd/csrc/prefill.hip"],
}
TRAFFIC_KERNELS = {"decode_ffn": ["ffn_kernel"], "prefill_gemm": ["grouped_gemm_kernel"]}
# FETCH_SIZE / WRITE_SIZE (KiB per dispatch) to bytes: what the counters read
# for a plain kernel of known size (--copy-calibration: 1 GiB read, 1 GiB written)
FETCH_SCALE, WRITE_SCALE = 2.0 * 1024, 1.0 * 1024
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def _sources_sha(kind):
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES[kind]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(kind, workload):
    """HBM bytes per launch from the committed counter record, or None when
    there is none, it was taken on another workload, or the kernel's source
    changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)[kind]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("workload") != workload or t.get("sha256") != _sources_sha(kind):
        return None
    return t["bytes_per_launch"]


def traffic_source(kind, workload):
    """Where `traffic` comes from: the committed counter record (two rocprofv3
    --pmc runs, FETCH_SIZE then WRITE_SIZE, of this bench on the named
    workload with this kernel source), not this run's counters."""
    if recorded_traffic(kind, workload) is None:
        return None
    with open(TRAFFIC_FILE) as fh:
        t = json.load(fh)[kind]
    return {"recorded": True, "file": "profiles/traffic.json", "workload": t["workload"],
            "kernel_source_sha256": t["sha256"][:16],
            "note": "HBM bytes per launch from earlier counter runs of this kernel source; "
                    "this run's algorithmic bytes are achieved's numerator"}


def record_traffic(kind, workload, fetch_dir, write_dir):
    """Write profiles/traffic.json[kind] from two rocprofv3 --pmc runs (one with
    FETCH_SIZE, one with WRITE_SIZE) of this bench: HBM bytes per dispatch of
    each of the kind's kernels, summed over them (the decode FFN is one
    launch per layer; the prefill GEMM is GEMM1 + GEMM2 per layer)."""
    def per_kernel(d, counter):
        sums = {}
        for f in glob.glob(os.path.join(d, "*counter_collection.csv")):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if r["Counter_Name"] != counter:
                        continue
                    name = r["Kernel_Name"]
                    key = next((k for k in TRAFFIC_KERNELS[kind] if k in name), None)
                    if key is None:
                        continue
                    tag = name.split("(")[0]
                    sums.setdefault(tag, []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in sums.items()}
    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")
    total = sum(fetch.values()) * FETCH_SCALE + sum(write.values()) * WRITE_SCALE
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        t = {}
    t[kind] = {"bytes_per_launch": round(total), "sha256": _sources_sha(kind), "workload": workload,
               "kernels": {k: {"fetch_kib": round(fetch.get(k, 0), 1),
                               "write_kib": round(write.get(k, 0), 1)} for k in sorted(set(fetch) | set(write))},
               "scale": {"FETCH_SIZE": FETCH_SCALE, "WRITE_SIZE": WRITE_SCALE}}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(t, fh, indent=1, sort_keys=True)
        fh.write("\n")
    return t[kind]


METRIC = "MoE-layer decode µs/layer + expert-FFN HBM GB/s (% of peak); prefill TFLOP/s"
HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="qwen3.6-35b-a3b-shape-bf16-decode")
    ap.add_argument("--mode", default="hybrid", choices=["hybrid", "offload", "cpu"])
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mxfp4", action="store_true",
                    help="leave out the DeepSeek-shaped MXFP4 decode leg")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-elastic", action="store_true", help="skip the resize-schedule leg")
    ap.add_argument("--max-fetch", type=int, default=0,
                    help="cap on PCIe fills per layer call (0: none); also bounds the victim list")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the decode run replayed from a captured HIP graph")
    ap.add_argument("--no-calibrated", action="store_true",
                    help="skip the decode run with B_P / B_H measured on this machine")
    ap.add_argument("--bw-profile", default=None, metavar="PATH",
                    help="also store the measured bandwidths in this JSON profile (keyed on "
                         "expert format + GPU name)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only the prefill leg (for profiling); prints its fields")
    ap.add_argument("--prefill-tokens", type=int, default=None,
                    help="with --prefill-only: chunk length other than the workload's 8,192")
    ap.add_argument("--prefill-main-only", action="store_true",
                    help="with --prefill-only: only the two-buffer passes (no one-buffer or "
                         "on-demand pass), so every GEMM launch covers a whole layer")
    ap.add_argument("--record-traffic", nargs=3, metavar=("KIND", "FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json[KIND] (decode_ffn | prefill_gemm) from the "
                         "counter CSVs of a FETCH_SIZE run and a WRITE_SIZE run of this bench "
                         "(decode: on --workload; prefill: its prefill workload)")
    ap.add_argument("--no-streams", action="store_true",
                    help="skip the 8-stream elastic workload leg")
    ap.add_argument("--streams-only", action="store_true",
                    help="run only the 8-stream elastic workload leg (for profiling); prints its fields")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain streaming kernel of known size, whose "
                         "FETCH_SIZE / WRITE_SIZE counter readings scale those counters to bytes")
    return ap.parse_args()


def bench_prefill(main_only=False, tokens=None):
    """One untimed pass and one timed pass of the DeepSeek-shaped MXFP4
    prefill chunk (8 layers x 8,192 tokens, two full-layer buffers of 256
    experts, the next layer's slab streamed while the current one computes),
    then one timed pass with one buffer, then one timed pass after the pool is
    resized to the DeepSeek-shaped decode budget (225 slots, fewer than two
    full layers: on-demand loading).  Returns the grouped-GEMM TFLOP/s (HIP
    events around the two GEMM kernels, two-buffer pass), the wall time per
    layer, the slab copy rate and the one-buffer and on-demand wall times."""
    import ctypes  # noqa: F401

    import numpy as np
    import torch

    import routed_expert_execution_moe_amd as B
    import workload as W

    wl = W.DSV4_PREFILL
    if tokens:  # another chunk length of the same workload (the one-buffer penalty sweep)
        import dataclasses
        wl = dataclasses.replace(wl, T=tokens)
    dev = torch.device("cuda:0")
    n_hd = 2 * wl.E + W.DSV4_MXFP4.n_slots  # two full-layer buffers + the decode budget
    cfg = B.config(wl.L, wl.E, wl.k, wl.H, wl.I, wl.w_dtype, wl.act_dtype, wl.n_slots,
                   max_slots=n_hd, max_tokens=1, bw_pcie_mbps=wl.bw_pcie_mbps,
                   bw_host_mbps=wl.bw_host_mbps, max_prefill_tokens=wl.T, timing=1)
    stride = B.moe_expert_bytes(cfg)
    pool_bytes = wl.n_ids * stride
    pool = B.moe_host_pool_alloc(pool_bytes)
    ctx = None
    try:
        W.fill_banks(wl, pool, 0, wl.n_ids)
        ctx = B.moe_create(cfg, pool, pool_bytes)
        lg = torch.from_numpy(np.stack([W.prefill_logits(wl, l) for l in range(wl.L)])).to(dev)
        xs = np.stack([W.hidden(wl, 0, l) for l in range(wl.L)])
        x = torch.from_numpy(xs.view(np.int16)).to(dev).view(torch.bfloat16)
        ids = torch.empty((wl.L, wl.T, wl.k), dtype=torch.int32, device=dev)
        w = torch.empty((wl.L, wl.T, wl.k), dtype=torch.float32, device=dev)
        y = torch.empty((wl.L, wl.T, wl.H), dtype=torch.bfloat16, device=dev)

        def one_pass():
            for l in range(wl.L):
                B.moe_route_topk(ctx, lg[l], wl.T, ids[l], w[l])
                B.moe_prefill_layer(ctx, l, x[l], wl.T, ids[l], w[l], y[l])

        one_pass()
        torch.cuda.synchronize()
        B.moe_ctx_timing(ctx, reset=True)
        t0 = time.perf_counter()
        one_pass()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        tm = B.moe_ctx_timing(ctx)
        # the same compute back to back: the last layer's buffer is resident and
        # the last layer prefetches nothing, so repeating its call runs the
        # GEMMs without the idle gaps of the transfer-bound pipeline (which let
        # the power controller clamp the clock during the second GEMM)
        last = wl.L - 1
        B.moe_ctx_timing(ctx, reset=True)
        for _ in range(wl.L):
            B.moe_route_topk(ctx, lg[last], wl.T, ids[last], w[last])
            B.moe_prefill_layer(ctx, last, x[last], wl.T, ids[last], w[last], y[last])
        torch.cuda.synchronize()
        tm_b2b = B.moe_ctx_timing(ctx)
        wall1 = wall_od = None
        hd = None
        used, n_od = 0, W.DSV4_MXFP4.n_slots
        if not main_only:
            # the ablation with the second full-layer buffer disabled: each
            # layer's slab copy waits for the previous layer's compute
            B.moe_prefill_set_buffers(ctx, 1)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            one_pass()
            torch.cuda.synchronize()
            wall1 = time.perf_counter() - t0
            B.moe_prefill_set_buffers(ctx, 2)
            # the pool shrunk (elastic resize) to the DeepSeek-shaped decode
            # budget, which cannot hold two full layers: on-demand loading
            n_od = W.DSV4_MXFP4.n_slots
            B.moe_cache_resize(ctx, n_od, 10000)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            one_pass()
            torch.cuda.synchronize()
            wall_od = time.perf_counter() - t0
            used = int((torch.bincount(ids[wl.L - 1].flatten().long(), minlength=wl.E) > 0).sum())
            # prefill after decode: the pool grown to two buffers plus the
            # decode budget; 16 decode steps of the DeepSeek-shaped decode
            # routing (T = 1) leave experts in slots outside the buffers, and
            # the next two-buffer pass copies those device to device
            B.moe_cache_resize(ctx, n_hd, 10000)
            dlg = torch.from_numpy(np.ascontiguousarray(W.decode_logits(W.DSV4_MXFP4, steps=16))).to(dev)
            i1 = torch.empty((1, wl.k), dtype=torch.int32, device=dev)
            w1 = torch.empty((1, wl.k), dtype=torch.float32, device=dev)
            y1 = torch.empty((1, wl.H), dtype=torch.bfloat16, device=dev)
            for s_ in range(16):
                for l in range(wl.L):
                    x1 = x[l, s_:s_ + 1]
                    B.moe_route_topk(ctx, dlg[s_, l], 1, i1, w1)
                    B.moe_cache_plan(ctx, l, i1, 1, x1)
                    B.moe_expert_ffn(ctx, l, x1, 1)
                    B.moe_merge(ctx, w1, 1, y1)
            torch.cuda.synchronize()
            sh0 = B.moe_ctx_stats(ctx)
            t0 = time.perf_counter()
            one_pass()
            torch.cuda.synchronize()
            wall_hd = time.perf_counter() - t0
            sh1 = B.moe_ctx_stats(ctx)
            hd = {"n_slots": n_hd, "decode_steps_before": 16, "layer_ms": round(wall_hd / wl.L * 1e3, 3),
                  "experts_device_to_device": sh1.prefill_d2d_experts - sh0.prefill_d2d_experts,
                  "experts_over_pcie": sh1.prefill_h2d_experts - sh0.prefill_h2d_experts,
                  "pcie_bytes_saved": (sh1.prefill_d2d_experts - sh0.prefill_d2d_experts)
                  * W.expert_bytes(wl)}
        flops = wl.L * 6.0 * wl.H * wl.I * wl.T * wl.k
        gemm_ms = tm["prefill_gemm"]["ms"]
        tflops = flops / (gemm_ms * 1e-3) / 1e12
        slab = wl.E * W.expert_bytes(wl)
        copy_ms = tm["prefill_copy"]["ms"]
        copies = tm["prefill_copy"]["calls"]
        return {
            "prefill_workload": wl.name,
            "prefill_tflops": round(tflops, 1),
            "prefill_roofline": {"bound": "mfma", "kernel": "grouped GEMM1 + GEMM2 (bf16 MFMA, "
                                 "MXFP4 dequantised in registers)", "achieved": round(tflops, 1),
                                 "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                 "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                                 "traffic": recorded_traffic("prefill_gemm", wl.name),
                                 "traffic_source": traffic_source("prefill_gemm", wl.name)},
            "prefill_gemm_ms_per_layer": round(gemm_ms / wl.L, 3),
            "prefill_gemm_back_to_back": {
                "note": "the last layer's compute repeated with its buffer resident, no idle between bursts",
                "tflops": round(flops / (tm_b2b["prefill_gemm"]["ms"] * 1e-3) / 1e12, 1),
                "frac": round(flops / (tm_b2b["prefill_gemm"]["ms"] * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                "gemm_ms_per_layer": round(tm_b2b["prefill_gemm"]["ms"] / wl.L, 3)},
            "prefill_group_ms_per_layer": round(tm["prefill_group"]["ms"] / wl.L, 3),
            "prefill_merge_ms_per_layer": round(tm["prefill_merge"]["ms"] / wl.L, 3),
            "prefill_layer_ms": round(wall / wl.L * 1e3, 3),
            "prefill_chunk_tok_s": round(wl.T / wall, 1),
            "prefill_copy_gbps": round(slab * copies / (copy_ms * 1e-3) / 1e9, 1) if copy_ms else None,
            "prefill_single_buffer": None if main_only else {
                "layer_ms": round(wall1 / wl.L * 1e3, 3), "penalty_pct": round((wall1 / wall - 1.0) * 100, 1)},
            "prefill_on_demand": None if main_only else {
                "n_slots": n_od, "layer_ms": round(wall_od / wl.L * 1e3, 3),
                "routed_experts_last_layer": used, "passes_last_layer": -(-used // n_od)},
            "prefill_after_decode_hit_d2d": hd,
        }
    finally:
        if ctx:
            B.moe_destroy(ctx)
        B.moe_host_pool_free(pool)


def bench_streams(steps=64, warmup=8):
    """The 8-stream elastic workload (Qwen3.6-35B-A3B shape, 8 concurrent
    batch-1 streams batched into T = 8 per layer call, its own seed and host
    pool) on its own state: `steps` decode steps, the first `warmup` untimed,
    with the workload's resize schedule (2,273 -> 921 -> 1,843 -> 1,843 slots)
    applied before steps steps/4, steps/2 and 3*steps/4 (the pages' schedule
    at 128 / 256 / 384 of 512 steps, scaled).  Per-phase HIP-event times over
    the timed steps (control kernel, FFN; resize calls excluded), the FFN's
    HBM rate, each resize's wall time, occupancy and bytes moved device to
    device, and a checksum of the whole host pool before and after."""
    import ctypes
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch

    import routed_expert_execution_moe_amd as B
    import workload as W

    wl = W.QWEN_ELASTIC
    dev = torch.device("cuda:0")
    points = sorted(wl.resize.items())
    at = {steps * (i + 1) // 4: n for i, (_, n) in enumerate(points)}
    cfg = B.config(wl.L, wl.E, wl.k, wl.H, wl.I, wl.w_dtype, wl.act_dtype, wl.n_slots,
                   max_slots=max([wl.n_slots] + list(wl.resize.values())), max_tokens=wl.T,
                   bw_pcie_mbps=wl.bw_pcie_mbps, bw_host_mbps=wl.bw_host_mbps, timing=1)
    stride = B.moe_expert_bytes(cfg)
    pool_bytes = wl.n_ids * stride
    pool = B.moe_host_pool_alloc(pool_bytes)
    ctx = None
    try:
        W.fill_banks(wl, pool, 0, wl.n_ids)
        pool_np = np.ctypeslib.as_array((ctypes.c_uint8 * pool_bytes).from_address(pool))

        def checksum():
            words = pool_np.view(np.uint64)
            parts = np.array_split(np.arange(len(words)), 16)
            with ThreadPoolExecutor(16) as ex:
                sums = ex.map(lambda r: int(np.add.reduce(words[r[0]:r[-1] + 1], dtype=np.uint64)), parts)
            return sum(sums) & (2 ** 64 - 1)

        logits = W.decode_logits(wl, steps=steps)
        lg_d = torch.from_numpy(np.ascontiguousarray(logits)).to(dev)
        xs = np.stack([np.stack([W.hidden(wl, s, l) for l in range(wl.L)]) for s in range(steps)])
        x_d = torch.from_numpy(xs.view(np.int16)).to(dev).view(torch.bfloat16)
        ids = torch.empty((wl.L, wl.T, wl.k), dtype=torch.int32, device=dev)
        w = torch.empty((wl.L, wl.T, wl.k), dtype=torch.float32, device=dev)
        y = torch.empty((wl.L, wl.T, wl.H), dtype=torch.bfloat16, device=dev)
        ck0 = checksum()
        ctx = B.moe_create(cfg, pool, pool_bytes)
        hiplib = ctypes.CDLL("libamdhip64.so.7")
        hiplib.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]

        def slot_table():
            v = B.moe_plan_view_get(ctx)
            out = np.empty(v.n_slots, np.int32)
            assert hiplib.hipMemcpy(out.ctypes.data, v.slot2id, out.nbytes, 2) == 0
            return out

        resizes, wall, timed_layers = [], 0.0, 0
        tm_sum = None
        st_a = st_b = None
        for s in range(steps):
            if s in at:
                tm_part = B.moe_ctx_timing(ctx, reset=True)  # harvest before the resize
                if s > warmup:
                    tm_sum = tm_part if tm_sum is None else {
                        k: dict(calls=tm_sum[k]["calls"] + v["calls"], ms=tm_sum[k]["ms"] + v["ms"])
                        for k, v in tm_part.items()}
                before = slot_table()
                t0 = time.perf_counter()
                B.moe_cache_resize(ctx, at[s], 60_000)
                ms = (time.perf_counter() - t0) * 1e3
                after = slot_table()
                where = {int(u): i for i, u in enumerate(before) if u >= 0}
                moved = sum(1 for i, u in enumerate(after) if u >= 0 and where[int(u)] != i)
                resizes.append({"before_step": s, "to_slots": at[s], "ms": round(ms, 3),
                                "occupied_before": len(where), "kept": int((after >= 0).sum()),
                                "moved_slots": moved, "moved_bytes_d2d": moved * stride})
            if s == warmup:
                torch.cuda.synchronize()
                B.moe_ctx_timing(ctx, reset=True)
                st_a = B.moe_ctx_stats(ctx)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for l in range(wl.L):
                B.moe_route_topk(ctx, lg_d[s, l], wl.T, ids[l], w[l])
                B.moe_cache_plan(ctx, l, ids[l], wl.T, x_d[s, l])
                B.moe_expert_ffn(ctx, l, x_d[s, l], wl.T)
                B.moe_merge(ctx, w[l], wl.T, y[l])
            torch.cuda.synchronize()
            if s >= warmup:
                wall += time.perf_counter() - t0
                timed_layers += wl.L
        st_b = B.moe_ctx_stats(ctx)
        tm_part = B.moe_ctx_timing(ctx)
        tm = tm_part if tm_sum is None else {
            k: dict(calls=tm_sum[k]["calls"] + v["calls"], ms=tm_sum[k]["ms"] + v["ms"])
            for k, v in tm_part.items()}
        # FFN bytes: the unique GPU-resident experts' weights plus the
        # activations (the fp32 partial rows, at most T*k*H*4 = 64 KB a call,
        # are left out: well under 0.1% of the ~250 MB of weights)
        gpu_experts = (st_b.hits - st_a.hits) + (st_b.fills - st_a.fills)
        ffn_bytes = gpu_experts * W.expert_bytes(wl) + timed_layers * wl.T * wl.H * 2
        per = {k: (round(v["ms"] * 1e3 / v["calls"], 2) if v["calls"] else None) for k, v in tm.items()}
        ffn_gbps = ffn_bytes / (tm["ffn"]["ms"] * 1e-3) / 1e9 if tm["ffn"]["ms"] else None
        acc = (st_b.hits - st_a.hits) + (st_b.fills - st_a.fills) + (st_b.cpu - st_a.cpu)
        return {
            "workload": wl.name, "tokens_per_call": wl.T, "steps": steps, "warmup": warmup,
            "resize_before_steps": sorted(at),
            "us_per_layer": round(wall / max(timed_layers, 1) * 1e6, 2),
            "control_kernel_us": per.get("plan"), "ffn_us": per.get("ffn"), "fill_us": per.get("fill"),
            "merge_us": per.get("merge"), "route_us": per.get("route"),
            "ffn_expert_bytes_per_layer": round(gpu_experts * W.expert_bytes(wl) / max(timed_layers, 1)),
            "ffn_gbps": round(ffn_gbps, 1) if ffn_gbps else None,
            "ffn_frac_of_hbm": round(ffn_gbps / HBM_PEAK_GBPS, 4) if ffn_gbps else None,
            "miss_rate": round(1 - (st_b.hits - st_a.hits) / max(acc, 1), 4),
            "fills_per_layer": round((st_b.fills - st_a.fills) / max(timed_layers, 1), 3),
            "cpu_experts_per_layer": round((st_b.cpu - st_a.cpu) / max(timed_layers, 1), 3),
            "resizes": resizes, "host_pool_unchanged": checksum() == ck0,
        }
    finally:
        if ctx:
            B.moe_destroy(ctx)
        B.moe_host_pool_free(pool)


def bench_mxfp4_decode(steps=60, warmup=8):
    """The DeepSeek-V4-Flash-shaped MXFP4 decode workload (8 of its layers,
    256 experts, 225 slots, one token per call) on its own context and host
    pool: `warmup` untimed steps, then `steps` timed ones with per-phase HIP
    events (control kernel, fill, FFN, merge) and the FFN's HBM rate over the
    same algorithmic bytes as the headline line (unique GPU experts' weights,
    activations, partial rows and the fp32 intermediate)."""
    import numpy as np
    import torch

    import routed_expert_execution_moe_amd as B
    import workload as W

    wl = W.DSV4_MXFP4
    dev = torch.device("cuda:0")
    n_run = warmup + steps
    cfg = B.config(wl.L, wl.E, wl.k, wl.H, wl.I, wl.w_dtype, wl.act_dtype, wl.n_slots,
                   max_tokens=wl.T, bw_pcie_mbps=wl.bw_pcie_mbps, bw_host_mbps=wl.bw_host_mbps,
                   timing=1)
    stride = B.moe_expert_bytes(cfg)
    pool_bytes = wl.n_ids * stride
    pool = B.moe_host_pool_alloc(pool_bytes)
    ctx = None
    try:
        W.fill_banks(wl, pool, 0, wl.n_ids)
        logits = W.decode_logits(wl, steps=n_run)
        lg_d = torch.from_numpy(np.ascontiguousarray(logits)).to(dev)
        xs = np.stack([np.stack([W.hidden(wl, s, l) for l in range(wl.L)]) for s in range(n_run)])
        x_d = torch.from_numpy(xs.view(np.int16)).to(dev).view(torch.bfloat16)
        ids = torch.empty((wl.L, wl.T, wl.k), dtype=torch.int32, device=dev)
        w = torch.empty((wl.L, wl.T, wl.k), dtype=torch.float32, device=dev)
        y = torch.empty((wl.L, wl.T, wl.H), dtype=torch.bfloat16, device=dev)
        ctx = B.moe_create(cfg, pool, pool_bytes)

        def step(s):
            for l in range(wl.L):
                B.moe_route_topk(ctx, lg_d[s, l], wl.T, ids[l], w[l])
                B.moe_cache_plan(ctx, l, ids[l], wl.T, x_d[s, l])
                B.moe_expert_ffn(ctx, l, x_d[s, l], wl.T)
                B.moe_merge(ctx, w[l], wl.T, y[l])

        for s in range(warmup):
            step(s)
        torch.cuda.synchronize()
        B.moe_ctx_timing(ctx, reset=True)
        st_a = B.moe_ctx_stats(ctx)
        t0 = time.perf_counter()
        for s in range(warmup, n_run):
            step(s)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        tm = B.moe_ctx_timing(ctx)
        st_b = B.moe_ctx_stats(ctx)
        calls = steps * wl.L
        gpu_experts = (st_b.hits - st_a.hits) + (st_b.fills - st_a.fills)
        # one token a call: each GPU expert serves one (token, expert) pair
        ffn_bytes = (gpu_experts * W.expert_bytes(wl) + calls * wl.T * wl.H * 2
                     + gpu_experts * (wl.H * 4 + 2 * wl.I * 4))
        per = {k: (round(v["ms"] * 1e3 / v["calls"], 2) if v["calls"] else None) for k, v in tm.items()}
        ffn_gbps = ffn_bytes / (tm["ffn"]["ms"] * 1e-3) / 1e9 if tm["ffn"]["ms"] else None
        acc = gpu_experts + (st_b.cpu - st_a.cpu)
        return {
            "workload": wl.name, "tokens_per_call": wl.T, "steps": steps, "warmup": warmup,
            "us_per_layer": round(wall / calls * 1e6, 2),
            "control_kernel_us": per.get("plan"), "ffn_us": per.get("ffn"), "fill_us": per.get("fill"),
            "merge_us": per.get("merge"), "route_us": per.get("route"),
            "ffn_algorithmic_bytes_per_launch": round(ffn_bytes / calls),
            "ffn_gbps": round(ffn_gbps, 1) if ffn_gbps else None,
            "ffn_frac_of_hbm": round(ffn_gbps / HBM_PEAK_GBPS, 4) if ffn_gbps else None,
            "miss_rate": round(1 - (st_b.hits - st_a.hits) / max(acc, 1), 4),
            "fills_per_layer": round((st_b.fills - st_a.fills) / calls, 3),
            "cpu_experts_per_layer": round((st_b.cpu - st_a.cpu) / calls, 3),
        }
    finally:
        if ctx:
            B.moe_destroy(ctx)
        B.moe_host_pool_free(pool)


def copy_calibration():
    """Four launches of an elementwise kernel (negate) that reads 1 GiB and
    writes 1 GiB of float32: the HBM traffic counters of these launches are
    what a counter reads for a known number of bytes.  Also times (HIP
    events) the same kernel at the decode FFN's size, 72 MB of traffic, and
    a one-element kernel, as references for
    what one short launch reaches between two events on this GPU (also
    with the events the library's timing uses, without a system-scope
    fence)."""
    import torch
    n = 1 << 28
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(4):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    assert float(b[-1]) == -1.0
    out = {"calibration_kernel": "torch.neg float32, 2^28 elements", "bytes_read": n * 4,
           "bytes_written": n * 4, "launches": 4}
    m = 72_000_000 // 8  # elements: 36 MB read + 36 MB written
    srcs = [torch.ones(m, dtype=torch.float32, device="cuda") for _ in range(8)]
    dst = torch.empty(m, dtype=torch.float32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for it in range(200):
        e0.record()
        torch.neg(srcs[it % 8], out=dst)
        e1.record()
        torch.cuda.synchronize()
        if it >= 20:
            ts.append(e0.elapsed_time(e1))
    us = sum(ts) / len(ts) * 1e3
    out["stream_72MB_us"] = round(us, 2)
    out["stream_72MB_gbps"] = round(2 * m * 4 / us / 1e3, 1)

    # the same references timed with the events the library's timing uses
    # (no system-scope fence), on torch's stream: a one-element kernel (the
    # floor of one launch between two events) and the 72 MB negation
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    ev = [ctypes.c_void_p(), ctypes.c_void_p()]
    for e in ev:
        assert hip.hipEventCreateWithFlags(ctypes.byref(e), 0x20000000) == 0  # hipEventDisableSystemFence
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def event_us(fn, reps=200, skip=20):
        t = []
        ms = ctypes.c_float()
        for it in range(reps):
            # a 2 GiB pass first keeps the GPU busy while the host enqueues the
            # events and the kernel, as the decode stream's fill does for the
            # expert FFN, so no host submission latency sits between the events
            torch.neg(a, out=b)
            assert hip.hipEventRecord(ev[0], stream) == 0
            fn(it)
            assert hip.hipEventRecord(ev[1], stream) == 0
            assert hip.hipEventSynchronize(ev[1]) == 0
            assert hip.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1]) == 0
            if it >= skip:
                t.append(ms.value * 1e3)
        return sum(t) / len(t)

    one = torch.zeros(1, dtype=torch.float32, device="cuda")
    out["fenceless_events"] = {
        "queued_behind": "a 2 GiB elementwise pass",
        "one_element_kernel_us": round(event_us(lambda it: one.add_(1.0)), 2),
        "stream_72MB_us": round(event_us(lambda it: torch.neg(srcs[it % 8], out=dst)), 2)}
    out["fenceless_events"]["stream_72MB_frac_of_8TBps"] = round(
        2 * m * 4 / (out["fenceless_events"]["stream_72MB_us"] * 1e-6) / 8e12, 4)
    for e in ev:
        hip.hipEventDestroy(e)
    return out


def cpu_baseline(wl, pool_np, stride, logits, xs, steps_range, budget_s):
    """The oracle as it stands (route, integer plan, fp64 expert FFN, merge),
    on the same calls in order, until the time budget is spent.  Beside it,
    the oracle's plan alone (Python integers, one thread) on every call of
    the warmup and timed steps, timed over the timed steps."""
    import numpy as np

    from oracle import expert as OX, layer as OY, plan as OP
    from oracle.route import route_topk

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    K = OP.victim_bound(wl.T, wl.k, wl.E, wl.n_slots)

    def weights(u):
        return OX.expert_weights(pool_np[u * stride:(u + 1) * stride], wl.w_dtype, wl.H, wl.I)

    # the plan alone, every call from a cold pool
    st = OP.Residency(wl.n_ids, wl.n_slots)
    plan_s, plan_calls = 0.0, 0
    for s in range(steps_range.stop):
        for l in range(wl.L):
            ids, _ = route_topk(logits[s, l], wl.k)
            t = time.perf_counter()
            OP.plan(st, l, ids.tolist(), wl.E, K, wl.bw_pcie_mbps, wl.bw_host_mbps)
            if s >= steps_range.start:
                plan_s += time.perf_counter() - t
                plan_calls += 1

    st = OP.Residency(wl.n_ids, wl.n_slots)
    calls, layer_s = 0, 0.0
    t0 = time.perf_counter()
    for s in steps_range:
        for l in range(wl.L):
            ids, w = route_topk(logits[s, l], wl.k)
            OP.plan(st, l, ids.tolist(), wl.E, K, wl.bw_pcie_mbps, wl.bw_host_mbps)
            x = xs(s, l)
            t = time.perf_counter()
            OY.moe_layer(x, ids, w, l, wl.E, weights)
            layer_s += time.perf_counter() - t
            calls += 1
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return dict(value=round(dt / calls * 1e6, 1), unit="us/layer", cores=cores,
                blas_threads=blas_threads, kind="oracle",
                sample=f"first {calls} layer calls of the timed steps (route, plan, fp64 expert "
                       f"FFN and merge from the pinned host banks; plan state starts cold)",
                plan_us_per_call=round(plan_s / max(plan_calls, 1) * 1e6, 1),
                plan_calls=plan_calls,
                ffn_merge_us_per_call=round(layer_s / max(calls, 1) * 1e6, 1))


def main():
    a = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {a.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import ctypes

    import numpy as np
    import torch

    import routed_expert_execution_moe_amd as B
    import workload as W

    if a.prefill_only:
        print(json.dumps(bench_prefill(a.prefill_main_only, a.prefill_tokens)), flush=True)
        return
    if a.record_traffic:
        kind, fd, wd = a.record_traffic
        # the counter runs were of the default bench: the decode workload the
        # default run times, or the prefill workload of its prefill leg
        wname = W.DSV4_PREFILL.name if kind == "prefill_gemm" else a.workload
        print(json.dumps(record_traffic(kind, wname, fd, wd)), flush=True)
        return
    if a.copy_calibration:
        print(json.dumps(copy_calibration()), flush=True)
        return
    if a.streams_only:
        print(json.dumps(bench_streams()), flush=True)
        return
    wl = {w.name: w for w in W.WORKLOADS}[a.workload]
    assert not wl.prefill, "decode workloads only"
    warmup = a.warmup if a.warmup is not None else min(32, wl.steps // 8)
    steps = a.steps if a.steps is not None else wl.steps - warmup
    assert warmup + steps <= wl.steps, "warmup + steps exceeds the workload's decode steps"
    mode = {"hybrid": B.MOE_HYBRID, "offload": B.MOE_OFFLOAD, "cpu": B.MOE_CPU}[a.mode]
    dev = torch.device("cuda:0")

    t_setup = time.perf_counter()

    def make_cfg(timing):
        return B.config(wl.L, wl.E, wl.k, wl.H, wl.I, wl.w_dtype, wl.act_dtype, wl.n_slots,
                        max_slots=max([wl.n_slots] + list(wl.resize.values())), max_tokens=wl.T,
                        bw_pcie_mbps=wl.bw_pcie_mbps, bw_host_mbps=wl.bw_host_mbps, mode=mode,
                        max_fetch=a.max_fetch, timing=timing)

    stride = B.moe_expert_bytes(make_cfg(0))
    pool_bytes = wl.n_ids * stride
    pool = B.moe_host_pool_alloc(pool_bytes)
    W.fill_banks(wl, pool, 0, wl.n_ids)
    pool_np = np.ctypeslib.as_array((ctypes.c_uint8 * pool_bytes).from_address(pool))
    n_run = warmup + steps
    logits = W.router_logits(wl)[:n_run]
    lg_d = torch.from_numpy(np.ascontiguousarray(logits)).to(dev)           # [S, L, T, E]
    xs_np = np.stack([np.stack([W.hidden(wl, s, l) for l in range(wl.L)]) for s in range(n_run)])
    if wl.act_dtype == "bf16":
        x_d = torch.from_numpy(xs_np.view(np.int16)).to(dev).view(torch.bfloat16)
        act = torch.bfloat16
    else:
        x_d = torch.from_numpy(xs_np).to(dev)
        act = torch.float32
    ids = torch.empty((wl.L, wl.T, wl.k), dtype=torch.int32, device=dev)
    w = torch.empty((wl.L, wl.T, wl.k), dtype=torch.float32, device=dev)
    y = torch.empty((wl.L, wl.T, wl.H), dtype=act, device=dev)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    print(f"# setup {setup_s:.1f} s: {wl.name}, host pool {pool_bytes / 1e9:.2f} GB, "
          f"{wl.n_slots} slots, warmup {warmup} steps, timed {steps} steps", file=sys.stderr,
          flush=True)

    def run(timing, prepare=None):
        """Fresh context (cold cache), warmup steps, then the timed steps.
        `prepare(ctx)` runs once on the fresh context first."""
        ctx = B.moe_create(make_cfg(timing), pool, pool_bytes)
        if prepare is not None:
            prepare(ctx)

        def step(s):
            for l in range(wl.L):
                B.moe_route_topk(ctx, lg_d[s, l], wl.T, ids[l], w[l])
                B.moe_cache_plan(ctx, l, ids[l], wl.T, x_d[s, l])
                B.moe_expert_ffn(ctx, l, x_d[s, l], wl.T)
                B.moe_merge(ctx, w[l], wl.T, y[l])

        try:
            for s in range(warmup):
                step(s)
            torch.cuda.synchronize()
            if timing:
                B.moe_ctx_timing(ctx, reset=True)
            st0 = B.moe_ctx_stats(ctx)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for s in range(warmup, n_run):
                step(s)
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
            tm = B.moe_ctx_timing(ctx) if timing else None
            st1 = B.moe_ctx_stats(ctx)
        finally:
            B.moe_destroy(ctx)
        return dt, tm, st0, st1

    def run_graph():
        """The same steps replayed from one captured HIP graph per step (all
        layers): the step's logits and hidden states are copied into the
        captured buffers, then the graph is launched; the copies are timed."""
        ctx = B.moe_create(make_cfg(0), pool, pool_bytes)
        try:
            lg_s = torch.empty_like(lg_d[0])
            x_s = torch.empty_like(x_d[0])
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for l in range(wl.L):
                    B.moe_route_topk(ctx, lg_s[l], wl.T, ids[l], w[l])
                    B.moe_cache_plan(ctx, l, ids[l], wl.T, x_s[l])
                    B.moe_expert_ffn(ctx, l, x_s[l], wl.T)
                    B.moe_merge(ctx, w[l], wl.T, y[l])
            torch.cuda.synchronize()

            def gstep(s):
                lg_s.copy_(lg_d[s])
                x_s.copy_(x_d[s])
                graph.replay()

            for s in range(warmup):
                gstep(s)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for s in range(warmup, n_run):
                gstep(s)
            torch.cuda.synchronize()
            return time.perf_counter() - t0
        finally:
            B.moe_destroy(ctx)

    # the number: events off; the per-phase breakdown: a second run with events on
    dt, _, st0, st1 = run(0)
    dt_timed, tm, _, _ = run(1)
    dt_graph = run_graph() if not a.no_graph else None
    # the same steps with B_P and B_H measured on this machine and the backend
    # the pages' rule picks for them (instead of the configured numbers)
    measured = {}

    def calibrate(ctx):
        from routed_expert_execution_moe_amd import bw_profile
        prof = bw_profile.measure(ctx, wl.w_dtype, torch.cuda.get_device_name(0), 8, 5, 2.0)
        if a.bw_profile:
            bw_profile.save(a.bw_profile, prof)
        mode_m = B.MOE_HYBRID if prof["backend"] == "hybrid" else B.MOE_OFFLOAD
        B.moe_set_split(ctx, prof["bw_pcie_mbps"], prof["bw_host_mbps"], mode_m)
        measured.update(bw_pcie_mbps=prof["bw_pcie_mbps"], bw_host_mbps=prof["bw_host_mbps"],
                        bw_h2d_mbps=prof["bw_h2d_mbps"], recommended_mode=prof["backend"])

    def run_elastic():
        """The 8-stream workload's resize schedule (37% -> 15% -> 30% -> 30% of
        the pool) applied to a decode context of this workload at a safe point
        between steps: wall time of each moe_cache_resize (synchronous), the
        slots kept and moved (device-to-device compaction), and a checksum of
        the whole host pool before and after (the library never writes it)."""
        from concurrent.futures import ThreadPoolExecutor
        hiplib = ctypes.CDLL("libamdhip64.so.7")
        hiplib.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]

        def slot_table(ctx):
            v = B.moe_plan_view_get(ctx)
            out = np.empty(v.n_slots, np.int32)
            assert hiplib.hipMemcpy(out.ctypes.data, v.slot2id, out.nbytes, 2) == 0
            return out

        def checksum():
            words = pool_np.view(np.uint64)
            parts = np.array_split(np.arange(len(words)), 16)
            with ThreadPoolExecutor(16) as ex:
                sums = ex.map(lambda r: int(np.add.reduce(words[r[0]:r[-1] + 1], dtype=np.uint64)), parts)
            return sum(sums) & (2 ** 64 - 1)

        ck0 = checksum()
        ctx = B.moe_create(make_cfg(0), pool, pool_bytes)
        try:
            def dec(s):
                for l in range(wl.L):
                    B.moe_route_topk(ctx, lg_d[s, l], wl.T, ids[l], w[l])
                    B.moe_cache_plan(ctx, l, ids[l], wl.T, x_d[s, l])
                    B.moe_expert_ffn(ctx, l, x_d[s, l], wl.T)
                    B.moe_merge(ctx, w[l], wl.T, y[l])
            for s in range(min(64, n_run)):
                dec(s)
            torch.cuda.synchronize()
            res = []
            for _, n_new in sorted(W.QWEN_ELASTIC.resize.items()):
                before = slot_table(ctx)
                t0 = time.perf_counter()
                B.moe_cache_resize(ctx, n_new, 60_000)
                ms = (time.perf_counter() - t0) * 1e3
                after = slot_table(ctx)
                where = {int(u): i for i, u in enumerate(before) if u >= 0}
                moved = sum(1 for i, u in enumerate(after) if u >= 0 and where[int(u)] != i)
                res.append({"to_slots": n_new, "ms": round(ms, 3), "occupied_before": len(where),
                            "kept": int((after >= 0).sum()), "moved_slots": moved,
                            "moved_bytes_d2d": moved * stride})
                for s in range(16):
                    dec((64 + 16 * len(res) + s) % n_run)
                torch.cuda.synchronize()
        finally:
            B.moe_destroy(ctx)
        return {"schedule": W.QWEN_ELASTIC.name + " resize points, on this decode context",
                "resizes": res, "host_pool_unchanged": checksum() == ck0}

    if not a.no_calibrated:
        dt_m, _, sm0, sm1 = run(0, calibrate)
        acc_m = (sm1.hits - sm0.hits) + (sm1.fills - sm0.fills) + (sm1.cpu - sm0.cpu)
        measured.update(us_per_layer=round(dt_m / (steps * wl.L) * 1e6, 2),
                        fills_per_layer=round((sm1.fills - sm0.fills) / (steps * wl.L), 3),
                        cpu_experts_per_layer=round((sm1.cpu - sm0.cpu) / (steps * wl.L), 3),
                        miss_rate=round(1 - (sm1.hits - sm0.hits) / max(acc_m, 1), 4))
    elastic = None if a.no_elastic else run_elastic()
    calls = steps * wl.L
    us_per_layer = dt / calls * 1e6
    n_gpu_experts = (st1.hits - st0.hits) + (st1.fills - st0.fills)
    pairs_gpu = n_gpu_experts * wl.T  # upper bound on GPU pairs is n_gpu * T; T == 1 here
    ab = 2 if wl.act_dtype == "bf16" else 4
    ffn_bytes = (n_gpu_experts * W.expert_bytes(wl) + calls * wl.T * wl.H * ab
                 + pairs_gpu * (wl.H * 4 + 2 * wl.I * 4))
    ffn = tm["ffn"]
    ffn_gbps = ffn_bytes / (ffn["ms"] * 1e-3) / 1e9 if ffn["ms"] > 0 else None
    fill_bytes = (st1.fills - st0.fills) * W.expert_bytes(wl)
    fill_gbps = fill_bytes / (tm["fill"]["ms"] * 1e-3) / 1e9 if tm["fill"]["ms"] > 0 else None
    per = {k: (round(v["ms"] * 1e3 / v["calls"], 2) if v["calls"] else None) for k, v in tm.items()}
    accesses = (st1.hits - st0.hits) + (st1.fills - st0.fills) + (st1.cpu - st0.cpu)

    cpu = None
    if not a.no_cpu_baseline:
        def xs(s, l):
            x = xs_np[s, l]
            return W.bf16_bits_to_f32(x).astype(np.float64) if wl.act_dtype == "bf16" \
                else x.astype(np.float64)
        cpu = cpu_baseline(wl, pool_np, stride, logits, xs, range(warmup, n_run),
                           a.cpu_baseline_seconds)

    out = {
        "metric": METRIC,
        "value": round(us_per_layer, 2),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(dt / steps * 1e3, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.w_dtype == "bf16" else wl.w_dtype,
        "data": "synthetic (seeded Philox weights N(0,0.02), Zipf routing with reuse; no checkpoint)",
        "config": {"workload": wl.name, "layers": wl.L, "experts": wl.E, "top_k": wl.k,
                   "hidden": wl.H, "inter": wl.I, "slots": wl.n_slots, "tokens_per_call": wl.T,
                   "mode": a.mode, "bw_pcie_mbps": wl.bw_pcie_mbps,
                   "bw_host_mbps": wl.bw_host_mbps, "max_fetch": a.max_fetch},
        "roofline": {
            "bound": "hbm",
            "kernel": "expert FFN (gate/up GEMV + down GEMV over the unique GPU-resident experts)",
            "achieved": round(ffn_gbps, 1) if ffn_gbps else None,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(ffn_gbps / HBM_PEAK_GBPS, 4) if ffn_gbps else None,
            "traffic": recorded_traffic("decode_ffn", wl.name),
            "traffic_source": traffic_source("decode_ffn", wl.name),
            "algorithmic_bytes_per_launch": round(ffn_bytes / calls),
            "timing": "HIP events bound to each FFN launch's dispatch (hipExtLaunchKernelGGL start and stop "
                      "events): the kernel's own start to end on its stream, averaged over the timed steps",
        },
        "cpu_baseline": cpu,
        "breakdown_us_per_call": per,
        "breakdown_run_us_per_layer": round(dt_timed / (steps * wl.L) * 1e6, 2),
        "calibrated_split": measured or None,
        "graph": ({"us_per_layer": round(dt_graph / (steps * wl.L) * 1e6, 2),
                   "note": "one captured HIP graph per step (all layers), inputs copied into its "
                           "buffers inside the timed region"} if dt_graph else None),
        "control_kernel_us": per.get("plan"),
        "ffn_us_per_layer": per.get("ffn"),
        "ffn_bytes_per_layer": round(ffn_bytes / calls),
        "fill_pcie_gbps": round(fill_gbps, 1) if fill_gbps else None,
        "miss_rate": round(1 - (st1.hits - st0.hits) / max(accesses, 1), 4),
        "fills_per_layer": round((st1.fills - st0.fills) / calls, 3),
        "cpu_experts_per_layer": round((st1.cpu - st0.cpu) / calls, 3),
        "elastic_resize": elastic,
    }
    pool_np = None
    B.moe_host_pool_free(pool)
    if not a.no_streams:
        out["streams_8"] = bench_streams()
    if not a.no_mxfp4:
        out["mxfp4_decode"] = bench_mxfp4_decode()
    if not a.no_prefill:
        out.update(bench_prefill())
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
