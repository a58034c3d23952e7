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
per launch over its HIP-event duration), a per-phase breakdown and the CPU
oracle timed on a bounded sample of the same calls.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer decode µs/layer + expert-FFN HBM GB/s (% of peak); prefill TFLOP/s"
HBM_PEAK_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="qwen3.6-35b-a3b-shape-bf16-decode")
    ap.add_argument("--mode", default="hybrid", choices=["hybrid", "offload", "cpu"])
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def cpu_baseline(wl, pool_np, stride, logits, xs, steps_range, budget_s):
    """The oracle as it stands (route, integer plan, fp64 expert FFN, merge),
    on the same calls in order, until the time budget is spent."""
    import numpy as np

    from oracle import expert as OX, layer as OY, plan as OP
    from oracle.route import route_topk

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = 1
    st = OP.Residency(wl.n_ids, wl.n_slots)
    K = OP.victim_bound(wl.T, wl.k, wl.E, wl.n_slots)

    def weights(u):
        return OX.expert_weights(pool_np[u * stride:(u + 1) * stride], wl.w_dtype, wl.H, wl.I)

    calls = 0
    t0 = time.perf_counter()
    for s in steps_range:
        for l in range(wl.L):
            ids, w = route_topk(logits[s, l], wl.k)
            OP.plan(st, l, ids.tolist(), wl.E, K, wl.bw_pcie_mbps, wl.bw_host_mbps)
            x = xs(s, l)
            OY.moe_layer(x, ids, w, l, wl.E, weights)
            calls += 1
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return dict(value=round(dt / calls * 1e6, 1), unit="us/layer", cores=blas_threads,
                kind="oracle",
                sample=f"first {calls} layer calls of the timed steps (route, plan, fp64 expert "
                       f"FFN and merge from the pinned host banks; plan state starts cold)")


def main():
    a = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {a.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import ctypes

    import numpy as np
    import torch

    import routed_expert_execution_moe_amd as B
    import workload as W

    wl = {w.name: w for w in W.WORKLOADS}[a.workload]
    assert not wl.prefill, "decode workloads only"
    warmup = a.warmup if a.warmup is not None else min(32, wl.steps // 8)
    steps = a.steps if a.steps is not None else wl.steps - warmup
    assert warmup + steps <= wl.steps, "warmup + steps exceeds the workload's decode steps"
    mode = {"hybrid": B.MOE_HYBRID, "offload": B.MOE_OFFLOAD, "cpu": B.MOE_CPU}[a.mode]
    dev = torch.device("cuda:0")

    t_setup = time.perf_counter()
    cfg = B.config(wl.L, wl.E, wl.k, wl.H, wl.I, wl.w_dtype, wl.act_dtype, wl.n_slots,
                   max_slots=max([wl.n_slots] + list(wl.resize.values())), max_tokens=wl.T,
                   bw_pcie_mbps=wl.bw_pcie_mbps, bw_host_mbps=wl.bw_host_mbps, mode=mode,
                   timing=1)
    stride = B.moe_expert_bytes(cfg)
    pool_bytes = wl.n_ids * stride
    pool = B.moe_host_pool_alloc(pool_bytes)
    W.fill_banks(wl, pool, 0, wl.n_ids)
    pool_np = np.ctypeslib.as_array((ctypes.c_uint8 * pool_bytes).from_address(pool))
    ctx = B.moe_create(cfg, pool, pool_bytes)
    n_run = warmup + steps
    logits = W.router_logits(wl)[:n_run]
    lg_d = torch.from_numpy(np.ascontiguousarray(logits)).to(dev)           # [S, L, T, E]
    if wl.act_dtype == "bf16":
        xs_np = np.stack([np.stack([W.hidden(wl, s, l) for l in range(wl.L)]) for s in range(n_run)])
        x_d = torch.from_numpy(xs_np.view(np.int16)).to(dev).view(torch.bfloat16)
        act = torch.bfloat16
    else:
        xs_np = np.stack([np.stack([W.hidden(wl, s, l) for l in range(wl.L)]) for s in range(n_run)])
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
    st0 = B.moe_ctx_stats(ctx)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(warmup, n_run):
        step(s)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    tm = B.moe_ctx_timing(ctx)
    st1 = B.moe_ctx_stats(ctx)

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
                   "bw_host_mbps": wl.bw_host_mbps},
        "roofline": {
            "bound": "hbm",
            "kernel": "expert FFN (gate/up GEMV + down GEMV over the unique GPU-resident experts)",
            "achieved": round(ffn_gbps, 1) if ffn_gbps else None,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(ffn_gbps / HBM_PEAK_GBPS, 4) if ffn_gbps else None,
            "traffic": None,
        },
        "cpu_baseline": cpu,
        "breakdown_us_per_call": per,
        "control_kernel_us": per.get("plan"),
        "ffn_us_per_layer": per.get("ffn"),
        "ffn_bytes_per_layer": round(ffn_bytes / calls),
        "fill_pcie_gbps": round(fill_gbps, 1) if fill_gbps else None,
        "miss_rate": round(1 - (st1.hits - st0.hits) / max(accesses, 1), 4),
        "fills_per_layer": round((st1.fills - st0.fills) / calls, 3),
        "cpu_experts_per_layer": round((st1.cpu - st0.cpu) / calls, 3),
        "prefill_tflops": None,
    }
    print(json.dumps(out), flush=True)
    B.moe_destroy(ctx)
    pool_np = None
    B.moe_host_pool_free(pool)


if __name__ == "__main__":
    main()
