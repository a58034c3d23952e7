"""Drivers that run one workload through the HIP library and through the
oracle side by side, for the GPU parity tests."""
from __future__ import annotations

import ctypes
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import workload as W
from oracle import expert as OX, layer as OY, plan as OP
from oracle.route import route_topk

_hip = None


def hip():
    """The process's HIP runtime (the one torch loaded), for raw copies."""
    global _hip
    if _hip is None:
        import torch  # noqa: F401
        _hip = ctypes.CDLL("libamdhip64.so.7")
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        _hip.hipMemcpy.restype = ctypes.c_int
    return _hip


def h2d(ptr: int, arr: np.ndarray) -> None:
    a = np.ascontiguousarray(arr)
    if a.nbytes:
        rc = hip().hipMemcpy(ptr, a.ctypes.data, a.nbytes, 1)
        assert rc == 0, f"hipMemcpy H2D failed: {rc}"


def d2h(ptr: int, count: int, dtype) -> np.ndarray:
    out = np.empty(count, dtype)
    if count:
        rc = hip().hipMemcpy(out.ctypes.data, ptr, out.nbytes, 2)
        assert rc == 0, f"hipMemcpy D2H failed: {rc}"
    return out


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class DeviceRun:
    """One context on cuda:0 with the workload's host pool."""

    def __init__(self, wl: W.Workload, mode=0, n_slots=None, max_slots=None, cpu_threads=0,
                 max_tokens=None, max_prefill_tokens=0, max_fetch=0):
        import torch
        import routed_expert_execution_moe_amd as B
        self.B, self.torch, self.wl = B, torch, wl
        n_slots = wl.n_slots if n_slots is None else n_slots
        max_slots = max(n_slots, max(wl.resize.values(), default=0)) if max_slots is None else max_slots
        self.cfg = B.config(wl.L, wl.E, wl.k, wl.H, wl.I, wl.w_dtype, wl.act_dtype, n_slots,
                            max_slots=max_slots, max_tokens=wl.T if max_tokens is None else max_tokens,
                            bw_pcie_mbps=wl.bw_pcie_mbps, bw_host_mbps=wl.bw_host_mbps,
                            max_fetch=max_fetch, mode=mode, cpu_threads=cpu_threads,
                            max_prefill_tokens=max_prefill_tokens)
        self.stride = B.moe_expert_bytes(self.cfg)
        assert self.stride == W.slot_stride(wl)
        self.pool_bytes = wl.n_ids * self.stride
        self.pool = B.moe_host_pool_alloc(self.pool_bytes)
        W.fill_banks(wl, self.pool, 0, wl.n_ids)
        self.pool_np = np.ctypeslib.as_array(
            (ctypes.c_uint8 * self.pool_bytes).from_address(self.pool))
        self.ctx = B.moe_create(self.cfg, self.pool, self.pool_bytes)
        self.dev = torch.device("cuda:0")
        act = torch.float32 if wl.act_dtype == "f32" else torch.bfloat16
        self.act = act
        T = wl.T
        self.ids = torch.empty((T, wl.k), dtype=torch.int32, device=self.dev)
        self.w = torch.empty((T, wl.k), dtype=torch.float32, device=self.dev)
        self.y = torch.empty((T, wl.H), dtype=act, device=self.dev)

    def bank(self, u: int) -> np.ndarray:
        return self.pool_np[u * self.stride:(u + 1) * self.stride]

    def to_dev_x(self, x: np.ndarray):
        t = self.torch.from_numpy(np.ascontiguousarray(x))
        if self.wl.act_dtype == "bf16":
            t = t.view(self.torch.int16).to(self.dev).view(self.torch.bfloat16)
        else:
            t = t.to(self.dev)
        return t

    def y_f64(self) -> np.ndarray:
        y = self.y
        if self.wl.act_dtype == "bf16":
            y = y.float()
        return y.cpu().numpy().astype(np.float64)

    def decode_call(self, layer, logits: np.ndarray, x: np.ndarray):
        B, torch = self.B, self.torch
        T = logits.shape[0]
        lg = torch.from_numpy(np.ascontiguousarray(logits)).to(self.dev)
        xd = self.to_dev_x(x)
        ids, w, y = self.ids[:T], self.w[:T], self.y[:T]
        B.moe_route_topk(self.ctx, lg, T, ids, w)
        B.moe_cache_plan(self.ctx, layer, ids, T, xd)
        B.moe_expert_ffn(self.ctx, layer, xd, T)
        B.moe_merge(self.ctx, w, T, y)
        torch.cuda.synchronize()
        return ids.cpu().numpy(), w.cpu().numpy().astype(np.float64)

    def plan_view(self, T):
        v = self.B.moe_plan_view_get(self.ctx)
        c = d2h(v.counts, 8, np.int32)
        names = ("n_uniq", "n_hit", "n_miss", "q", "n_cpu", "n_gpu", "K", "tick_lo")
        cnt = dict(zip(names, c.tolist()))
        out = dict(counts=cnt)
        out["uniq"] = d2h(v.uniq, cnt["n_uniq"], np.int32).tolist()
        out["hits"] = d2h(v.hits, cnt["n_hit"], np.int32).tolist()
        out["misses"] = d2h(v.misses, cnt["n_miss"], np.int32).tolist()
        out["victims"] = d2h(v.victims, cnt["K"], np.int32).tolist()
        q = cnt["q"]
        out["fills"] = list(zip(d2h(v.fill_u, q, np.int32).tolist(),
                                d2h(v.fill_slot, q, np.int32).tolist(),
                                d2h(v.fill_old, q, np.int32).tolist()))
        out["cpu"] = d2h(v.cpu_u, cnt["n_cpu"], np.int32).tolist()
        out["gpu"] = list(zip(d2h(v.gpu_u, cnt["n_gpu"], np.int32).tolist(),
                              d2h(v.gpu_slot, cnt["n_gpu"], np.int32).tolist()))
        out["slot_map"] = d2h(v.slot_map, T * self.wl.k, np.int32).reshape(T, self.wl.k).tolist()
        out["n_slots"] = v.n_slots
        return out

    def tables(self):
        v = self.B.moe_plan_view_get(self.ctx)
        n = v.n_slots
        return (d2h(v.id2slot, self.wl.n_ids, np.int32).tolist(),
                d2h(v.slot2id, n, np.int32).tolist(),
                d2h(v.slot_ts, n, np.int64).tolist(),
                int(d2h(v.tick, 1, np.int64)[0]))

    def slot_bytes(self, s: int) -> np.ndarray:
        v = self.B.moe_plan_view_get(self.ctx)
        return d2h(v.slot_base + s * self.stride, self.stride, np.uint8)

    def p_gpu_rows(self, T):
        v = self.B.moe_plan_view_get(self.ctx)
        return d2h(v.p_gpu, T * self.wl.k * self.wl.H, np.float32).reshape(T, self.wl.k, self.wl.H)

    def prefill_grouping(self, T):
        """(counts, offsets[E+1], n_tiles, perm, tiles) of the last prefill
        layer, read back from the device."""
        v = self.B.moe_prefill_view_get(self.ctx)
        E, Tk = self.wl.E, T * self.wl.k
        counts = d2h(v.counts, E, np.int32)
        off = d2h(v.offsets, E + 2, np.int32)
        n_tiles = int(off[E + 1])
        return counts, off[:E + 1], n_tiles, d2h(v.perm, Tk, np.int32), d2h(v.tiles, n_tiles, np.int32)

    def close(self):
        if getattr(self, "ctx", None):
            self.B.moe_destroy(self.ctx)
            self.ctx = None
        if getattr(self, "pool", None):
            self.pool_np = None
            self.B.moe_host_pool_free(self.pool)
            self.pool = None


def oracle_threads() -> int:
    """Threads for decoding expert banks: the host cores this process may
    use, at most 16 (the GPU machine's CPU share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


class WindowedWeights:
    """weights_of(u) for a known order of calls: the next `window` experts of
    `order` are decoded ahead on a thread pool (numpy releases the GIL while
    it converts), each handed out once.  Only the scheduling is parallel; the
    decoding is the oracle's own expert_weights."""

    def __init__(self, order, decode, window=None, pool=None):
        self.order = list(order)
        self.decode = decode
        self.window = window or 2 * oracle_threads()
        self.pool = pool
        self.futs = {}
        self.next = 0
        self._fill()

    def _fill(self):
        while self.next < len(self.order) and len(self.futs) < self.window:
            u = self.order[self.next]
            self.futs[u] = self.pool.submit(self.decode, u)
            self.next += 1

    def __call__(self, u):
        f = self.futs.pop(u, None)
        w = self.decode(u) if f is None else f.result()
        self._fill()
        return w


class OracleRun:
    """The oracle's state machine for the same workload."""

    def __init__(self, wl: W.Workload, weights_source, mode=0, n_slots=None, max_fetch=0,
                 max_tokens=None):
        self.wl = wl
        self.mode = mode
        self.max_fetch = max_fetch
        self.max_tokens = wl.T if max_tokens is None else max_tokens
        n = wl.n_slots if n_slots is None else n_slots
        self.st = OP.Residency(wl.n_ids, n)
        self.K = OP.victim_bound(self.max_tokens, wl.k, wl.E, n, max_fetch)
        self._src = weights_source
        self._cache = {}

    def weights(self, u):
        w = self._cache.get(u)
        if w is None:
            w = OX.expert_weights(self._src(u), self.wl.w_dtype, self.wl.H, self.wl.I)
            if len(self._cache) > 64:
                self._cache.clear()
            self._cache[u] = w
        return w

    def route(self, logits):
        return route_topk(logits, self.wl.k)

    def plan(self, layer, ids):
        return OP.plan(self.st, layer, ids.tolist(), self.wl.E, self.K, self.wl.bw_pcie_mbps,
                       self.wl.bw_host_mbps, self.mode, self.max_fetch)

    def resize(self, n_new):
        moves = OP.resize(self.st, n_new)
        self.K = OP.victim_bound(self.max_tokens, self.wl.k, self.wl.E, n_new, self.max_fetch)
        return moves

    def decode_weights(self, u):
        return OX.expert_weights(self._src(u), self.wl.w_dtype, self.wl.H, self.wl.I)

    def output(self, layer, x, ids, w):
        """The fp64 MoE-layer output; the experts are decoded ahead in the
        order the oracle's layer evaluation asks for them (ascending e)."""
        order = [layer * self.wl.E + e for e in sorted(set(np.asarray(ids).ravel().tolist()))]
        if len(order) <= 1:
            return OY.moe_layer(x, ids, w, layer, self.wl.E, self.weights)
        with ThreadPoolExecutor(oracle_threads()) as pool:
            ww = WindowedWeights(order, self.decode_weights, pool=pool)
            return OY.moe_layer(x, ids, w, layer, self.wl.E, ww)


def x_f64(wl, x):
    if wl.act_dtype == "bf16":
        return W.bf16_bits_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


def compare_plan(gp: dict, op, T):
    """Bit-exact comparison of every plan output."""
    c = gp["counts"]
    assert c["n_uniq"] == len(op.uniq) and gp["uniq"] == op.uniq
    assert gp["hits"] == op.hits, (gp["hits"], op.hits)
    assert gp["misses"] == op.misses
    assert c["q"] == op.q, (c, op.q)
    assert gp["victims"] == op.victims, (gp["victims"], op.victims)
    assert gp["fills"] == [tuple(f) for f in op.fills], (gp["fills"], op.fills)
    assert gp["cpu"] == op.cpu
    assert gp["gpu"] == [tuple(g) for g in op.gpu]
    assert gp["slot_map"] == op.slot_map
    assert c["tick_lo"] == ((op.tick + 2**31) % 2**32) - 2**31  # low 32 bits, signed


def check_grouping(g, ids, E, T, tile_rows=128):
    """The GPU's grouping of the prefill layer's T*k pairs against the
    oracle's (oracle.layer.group_by_expert): per-expert counts and offsets
    bit-exact; the pairs at each expert's positions are exactly that expert's
    pairs (order inside an expert is free: every output row is computed on its
    own); the M-tile list covers each expert's rows once, in order."""
    from oracle import layer as OY
    counts, off, n_tiles, perm, tiles = g.prefill_grouping(T)
    c_o, off_o, perm_o = OY.group_by_expert(ids, E)
    assert np.array_equal(counts, c_o)
    assert np.array_equal(off, off_o)
    assert np.array_equal(np.sort(perm), np.arange(ids.size))  # a permutation of the pairs
    expert_at = np.repeat(np.arange(E), c_o)                  # expert of each position
    assert np.array_equal(np.asarray(ids).ravel()[perm], expert_at)
    want = []
    for e in range(E):
        for m in range((int(c_o[e]) + tile_rows - 1) // tile_rows):
            half = int(c_o[e]) - m * tile_rows <= tile_rows // 2
            want.append((e << 20) | ((m * tile_rows // 64) << 1) | int(half))
    assert n_tiles == len(want) and tiles.tolist() == want
    return c_o


def rel_err(y_gpu, y_ref):
    """max |y_gpu - y_ref| / RMS(y_ref), per token row (each row is one
    stream's MoE-layer output), maximised over rows."""
    y_gpu = np.atleast_2d(y_gpu)
    y_ref = np.atleast_2d(y_ref)
    rms = np.sqrt(np.mean(y_ref ** 2, axis=1))
    err = np.max(np.abs(y_gpu - y_ref), axis=1) / np.maximum(rms, 1e-300)
    return float(err.max()), float(rms.min())


def bf16_round_err(y_ref):
    """The part of rel_err that rounding the exact output to bfloat16 alone
    already causes (round-to-nearest-even on the fp64 -> fp32 value)."""
    y32 = np.atleast_2d(y_ref).astype(np.float32)
    u = y32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    yb = u.astype(np.uint32).view(np.float32).astype(np.float64)
    return rel_err(yb, y_ref)[0]
