"""ctypes binding of libmoert.so: the C-ABI calls under the same names.

Argument marshalling only: tensors become device pointers, torch streams
become hipStream_t handles, statuses become exceptions.  Every step of the
MoE layer runs in the library's HIP kernels and host code.  torch is imported
first so the library binds to the HIP runtime torch already loaded (both
carry the SONAME libamdhip64.so.7): one runtime per process.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the process's HIP runtime before libmoert)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoert.so")

MOE_OK, MOE_EINVAL, MOE_ENOMEM, MOE_ENOSPC, MOE_EHIP, MOE_EBUSY, MOE_ETIMEDOUT, \
    MOE_EUNSUPPORTED = 0, -1, -2, -3, -4, -5, -6, -7
MOE_F32, MOE_BF16, MOE_MXFP4 = 0, 1, 2
MOE_HYBRID, MOE_OFFLOAD, MOE_CPU = 0, 1, 2
DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "mxfp4": MOE_MXFP4}


class MoeConfig(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("w_dtype", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("n_slots", ctypes.c_int32), ("max_slots", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("bw_pcie_mbps", ctypes.c_int64),
                ("bw_host_mbps", ctypes.c_int64), ("max_fetch", ctypes.c_int32),
                ("mode", ctypes.c_int32), ("cpu_threads", ctypes.c_int32),
                ("max_prefill_tokens", ctypes.c_int32), ("timing", ctypes.c_int32)]


class PlanCounts(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n_uniq", "n_hit", "n_miss", "q", "n_cpu", "n_gpu", "K", "tick_lo")]


class PlanView(ctypes.Structure):
    _fields_ = [("counts", ctypes.c_void_p), ("uniq", ctypes.c_void_p), ("hits", ctypes.c_void_p),
                ("misses", ctypes.c_void_p), ("victims", ctypes.c_void_p),
                ("fill_u", ctypes.c_void_p), ("fill_slot", ctypes.c_void_p),
                ("fill_old", ctypes.c_void_p), ("cpu_u", ctypes.c_void_p),
                ("gpu_u", ctypes.c_void_p), ("gpu_slot", ctypes.c_void_p),
                ("slot_map", ctypes.c_void_p), ("id2slot", ctypes.c_void_p),
                ("slot2id", ctypes.c_void_p), ("slot_ts", ctypes.c_void_p),
                ("tick", ctypes.c_void_p), ("p_gpu", ctypes.c_void_p), ("p_cpu", ctypes.c_void_p),
                ("slot_base", ctypes.c_void_p), ("n_slots", ctypes.c_int32),
                ("max_slots", ctypes.c_int32), ("umax", ctypes.c_int32), ("kmax", ctypes.c_int32),
                ("h_marked", ctypes.c_void_p)]


class PrefillView(ctypes.Structure):
    _fields_ = [("counts", ctypes.c_void_p), ("offsets", ctypes.c_void_p), ("perm", ctypes.c_void_p),
                ("tiles", ctypes.c_void_p), ("hmid", ctypes.c_void_p), ("prow", ctypes.c_void_p),
                ("n_experts", ctypes.c_int32), ("max_pairs", ctypes.c_int32),
                ("max_tiles", ctypes.c_int32)]


class Stats(ctypes.Structure):
    _fields_ = [("n_slots", ctypes.c_int32), ("occupied", ctypes.c_int32),
                ("plans", ctypes.c_int64), ("hits", ctypes.c_int64), ("fills", ctypes.c_int64),
                ("cpu", ctypes.c_int64), ("evictions", ctypes.c_int64),
                ("prefill_layers", ctypes.c_int64), ("resizes", ctypes.c_int64),
                ("prefill_h2d_experts", ctypes.c_int64), ("prefill_d2d_experts", ctypes.c_int64)]


PHASES = ("route", "plan", "fill", "ffn", "merge", "host", "prefill_copy", "prefill_group",
          "prefill_gemm", "prefill_merge")


class Timing(ctypes.Structure):
    _fields_ = [("calls", ctypes.c_int64 * len(PHASES)), ("ms", ctypes.c_double * len(PHASES))]

    def as_dict(self):
        return {p: dict(calls=self.calls[i], ms=self.ms[i]) for i, p in enumerate(PHASES)}


class MoertError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({_strerror(status)}): {detail}")


_lib = None


def lib():
    """Load libmoert.so; fails loudly when the HIP library has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m routed_expert_execution_moe_amd.build or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        cfgp = ctypes.POINTER(MoeConfig)
        sig = {
            "moe_expert_bytes": ([cfgp], sz),
            "moe_host_pool_alloc": ([sz, ctypes.POINTER(vp)], i32),
            "moe_host_pool_free": ([vp], i32),
            "moe_create": ([cfgp, vp, sz, ctypes.POINTER(vp)], i32),
            "moe_destroy": ([vp], i32),
            "moe_route_topk": ([vp, vp, i32, vp, vp, vp], i32),
            "moe_cache_plan": ([vp, i32, vp, i32, vp, vp], i32),
            "moe_expert_ffn": ([vp, i32, vp, i32, vp], i32),
            "moe_merge": ([vp, vp, i32, vp, vp], i32),
            "moe_cache_resize": ([vp, i32, i32], i32),
            "moe_measure_bandwidth": ([vp, i32, i32, ctypes.POINTER(i64), ctypes.POINTER(i64),
                                      ctypes.POINTER(i64)], i32),
            "moe_recommend_mode": ([i64, i64, ctypes.c_double, ctypes.POINTER(i32)], i32),
            "moe_set_split": ([vp, i64, i64, i32], i32),
            "moe_prefill_set_buffers": ([vp, i32], i32),
            "moe_set_cpu_layers": ([vp, ctypes.POINTER(ctypes.c_uint8), i32], i32),
            "moe_prefill_layer": ([vp, i32, vp, i32, vp, vp, vp, vp], i32),
            "moe_prefill_layer_noalloc": ([vp, i32, vp, i32, vp, vp, vp, vp], i32),
            "moe_plan_view_get": ([vp, ctypes.POINTER(PlanView)], i32),
            "moe_prefill_view_get": ([vp, ctypes.POINTER(PrefillView)], i32),
            "moe_ctx_stats": ([vp, ctypes.POINTER(Stats)], i32),
            "moe_ctx_timing": ([vp, ctypes.POINTER(Timing), i32], i32),
            "moe_strerror": ([i32], ctypes.c_char_p),
            "moe_last_error": ([], ctypes.c_char_p),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _strerror(s: int) -> str:
    return lib().moe_strerror(s).decode()


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoertError(status, where, lib().moe_last_error().decode())


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s) -> int | None:
    if s is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def config(L, E, k, H, I, w_dtype, act_dtype, n_slots, max_slots=None, max_tokens=1,
           bw_pcie_mbps=1, bw_host_mbps=1, max_fetch=0, mode=MOE_HYBRID, cpu_threads=0,
           max_prefill_tokens=0, timing=0) -> MoeConfig:
    return MoeConfig(L, E, k, H, I, DTYPES.get(w_dtype, w_dtype), DTYPES.get(act_dtype, act_dtype),
                     n_slots, n_slots if max_slots is None else max_slots, max_tokens,
                     bw_pcie_mbps, bw_host_mbps, max_fetch, mode, cpu_threads, max_prefill_tokens,
                     timing)


# ------------------------------------------------------------------ the C-ABI calls
def moe_expert_bytes(cfg: MoeConfig) -> int:
    return lib().moe_expert_bytes(ctypes.byref(cfg))


def moe_host_pool_alloc(nbytes: int) -> int:
    p = ctypes.c_void_p()
    _check(lib().moe_host_pool_alloc(nbytes, ctypes.byref(p)), "moe_host_pool_alloc")
    return p.value


def moe_host_pool_free(addr: int) -> None:
    _check(lib().moe_host_pool_free(addr), "moe_host_pool_free")


def moe_create(cfg: MoeConfig, host_pool: int, host_pool_bytes: int) -> int:
    out = ctypes.c_void_p()
    _check(lib().moe_create(ctypes.byref(cfg), host_pool, host_pool_bytes, ctypes.byref(out)),
           "moe_create")
    return out.value


def moe_destroy(ctx: int) -> None:
    _check(lib().moe_destroy(ctx), "moe_destroy")


def moe_route_topk(ctx, logits, T, ids, w, stream=None):
    _check(lib().moe_route_topk(ctx, _ptr(logits), T, _ptr(ids), _ptr(w), _stream(stream)),
           "moe_route_topk")


def moe_cache_plan(ctx, layer, ids, T, x, stream=None):
    _check(lib().moe_cache_plan(ctx, layer, _ptr(ids), T, _ptr(x), _stream(stream)),
           "moe_cache_plan")


def moe_expert_ffn(ctx, layer, x, T, stream=None):
    _check(lib().moe_expert_ffn(ctx, layer, _ptr(x), T, _stream(stream)), "moe_expert_ffn")


def moe_merge(ctx, w, T, y, stream=None):
    _check(lib().moe_merge(ctx, _ptr(w), T, _ptr(y), _stream(stream)), "moe_merge")


def moe_cache_resize(ctx, new_n_slots, timeout_ms=300_000):
    _check(lib().moe_cache_resize(ctx, new_n_slots, timeout_ms), "moe_cache_resize")


def moe_measure_bandwidth(ctx, n_experts=8, reps=5, h2d=False):
    """(B_P, B_H) in MB/s, measured on the context's expert shape; with
    h2d=True also the pinned host-to-device copy rate: (B_P, B_H, B_H2D)."""
    bp, bh, bc = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib().moe_measure_bandwidth(ctx, n_experts, reps, ctypes.byref(bp), ctypes.byref(bh),
                                       ctypes.byref(bc) if h2d else None), "moe_measure_bandwidth")
    return (bp.value, bh.value, bc.value) if h2d else (bp.value, bh.value)


def moe_recommend_mode(bw_pcie_mbps, bw_host_mbps, threshold=2.0):
    m = ctypes.c_int32()
    _check(lib().moe_recommend_mode(bw_pcie_mbps, bw_host_mbps, threshold, ctypes.byref(m)),
           "moe_recommend_mode")
    return m.value


def moe_set_cpu_layers(ctx, flags):
    """flags: sequence of L truthy values (layers that decode on the host), or None."""
    if flags is None:
        _check(lib().moe_set_cpu_layers(ctx, None, 0), "moe_set_cpu_layers")
        return
    arr = (ctypes.c_uint8 * len(flags))(*[1 if f else 0 for f in flags])
    _check(lib().moe_set_cpu_layers(ctx, arr, len(flags)), "moe_set_cpu_layers")


def moe_set_split(ctx, bw_pcie_mbps, bw_host_mbps, mode):
    _check(lib().moe_set_split(ctx, bw_pcie_mbps, bw_host_mbps, mode), "moe_set_split")


def moe_prefill_set_buffers(ctx, n_buffers):
    _check(lib().moe_prefill_set_buffers(ctx, n_buffers), "moe_prefill_set_buffers")


def moe_prefill_layer(ctx, layer, x, T, ids, w, y, stream=None):
    _check(lib().moe_prefill_layer(ctx, layer, _ptr(x), T, _ptr(ids), _ptr(w), _ptr(y),
                                   _stream(stream)), "moe_prefill_layer")


def moe_prefill_layer_noalloc(ctx, layer, x, T, ids, w, y, stream=None):
    _check(lib().moe_prefill_layer_noalloc(ctx, layer, _ptr(x), T, _ptr(ids), _ptr(w), _ptr(y),
                                           _stream(stream)), "moe_prefill_layer_noalloc")


def moe_plan_view_get(ctx) -> PlanView:
    v = PlanView()
    _check(lib().moe_plan_view_get(ctx, ctypes.byref(v)), "moe_plan_view_get")
    return v


def moe_prefill_view_get(ctx) -> PrefillView:
    v = PrefillView()
    _check(lib().moe_prefill_view_get(ctx, ctypes.byref(v)), "moe_prefill_view_get")
    return v


def moe_ctx_stats(ctx) -> Stats:
    s = Stats()
    _check(lib().moe_ctx_stats(ctx, ctypes.byref(s)), "moe_ctx_stats")
    return s


def moe_ctx_timing(ctx, reset=False) -> dict:
    t = Timing()
    _check(lib().moe_ctx_timing(ctx, ctypes.byref(t), 1 if reset else 0), "moe_ctx_timing")
    return t.as_dict()


def moe_strerror(status: int) -> str:
    return _strerror(status)


def moe_last_error() -> str:
    return lib().moe_last_error().decode()
