"""Seeded synthetic inputs shared by the oracle, the tests, smoke() and bench.py.

This package draws numbers and lays them out; it contains no step of the MoE
method (no routing decision, cache policy, expert arithmetic or merge).  The
random source is the Philox4x32-10 counter-based generator in ``gen.c``; each
tensor is addressed by (root seed, tag, id b, id c) so it can be regenerated
alone.

Tags (the ``a`` id of a Philox stream):
  1  expert weights     (1, flat expert id u, matrix 0 gate / 1 up / 2 down)
  2  hidden states      (2, step, layer)      T*H normals
  3  routing noise      (3, step, layer)      T*E uniforms -> Gumbel(0,1)
  4  popularity order   (4, layer, 0)         E uniforms  -> Fisher-Yates
  5  router matrix      (5, layer, 0)         E*H normals (tiny config only)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

from .configs import (WORKLOADS, Workload, expert_bytes, slot_stride,  # noqa: F401
                      TINY, QWEN_BF16, DSV4_MXFP4, DSV4_PREFILL, QWEN_ELASTIC)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "_gen.so")
_lock = threading.Lock()
_lib = None

TAG_WEIGHT, TAG_HIDDEN, TAG_NOISE, TAG_PERM, TAG_ROUTER = 1, 2, 3, 4, 5


def build(force: bool = False) -> str:
    """Compile gen.c into _gen.so with gcc (OpenMP).  -ffast-math is a compile
    flag only: linking with it would add the startup code that sets
    flush-to-zero / denormals-are-zero for the whole process when the library
    loads, changing the arithmetic of every other module in it."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        obj = tmp + ".o"
        subprocess.check_call(["gcc", "-O3", "-ffast-math", "-mavx2", "-mfma", "-fopenmp", "-fPIC", "-c",
                               "-o", obj, _SRC])
        subprocess.check_call(["gcc", "-shared", "-fopenmp", "-o", tmp, obj, "-lm"])
        os.remove(obj)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build()
            L = ctypes.CDLL(_LIB)
            u64, u32, i64, i32, f32 = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
                                       ctypes.c_int, ctypes.c_float)
            vp = ctypes.c_void_p
            L.wl_philox4x32_10.argtypes = [vp, vp, vp]
            L.wl_uniform_f64.argtypes = [u64, u32, u32, u32, i64, vp]
            L.wl_normal_f32.argtypes = [u64, u32, u32, u32, i64, f32, vp]
            L.wl_normal_bf16.argtypes = [u64, u32, u32, u32, i64, f32, vp]
            L.wl_expert_bytes.argtypes = [i32, i64, i64]
            L.wl_expert_bytes.restype = i64
            L.wl_fill_banks.argtypes = [u64, i32, i64, i64, i64, i64, f32, vp, i64, i32]
            L.wl_fill_banks.restype = i32
            L.wl_normal_bf16_streams.argtypes = [u64, u32, u32, u32, i64, i64, f32, vp, i32]
            L.wl_normal_f32_streams.argtypes = [u64, u32, u32, u32, i64, i64, f32, vp, i32]
            L.wl_uniform_f64_streams.argtypes = [u64, u32, u32, u32, i64, i64, vp, i32]
            _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def philox_block(ctr, key):
    c = np.asarray(ctr, np.uint32)
    k = np.asarray(key, np.uint32)
    out = np.zeros(4, np.uint32)
    lib().wl_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def uniform(seed: int, a: int, b: int, c: int, n: int) -> np.ndarray:
    out = np.empty(n, np.float64)
    lib().wl_uniform_f64(seed, a, b, c, n, _ptr(out))
    return out


def normal_f32(seed: int, a: int, b: int, c: int, n: int, sigma: float = 1.0) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().wl_normal_f32(seed, a, b, c, n, sigma, _ptr(out))
    return out


def normal_bf16(seed: int, a: int, b: int, c: int, n: int, sigma: float = 1.0) -> np.ndarray:
    """bfloat16 bit patterns (uint16), float normals rounded to nearest even."""
    out = np.empty(n, np.uint16)
    lib().wl_normal_bf16(seed, a, b, c, n, sigma, _ptr(out))
    return out


# ---------------------------------------------------------------- weights
DTYPE_CODE = {"f32": 0, "bf16": 1, "mxfp4": 2}


def fill_banks(wl: Workload, dst, u_begin: int, u_end: int, threads: int = 0) -> None:
    """Write expert banks u_begin..u_end-1 of ``wl`` into ``dst`` (a numpy
    uint8 array or an integer host address) at the slot stride."""
    stride = slot_stride(wl)
    if isinstance(dst, np.ndarray):
        assert dst.nbytes >= (u_end - u_begin) * stride
        addr = _ptr(dst)
    else:
        addr = int(dst)
    rc = lib().wl_fill_banks(wl.seed, DTYPE_CODE[wl.w_dtype], wl.H, wl.I, u_begin, u_end,
                             wl.w_sigma, addr, stride, threads)
    if rc != 0:
        raise ValueError("wl_fill_banks rejected its arguments")


def bank(wl: Workload, u: int) -> np.ndarray:
    """One expert bank of flat id u, as raw bytes."""
    out = np.empty(slot_stride(wl), np.uint8)
    fill_banks(wl, out, u, u + 1, threads=1)
    return out


# ---------------------------------------------------------------- activations
def hidden(wl: Workload, step: int, layer: int) -> np.ndarray:
    """Hidden states [T, H] of one layer call: N(0,1), float32 or bf16 bits."""
    n = wl.T * wl.H
    if wl.act_dtype == "f32":
        return normal_f32(wl.seed, TAG_HIDDEN, step, layer, n).reshape(wl.T, wl.H)
    out = np.empty(n, np.uint16)
    lib().wl_normal_bf16(wl.seed, TAG_HIDDEN, step, layer, n, 1.0, _ptr(out))
    return out.reshape(wl.T, wl.H)


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- routing inputs
def popularity_order(wl: Workload, layer: int) -> np.ndarray:
    """Seeded permutation pi_l (Fisher-Yates): expert pi_l[r] has Zipf rank r."""
    u = uniform(wl.seed, TAG_PERM, layer, 0, wl.E)
    perm = np.arange(wl.E)
    for i in range(wl.E - 1, 0, -1):
        j = int(u[i] * (i + 1))
        perm[i], perm[j] = perm[j], perm[i]
    return perm


def log_popularity(wl: Workload, layer: int) -> np.ndarray:
    """log p_l[e] with p_l(pi_l[r]) proportional to (r+1)^-s."""
    perm = popularity_order(wl, layer)
    r = np.arange(wl.E, dtype=np.float64)
    logp_rank = -wl.zipf_s * np.log(r + 1.0)
    logp_rank -= np.log(np.exp(logp_rank).sum())
    out = np.empty(wl.E)
    out[perm] = logp_rank
    return out


def gumbel(wl: Workload, step: int, layer: int) -> np.ndarray:
    u = uniform(wl.seed, TAG_NOISE, step, layer, wl.T * wl.E)
    return (-np.log(-np.log(u))).reshape(wl.T, wl.E)


def _sample_sets(logits: np.ndarray, k: int) -> np.ndarray:
    """The generator's own Gumbel-top-k sample (which experts got the bonus
    next step).  Input synthesis only."""
    return np.argpartition(-logits, k - 1, axis=-1)[..., :k]


def decode_logits(wl: Workload, beta: float | None = None, steps: int | None = None) -> np.ndarray:
    """Router logits for every decode call: float32 [steps, L, T, E].

    logit = log p_l + Gumbel + beta * [e was in this stream's previous sample]:
    Gumbel-top-k sampling without replacement proportional to a Zipf(s)
    popularity, with a stickiness bonus that sets the step-to-step reuse.
    """
    beta = wl.beta if beta is None else beta
    steps = wl.steps if steps is None else steps
    logp = np.stack([log_popularity(wl, l) for l in range(wl.L)])  # [L, E]
    out = np.empty((steps, wl.L, wl.T, wl.E), np.float32)
    prev = np.zeros((wl.L, wl.T, wl.E), bool)
    for s in range(steps):
        g = np.stack([gumbel(wl, s, l) for l in range(wl.L)])  # [L, T, E]
        lg = logp[:, None, :] + g + beta * prev
        out[s] = lg.astype(np.float32)
        sel = _sample_sets(out[s].astype(np.float64), wl.k)
        prev[:] = False
        np.put_along_axis(prev, sel, True, axis=-1)
    return out


def tiny_router_logits(wl: Workload) -> np.ndarray:
    """Tiny config: logits = fp32(x . W_g^T) from the fp32 hidden state of each
    call and a seeded N(0, 0.02) router matrix per layer; [steps, L, T, E]."""
    out = np.empty((wl.steps, wl.L, wl.T, wl.E), np.float32)
    for l in range(wl.L):
        wg = normal_f32(wl.seed, TAG_ROUTER, l, 0, wl.E * wl.H, 0.02).reshape(wl.E, wl.H)
        for s in range(wl.steps):
            x = hidden(wl, s, l).astype(np.float64)
            out[s, l] = (x @ wg.astype(np.float64).T).astype(np.float32)
    return out


def prefill_logits(wl: Workload, layer: int) -> np.ndarray:
    """Prefill chunk routing logits [T, E] float32: Zipf popularity + Gumbel."""
    return (log_popularity(wl, layer)[None, :] + gumbel(wl, 0, layer)).astype(np.float32)


def router_logits(wl: Workload) -> np.ndarray:
    if wl.router == "matrix":
        return tiny_router_logits(wl)
    return decode_logits(wl)


def reuse_fraction(logits: np.ndarray, k: int) -> float:
    """Mean |S_t intersect S_t-1| / k of the generator's own samples, over
    steps, layers and streams (input statistics only)."""
    sets = _sample_sets(logits.astype(np.float64), k)  # [steps, L, T, k]
    tot, cnt = 0.0, 0
    for s in range(1, sets.shape[0]):
        a, b = sets[s], sets[s - 1]
        inter = (a[..., :, None] == b[..., None, :]).any(-1).sum(-1)
        tot += inter.sum() / k
        cnt += inter.size
    return tot / max(cnt, 1)
