"""The C-ABI library loads and exports every function include/moert.h
declares, and its host-side validation behaves (CPU only: no call here
touches a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moert.h")
LIB = os.path.join(ROOT, "routed_expert_execution_moe_amd", "libmoert.so")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(moe_[a-z_]+)\s*\(", src)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from routed_expert_execution_moe_amd.build import build
        build(force=False)
    return ctypes.CDLL(LIB)


def test_header_declares_the_six_calls():
    names = declared_functions()
    for n in ("moe_route_topk", "moe_cache_plan", "moe_expert_ffn", "moe_merge",
              "moe_cache_resize", "moe_prefill_layer"):
        assert n in names


def test_every_declared_symbol_exported(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_expert_bytes_and_validation(lib):
    from routed_expert_execution_moe_amd.binding import MoeConfig
    f = lib.moe_expert_bytes
    f.argtypes = [ctypes.POINTER(MoeConfig)]
    f.restype = ctypes.c_size_t

    def cfg(**kw):
        base = dict(n_layers=48, n_experts=128, top_k=8, hidden=2048, inter=768, w_dtype=1,
                    act_dtype=1, n_slots=2273, max_slots=2273, max_tokens=8,
                    bw_pcie_mbps=52700, bw_host_mbps=77300, max_fetch=0, mode=0,
                    cpu_threads=0, max_prefill_tokens=0)
        base.update(kw)
        return MoeConfig(**base)

    assert f(ctypes.byref(cfg())) == 9_437_184
    assert f(ctypes.byref(cfg(n_layers=8, n_experts=256, hidden=4096, inter=2048,
                              w_dtype=2))) == 13_369_344
    assert f(ctypes.byref(cfg(n_layers=2, n_experts=8, hidden=64, inter=128, w_dtype=0,
                              act_dtype=0, n_slots=6, max_slots=6, max_tokens=1))) == 98_304
    for bad in (dict(n_experts=0), dict(n_experts=2048), dict(top_k=0), dict(top_k=200),
                dict(n_slots=3000), dict(max_tokens=0), dict(max_tokens=300),
                dict(bw_pcie_mbps=0), dict(mode=7), dict(w_dtype=5), dict(act_dtype=2),
                dict(hidden=100), dict(max_slots=40000), dict(max_fetch=-1)):
        assert f(ctypes.byref(cfg(**bad))) == 0, bad


def test_prefill_row_offsets_stay_32_bit(lib):
    """The grouped GEMM addresses activation rows with 32-bit byte offsets, so
    a prefill chunk with T*H*2 or T*k*I*2 at 2^32 bytes or more is refused;
    the largest chunks just below the bound are accepted."""
    from routed_expert_execution_moe_amd.binding import MoeConfig
    f = lib.moe_expert_bytes
    f.argtypes = [ctypes.POINTER(MoeConfig)]
    f.restype = ctypes.c_size_t

    def ok(T, k, H, I):
        c = MoeConfig(n_layers=2, n_experts=256, top_k=k, hidden=H, inter=I, w_dtype=2,
                      act_dtype=1, n_slots=0, max_slots=0, max_tokens=1, bw_pcie_mbps=1,
                      bw_host_mbps=1, max_fetch=0, mode=0, cpu_threads=0, max_prefill_tokens=T)
        return f(ctypes.byref(c)) != 0

    assert ok(8192, 8, 4096, 2048)           # the DeepSeek-shaped chunk
    assert ok(65536, 8, 4096, 2048)          # T*k*I*2 = 2^31
    assert ok(65535, 16, 16384, 2048)        # T*H*2 = 2^31 - 2^15, T*k*I*2 just below 2^32
    assert not ok(65536, 16, 4096, 2048)     # T*k*I*2 = 2^32
    assert not ok(65536, 8, 4096, 8192)      # T*k*I*2 = 2^33
    assert not ok(65536, 1, 16384 * 2, 64)   # hidden out of range anyway
    assert not ok(65536, 32, 64, 4096)       # T*k*I*2 = 2^34


def test_strerror(lib):
    lib.moe_strerror.restype = ctypes.c_char_p
    lib.moe_strerror.argtypes = [ctypes.c_int]
    for s in range(0, -8, -1):
        assert lib.moe_strerror(s)
    assert b"unknown" in lib.moe_strerror(-99)


def test_recommend_mode_matches_the_pages_rule(lib, golden_dir):
    """moe_recommend_mode (host arithmetic, no GPU) against the oracle's rule,
    which is pinned to the six machines of the pages' calibration table: the
    six rows, ties (B_H exactly 2 B_P stays offload), random pairs, bad input."""
    import json
    import random
    from oracle import costmodel
    f = lib.moe_recommend_mode
    f.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_double, ctypes.POINTER(ctypes.c_int32)]
    f.restype = ctypes.c_int32
    HYBRID, OFFLOAD = 0, 1

    def rec(bp, bh, th=2.0):
        out = ctypes.c_int32(-1)
        assert f(bp, bh, th, ctypes.byref(out)) == 0
        return out.value

    g = json.load(open(os.path.join(golden_dir, "split_policy.json")))
    for row in g["bw_table"]:
        bp, bh = int(round(row["bp"] * 1000)), int(round(row["bh"] * 1000))
        assert rec(bp, bh, g["threshold"]) == (HYBRID if row["backend"] == "hybrid" else OFFLOAD), row
    assert rec(25_000, 50_000) == OFFLOAD and rec(25_000, 50_001) == HYBRID
    r = random.Random(7)
    for _ in range(2000):
        bp, bh, th = r.randint(1, 200_000), r.randint(1, 400_000), r.choice([1.0, 1.5, 2.0, 3.0])
        want = HYBRID if costmodel.recommend_hybrid(bp, bh, th) else OFFLOAD
        assert rec(bp, bh, th) == want, (bp, bh, th)
    out = ctypes.c_int32()
    for bad in ((0, 1, 2.0), (1, 0, 2.0), (1, 1, 0.0), (1, 1, -1.0)):
        assert f(*bad, ctypes.byref(out)) == -1
