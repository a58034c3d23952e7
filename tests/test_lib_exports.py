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


def test_strerror(lib):
    lib.moe_strerror.restype = ctypes.c_char_p
    lib.moe_strerror.argtypes = [ctypes.c_int]
    for s in range(0, -8, -1):
        assert lib.moe_strerror(s)
    assert b"unknown" in lib.moe_strerror(-99)
