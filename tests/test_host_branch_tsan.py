"""The host branch on the CPU alone, under ThreadSanitizer.

The misses assigned to the CPU run on a persistent, core-pinned worker pool
that reads the pinned host banks in place (snackonai, "Technical Moats";
"The split policy itself": the CPU set executes where its weights live).
tests/native/host_branch_check.cpp links the library's cpu_branch.cpp (the
doorbell poller and the worker pool) into a program built with
-fsanitize=thread, which stands in for the control kernel (writes each call's
host block and rings the doorbell) and for the merge (waits for the
completion word).  Checked here: no data race reported, every doorbell
answered, and every host row equals the fp64 oracle's SwiGLU of its expert to
fp32 rounding; pairs with an id outside [0, E) get zero rows.  No GPU."""
import dataclasses
import os
import subprocess

import numpy as np
import pytest

import workload as W
from oracle import expert as OX

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRCS = [os.path.join(ROOT, "tests", "native", "host_branch_check.cpp"),
        os.path.join(ROOT, "routed_expert_execution_moe_amd", "csrc", "cpu_branch.cpp")]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ACT = {"f32": 0, "bf16": 1}
WDT = {"f32": 0, "bf16": 1, "mxfp4": 2}


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("hb") / "host_branch_check")
    # host code only (g++, no device code): the sanitizer instruments the
    # poller, the workers and the stand-in for the device side
    subprocess.check_call(["g++", "-O1", "-g", "-fsanitize=thread", "-std=c++17", "-mavx2", "-mfma",
                           "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"),
                           "-I" + os.path.join(ROOT, "include"), "-o", out] + SRCS + ["-lpthread"])
    return out


def make_calls(wl, n_calls, rng):
    """Per call: layer, ids [T,k], slot map (-1 = host; a few pairs stay on
    the 'GPU'), activations in the act dtype, with tokens sharing experts and
    one out-of-range id now and then."""
    calls = []
    for c in range(n_calls):
        layer = int(rng.integers(wl.L))
        ids = np.stack([rng.choice(wl.E, wl.k, replace=False) for _ in range(wl.T)]).astype(np.int32)
        if c % 3 == 2:
            ids[0, -1] = wl.E + 3  # caller error: the host writes a zero row
        smap = np.where(rng.random(ids.shape) < 0.7, -1, 0).astype(np.int32)
        x = W.hidden(wl, c, layer)
        calls.append((layer, ids, smap, x))
    return calls


@pytest.mark.parametrize("w_dtype,act", [("bf16", "bf16"), ("mxfp4", "bf16"), ("f32", "f32")])
def test_host_branch_under_tsan(exe, tmp_path, w_dtype, act):
    wl = dataclasses.replace(W.TINY, L=2, E=8, k=3, H=256, I=128, w_dtype=w_dtype, act_dtype=act,
                             T=4, steps=1, seed=4242)
    stride = W.slot_stride(wl)
    pool = np.empty(wl.n_ids * stride, np.uint8)
    W.fill_banks(wl, pool, 0, wl.n_ids)
    rng = np.random.default_rng(11)
    calls = make_calls(wl, 12, rng)
    threads = 3
    inp = tmp_path / "in.bin"
    with open(inp, "wb") as f:
        f.write(np.array([wl.L, wl.E, wl.k, wl.H, wl.I, WDT[w_dtype], ACT[act], wl.T, len(calls),
                          threads], np.int32).tobytes())
        f.write(np.array([stride], np.int64).tobytes())
        f.write(pool.tobytes())
        for layer, ids, smap, x in calls:
            f.write(np.array([layer], np.int32).tobytes())
            f.write(ids.tobytes())
            f.write(smap.tobytes())
            f.write(np.ascontiguousarray(x).tobytes())
    out = tmp_path / "out.bin"
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 exitcode=66 second_deadlock_stack=1")
    r = subprocess.run([exe, str(inp), str(out)], capture_output=True, text=True, env=env, timeout=300)
    assert "ThreadSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, (r.returncode, r.stderr[-2000:])
    rows = np.fromfile(out, np.float32).reshape(len(calls), wl.T * wl.k, wl.H)

    def weights(u):
        return OX.expert_weights(pool[u * stride:(u + 1) * stride], w_dtype, wl.H, wl.I)

    worst = 0.0
    for c, (layer, ids, smap, x) in enumerate(calls):
        xf = W.bf16_bits_to_f32(x).astype(np.float64) if act == "bf16" else x.astype(np.float64)
        for t in range(wl.T):
            for j in range(wl.k):
                p = t * wl.k + j
                got = rows[c, p].astype(np.float64)
                if smap[t, j] >= 0:
                    continue
                e = int(ids[t, j])
                if not 0 <= e < wl.E:
                    assert not got.any(), (c, t, j)
                    continue
                ref = OX.ffn(xf[t:t + 1], weights(layer * wl.E + e))[0]
                rms = float(np.sqrt(np.mean(ref ** 2)))
                err = float(np.abs(got - ref).max()) / rms
                worst = max(worst, err)
                assert err <= 1e-4, (c, t, j, err)
    assert worst > 0.0  # rows were compared
