"""Build libmoert.so (HIP for gfx950 + host C++) in-tree.

    python -m routed_expert_execution_moe_amd.build [--force]

Device code is compiled with hipcc --offload-arch=gfx950 and packed-FP32
instructions disabled; the host branch is compiled with the host compiler
(AVX2 + FMA).  Objects go to _build/, the library next to this file.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmoert.so")
BUILD = os.path.join(ROOT, "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

HIP_SOURCES = ["route.hip", "plan.hip", "decode.hip", "ffn_f32.hip", "ffn_bf16.hip", "ffn_mx.hip",
               "prefill.hip", "ctx.cpp"]
HOST_SOURCES = ["cpu_branch.cpp"]
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
             "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics", "-I" + os.path.join(ROOT, "include")]
HOST_FLAGS = ["-O3", "-fPIC", "-std=c++17", "-mavx2", "-mfma", "-D__HIP_PLATFORM_AMD__",
              "-I" + os.path.join(ROCM, "include"), "-I" + os.path.join(ROOT, "include")]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r.stderr


def build(force: bool = True, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    headers = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    headers.append(os.path.join(ROOT, "include", "moert.h"))
    hdr_time = max(os.path.getmtime(h) for h in headers)
    jobs_list = []
    objs = []
    for src in HIP_SOURCES + HOST_SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        stale = force or not os.path.exists(obj) or \
            os.path.getmtime(obj) < max(os.path.getmtime(path), hdr_time)
        if not stale:
            continue
        if src in HIP_SOURCES:
            cmd = [HIPCC] + HIP_FLAGS + (["-x", "hip"] if src.endswith(".hip") else []) + \
                ["-c", path, "-o", obj]
        else:
            cmd = ["g++"] + HOST_FLAGS + ["-c", path, "-o", obj]
        jobs_list.append(cmd)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for warn in ex.map(_run, jobs_list):
            pass
    tmp = OUT + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs +
         ["-lpthread"])
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(force="--force" in sys.argv))
