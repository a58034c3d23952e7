"""Bandwidth profile: the two rates the split uses, measured once per machine
and stored under a key of expert format and GPU name, so that a profile taken
on other hardware is ignored rather than applied (snackonai, "The Code,
Annotated": calibration on the deployed expert shapes decides the backend).

The measurements themselves run in libmoert.so (moe_measure_bandwidth,
moe_recommend_mode); this module only names, stores and looks up results."""
from __future__ import annotations

import json
import os

from . import binding as B


def profile_key(w_dtype: str, gpu_name: str) -> str:
    return f"{w_dtype}|{gpu_name}"


def measure(ctx, w_dtype: str, gpu_name: str, n_experts: int = 8, reps: int = 5,
            threshold: float = 2.0) -> dict:
    """Measure B_P (device pull), B_H (host expert kernel) and the pinned
    host-to-device copy rate on `ctx`'s expert shape; add the backend the
    threshold rule picks."""
    bp, bh, bc = B.moe_measure_bandwidth(ctx, n_experts, reps, h2d=True)
    mode = B.moe_recommend_mode(bp, bh, threshold)
    return {"key": profile_key(w_dtype, gpu_name), "w_dtype": w_dtype, "gpu": gpu_name,
            "bw_pcie_mbps": bp, "bw_host_mbps": bh, "bw_h2d_mbps": bc, "threshold": threshold,
            "backend": "hybrid" if mode == B.MOE_HYBRID else "offload",
            "n_experts": n_experts, "reps": reps}


def save(path: str, entry: dict) -> None:
    """Add or replace the entry under its key in the JSON profile at `path`."""
    prof = {}
    if os.path.exists(path):
        with open(path) as f:
            prof = json.load(f)
    prof[entry["key"]] = entry
    tmp = path + ".tmp"
    with open(tmp, "w") as f:
        json.dump(prof, f, indent=1, sort_keys=True)
        f.write("\n")
    os.replace(tmp, path)


def lookup(path: str, w_dtype: str, gpu_name: str) -> dict | None:
    """The entry measured for this expert format on this GPU, or None: an
    entry for another format or another GPU is never returned."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        prof = json.load(f)
    e = prof.get(profile_key(w_dtype, gpu_name))
    if e is None or e.get("w_dtype") != w_dtype or e.get("gpu") != gpu_name:
        return None
    return e
