"""The bandwidth profile's keying (CPU only): an entry is returned only for
the expert format and GPU it was measured on, so a profile copied from other
hardware is ignored (snackonai, "The Code, Annotated")."""
from routed_expert_execution_moe_amd import bw_profile as P


def _entry(w, gpu, bp, bh):
    return {"key": P.profile_key(w, gpu), "w_dtype": w, "gpu": gpu, "bw_pcie_mbps": bp,
            "bw_host_mbps": bh, "backend": "hybrid" if bh > 2 * bp else "offload"}


def test_lookup_only_matches_format_and_gpu(tmp_path):
    path = str(tmp_path / "bw.json")
    assert P.lookup(path, "bf16", "GPU A") is None
    P.save(path, _entry("bf16", "GPU A", 52_700, 77_300))
    P.save(path, _entry("mxfp4", "GPU A", 52_000, 140_000))
    P.save(path, _entry("bf16", "GPU B", 25_300, 56_700))
    assert P.lookup(path, "bf16", "GPU A")["bw_host_mbps"] == 77_300
    assert P.lookup(path, "mxfp4", "GPU A")["backend"] == "hybrid"
    assert P.lookup(path, "bf16", "GPU B")["bw_pcie_mbps"] == 25_300
    assert P.lookup(path, "mxfp4", "GPU B") is None      # other format on that GPU
    assert P.lookup(path, "bf16", "GPU C") is None       # other hardware
    P.save(path, _entry("bf16", "GPU A", 56_000, 250_000))  # re-measuring replaces
    assert P.lookup(path, "bf16", "GPU A")["bw_host_mbps"] == 250_000


def test_entry_with_mismatched_fields_is_ignored(tmp_path):
    """A hand-edited entry whose fields disagree with its key is not applied."""
    import json
    path = str(tmp_path / "bw.json")
    e = _entry("bf16", "GPU B", 1, 2)
    with open(path, "w") as f:
        json.dump({P.profile_key("bf16", "GPU A"): e}, f)
    assert P.lookup(path, "bf16", "GPU A") is None
