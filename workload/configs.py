"""The five synthetic workloads (shapes, sizes, seeds, bandwidths, schedules).

Slot counts are floor(capacity * number of generated expert ids).  Bandwidths
are integers in MB/s: the tiny workload states its own (25 / 50 GB/s); the
others use the measured RTX 5090 server profile printed in the snackonai
teardown's Bp/Bh table (52.7 / 77.3 GB/s), the machine whose PCIe rate backs
the pages' prefill figure.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    L: int                 # MoE layers generated
    E: int                 # routed experts per layer
    k: int                 # top-k
    H: int                 # hidden size
    I: int                 # expert intermediate size
    w_dtype: str           # "f32" | "bf16" | "mxfp4"
    act_dtype: str         # "f32" | "bf16"
    n_slots: int           # initial device slot budget
    bw_pcie_mbps: int
    bw_host_mbps: int
    steps: int             # decode steps (1 for the prefill chunk)
    T: int                 # tokens per layer call
    seed: int
    router: str = "zipf"   # "matrix" (x . W_g^T) or "zipf" (synthetic logits)
    zipf_s: float = 1.0
    beta: float = 0.0      # stickiness bonus giving the stated step-to-step reuse
    w_sigma: float = 0.02
    prefill: bool = False
    resize: dict = field(default_factory=dict)  # step -> new slot budget, applied before it

    @property
    def n_ids(self) -> int:
        return self.L * self.E


def expert_bytes(wl: Workload) -> int:
    H, I = wl.H, wl.I
    if wl.w_dtype == "f32":
        return 12 * H * I
    if wl.w_dtype == "bf16":
        return 6 * H * I
    return 3 * H * I // 2 + 3 * H * I // 32


def slot_stride(wl: Workload) -> int:
    """Bank / slot stride: expert bytes rounded up to 256 B."""
    return (expert_bytes(wl) + 255) // 256 * 256


TINY = Workload(
    name="tiny-fp32", L=2, E=8, k=2, H=64, I=128, w_dtype="f32", act_dtype="f32",
    n_slots=6, bw_pcie_mbps=25_000, bw_host_mbps=50_000, steps=16, T=1, seed=1001,
    router="matrix")

# 37% of 48*128 = 6144 ids -> 2273 slots.  beta gives mean reuse 0.60 (see
# workload/calibrate.py, which records it here).
QWEN_BF16 = Workload(
    name="qwen3.6-35b-a3b-shape-bf16-decode", L=48, E=128, k=8, H=2048, I=768,
    w_dtype="bf16", act_dtype="bf16", n_slots=2273, bw_pcie_mbps=52_700, bw_host_mbps=77_300,
    steps=256, T=1, seed=1002, zipf_s=1.1, beta=1.74)

# 11% of 8*256 = 2048 ids -> 225 slots.
DSV4_MXFP4 = Workload(
    name="deepseek-v4-flash-shape-mxfp4-decode", L=8, E=256, k=8, H=4096, I=2048,
    w_dtype="mxfp4", act_dtype="bf16", n_slots=225, bw_pcie_mbps=52_700, bw_host_mbps=77_300,
    steps=128, T=1, seed=1003, zipf_s=1.0, beta=0.0)

# Two full-layer buffers (2 * 256 slots) out of the shared pool.
DSV4_PREFILL = Workload(
    name="deepseek-v4-flash-shape-mxfp4-prefill-8192", L=8, E=256, k=8, H=4096, I=2048,
    w_dtype="mxfp4", act_dtype="bf16", n_slots=512, bw_pcie_mbps=52_700, bw_host_mbps=77_300,
    steps=1, T=8192, seed=1004, zipf_s=1.0, beta=0.0, prefill=True)

# 8 concurrent batch-1 streams batched per layer call; budget 37% -> 15% -> 30%
# (2273 -> 921 -> 1843), then an identity rebuild at 30%.
QWEN_ELASTIC = Workload(
    name="qwen3.6-35b-a3b-shape-bf16-elastic-8-streams", L=48, E=128, k=8, H=2048, I=768,
    w_dtype="bf16", act_dtype="bf16", n_slots=2273, bw_pcie_mbps=52_700, bw_host_mbps=77_300,
    steps=512, T=8, seed=1005, zipf_s=1.1, beta=1.73,
    resize={128: 921, 256: 1843, 384: 1843})

WORKLOADS = [TINY, QWEN_BF16, DSV4_MXFP4, DSV4_PREFILL, QWEN_ELASTIC]
