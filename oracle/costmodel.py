"""Two-branch time model behind the q split (oracle).

Both the PCIe fill and the host expert kernel read host memory, so a
saturated transfer leaves B_H - B_P for the CPU branch; with m misses of S
bytes each and q of them filled (satyajit, "Decode: the one equation";
snackonai, "The split policy itself"):

    T_fill = q S / B_P,   T_cpu = (m - q) S / (B_H - B_P),
    exposed = max(T_fill, T_cpu)   (the CPU branch launches first and both run
                                    concurrently: snackonai, "The split policy
                                    itself", note on execution order)

Balancing the two gives q* = m B_P / B_H, where S cancels; at q* the exposed
time is m S / B_H.  The worked laptop numbers (snackonai, "It In Action";
"Insights", Insight Two) are evaluated with S = 1 and bandwidths in GB/s.
"""
from __future__ import annotations


def q_star(m: float, bp: float, bh: float) -> float:
    return m * bp / bh


def t_fill(q: float, bp: float, S: float = 1.0) -> float:
    return q * S / bp


def t_cpu(m: float, q: float, bp: float, bh: float, S: float = 1.0) -> float:
    return (m - q) * S / (bh - bp)


def exposed(m: float, q: float, bp: float, bh: float, S: float = 1.0) -> float:
    if q == m:
        return t_fill(q, bp, S)
    return max(t_fill(q, bp, S), t_cpu(m, q, bp, bh, S))


def all_pcie(m: float, bp: float, S: float = 1.0) -> float:
    return m * S / bp


def pure_cpu(m: float, bh: float, S: float = 1.0) -> float:
    """No transfer competes for host bandwidth, so the CPU gets all of B_H."""
    return m * S / bh


def recommend_hybrid(bp: float, bh: float, threshold: float = 2.0) -> bool:
    """Backend recommendation rule: hybrid when B_H > threshold * B_P
    (snackonai, "Calibration decides the backend, not the GPU")."""
    return bh > threshold * bp
