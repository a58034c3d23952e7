"""Bisect the stickiness bonus beta so that the mean step-to-step reuse
|S_t & S_t-1| / k of a Zipf workload's generated routing is 0.60.

    python -m workload.calibrate            # prints beta for the Qwen-shaped decode

The value is then written into configs.py by hand (it is an input recipe
constant, not a result)."""
import dataclasses
import sys

from . import QWEN_BF16, QWEN_ELASTIC, decode_logits, reuse_fraction


def calibrate(wl, target=0.60, steps=128, lo=0.0, hi=6.0, iters=30):
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        r = reuse_fraction(decode_logits(wl, beta=mid, steps=steps), wl.k)
        if r < target:
            lo = mid
        else:
            hi = mid
    return round(0.5 * (lo + hi), 2)


if __name__ == "__main__":
    for wl in (QWEN_BF16, QWEN_ELASTIC):
        b = calibrate(wl)
        r = reuse_fraction(decode_logits(dataclasses.replace(wl, beta=b), steps=128), wl.k)
        print(f"{wl.name}: beta={b} reuse={r:.4f}")
    sys.exit(0)
