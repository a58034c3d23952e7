"""The control kernel's 32-bit recency keys (csrc/lru_key.h), compiled for
the host from the same header and checked against the order the oracle's LRU
uses: ascending (tick, slot) with unbounded integer ticks, empty slots (tick
-1) first (satyajit, "Residency that follows the router").  The cases cross
2^32, where truncating a tick to 32 bits would invert the order."""
import os
import random
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "lru_key_check.cpp")
NOT_CANDIDATE = 0xFFFFFFFF
SPAN = 0xFFFFFFFE  # ticks within the last 2^32 - 3 calls keep their order


@pytest.fixture(scope="module")
def keys(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("lru") / "lru_key_check")
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-Wall", "-o", exe, SRC])

    def run(pairs):
        inp = "".join(f"{t} {n}\n" for t, n in pairs)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return [int(v) for v in out.split()]
    return run


def lru_order(slots):
    """Oracle order of candidate slots: (tick, slot) ascending."""
    return sorted(range(len(slots)), key=lambda s: (slots[s], s))


def key_order(keys_):
    return sorted(range(len(keys_)), key=lambda s: (keys_[s], s))


@pytest.mark.parametrize("now", [1, 5, 1000, 2**32 - 3, 2**32 - 1, 2**32, 2**32 + 7, 2**33 + 12345,
                                 2**62])
def test_order_matches_ticks_within_the_span(keys, now):
    rng = random.Random(now)
    lo = max(0, now - SPAN + 1)  # oldest tick still distinguished
    ticks = [-1, -1, lo, now - 1, now - 1]
    ticks += [rng.randint(lo, now - 1) for _ in range(200)]
    # neighbours of 2^32 and of the span's edge when they are candidates
    for t in (2**32 - 2, 2**32 - 1, 2**32, 2**32 + 1, lo + 1, lo + 2):
        if lo <= t < now:
            ticks.append(t)
    rng.shuffle(ticks)
    k = keys([(t, now) for t in ticks])
    assert all(0 <= v < NOT_CANDIDATE for v in k)
    assert key_order(k) == lru_order(ticks)
    assert all((v == 0) == (t < 0) for v, t in zip(k, ticks))


def test_truncation_case_crossing_2_32(keys):
    """Ticks on both sides of 2^32: a key of the low 32 bits of tick + 1 would
    put 2^32 + 1 before 2^32 - 2 (and collide with the non-candidate value)."""
    now = 2**32 + 2
    ticks = [2**32 - 2, 2**32 - 1, 2**32, 2**32 + 1, -1]
    k = keys([(t, now) for t in ticks])
    assert k[4] == 0 and k[0] < k[1] < k[2] < k[3] < NOT_CANDIDATE
    truncated = [(t + 1) & 0xFFFFFFFF for t in ticks]
    assert key_order(truncated) != lru_order(ticks)


def test_saturation_beyond_the_span(keys):
    """Slots untouched for 2^32 - 2 calls or more share key 1: after every
    empty slot, before every slot touched later, ordered among themselves by
    slot index (the one departure from exact LRU, documented)."""
    now = 2**40
    old = [now - SPAN, now - SPAN - 1, 5, 0]
    recent = [now - SPAN + 1, now - 1]
    k = keys([(t, now) for t in old + recent + [-1]])
    assert k[:4] == [1, 1, 1, 1]
    assert k[6] == 0
    assert 1 < k[4] < k[5] <= SPAN
