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
SPAN = 0xFFFFFFFD  # occupied candidates' ticks within this span of the oldest keep their order


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


@pytest.mark.parametrize("tmin", [0, 5, 1000, 2**32 - 3, 2**32 - 1, 2**32, 2**32 + 7, 2**33 + 12345,
                                  2**62])
def test_order_matches_ticks_within_the_span(keys, tmin):
    """Empty slots and occupied ticks in [tmin, tmin + SPAN): the keys order
    the slots exactly as (tick, slot) does."""
    rng = random.Random(tmin)
    hi = tmin + SPAN - 1  # newest tick still distinguished
    ticks = [-1, -1, tmin, tmin, hi, hi]
    ticks += [rng.randint(tmin, hi) for _ in range(200)]
    ticks += [rng.randint(tmin, tmin + 50) for _ in range(50)]  # near-ties
    for t in (2**32 - 2, 2**32 - 1, 2**32, 2**32 + 1, tmin + 1, hi - 1):
        if tmin <= t <= hi:
            ticks.append(t)
    rng.shuffle(ticks)
    k = keys([(t, tmin) for t in ticks])
    assert all(0 <= v < NOT_CANDIDATE for v in k)
    assert key_order(k) == lru_order(ticks)
    assert all((v == 0) == (t < 0) for v, t in zip(k, ticks))
    assert all(v == 1 for v, t in zip(k, ticks) if t == tmin)


def test_truncation_case_crossing_2_32(keys):
    """Ticks on both sides of 2^32: a key of the low 32 bits of tick + 1 would
    put 2^32 + 1 before 2^32 - 2 (and collide with the non-candidate value)."""
    tmin = 2**32 - 2
    ticks = [2**32 - 2, 2**32 - 1, 2**32, 2**32 + 1, -1]
    k = keys([(t, tmin) for t in ticks])
    assert k[4] == 0 and k[0] < k[1] < k[2] < k[3] < NOT_CANDIDATE
    truncated = [(t + 1) & 0xFFFFFFFF for t in ticks]
    assert key_order(truncated) != lru_order(ticks)


def test_saturation_beyond_the_span(keys):
    """Occupied candidates touched SPAN calls or more after the oldest share
    the largest key: after every other candidate, ordered among themselves by
    slot index (the one departure from exact LRU; the oldest, which the
    victims are drawn from, stay exact)."""
    tmin = 2**40
    inside = [tmin, tmin + 1, tmin + SPAN - 1]
    beyond = [tmin + SPAN, tmin + SPAN + 5, tmin + 2**33]
    k = keys([(t, tmin) for t in inside + beyond + [-1]])
    assert k[6] == 0
    assert k[0] == 1 and k[0] < k[1] < k[2] < k[3]
    assert k[3:6] == [0xFFFFFFFE] * 3


def test_small_spread_means_small_keys(keys):
    """The keys' range is the candidates' age range (what the select's digit
    skipping relies on), also with empty slots present and far-off absolute
    ticks."""
    tmin = 2**35 + 17
    ticks = [-1, tmin, tmin + 3, tmin + 1000]
    assert keys([(t, tmin) for t in ticks]) == [0, 1, 4, 1001]
