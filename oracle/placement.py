"""Routing-blind static placements and miss counting (oracle).

The snackonai teardown ("The Locality Result Nobody Is Quoting") observes
that a placement uncorrelated with routing misses at 1 - capacity, and
satyajit ("Residency that follows the router") that the global LRU beats the
static split at every capacity short of the full pool.  These helpers build
the two static placements used to check those statements:
  * a fixed set of floor(c * N) ids chosen uniformly at random (partial
    Fisher-Yates on uniforms supplied by the caller);
  * whole layers from layer 0 (a load-time layer split).
"""
from __future__ import annotations

import math


def random_set(N: int, c: float, uniforms) -> set:
    n = int(math.floor(c * N))
    ids = list(range(N))
    for i in range(n):
        j = i + int(uniforms[i] * (N - i))
        ids[i], ids[j] = ids[j], ids[i]
    return set(ids[:n])


def whole_layers(L: int, E: int, c: float) -> set:
    n_layers = int(math.floor(c * L * E)) // E
    return set(range(n_layers * E))


def static_misses(calls, resident: set):
    """calls: iterable of (layer, uniq flattened ids).  Returns (misses, accesses)."""
    miss = acc = 0
    for _, uniq in calls:
        for u in uniq:
            acc += 1
            miss += u not in resident
    return miss, acc
