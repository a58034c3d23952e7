"""Residency planning for one MoE-layer call (oracle, integers only).

What the pages fix:
  * one global pool of complete-expert slots shared by every layer, each
    expert named by the flattened id u = l*E + e (snackonai, "The
    Architecture, Unpacked", first decision; signalovernoise essay);
  * one control step per MoE layer: deduplicate the routed experts, classify
    them against the residency table, derive q, choose victims, rewrite
    logical ids into slot ids or a CPU flag (snackonai, "The Architecture,
    Unpacked", third decision; satyajit, "Residency that follows the router");
  * a global LRU: a hit refreshes recency, a fill admits, an eviction removes
    the least recently demanded expert (satyajit, "Residency that follows the
    router");
  * victims: the K least recently used slots surfaced in one pass, the first
    q <= K consumed (satyajit, "Residency that follows the router");
  * q = round(m * B_P / B_H), clamped to at least one fill and at most m;
    the first q misses are filled, the rest run on the CPU where the weights
    live (snackonai, "The Code, Annotated" / "The split policy itself";
    satyajit, "Decode: the one equation");
  * backends offload (every miss crosses PCIe) and cpu (misses run on the
    host) (satyajit, "Four backends, and the one that has to be measured");
  * a per-layer cap on PCIe fetches (same section, --moe-hybrid-max-fetch).

Readings where the pages are silent or loose:
  * rounding is half-to-even (the printed split uses Python's round), done
    exactly on integer MB/s bandwidths; m = 0 gives q = 0;
  * the q misses filled are the smallest flattened ids (U is ascending);
  * one LRU tick per call; every slot touched by the call takes that tick;
    recency order is (tick, slot index); empty slots carry tick -1 and so
    go first, lowest index first; current hits are never victims;
  * q is also capped by the slots not holding a current hit;
  * K = min(max_tokens * k, E, n_slots), and min(K, max_fetch) when a cap is
    set; the surfaced list is padded with -1;
  * CPU-assigned misses are not admitted and do not touch recency;
  * the CPU flag in the slot map is -1.
"""
from __future__ import annotations

from dataclasses import dataclass, field

HYBRID, OFFLOAD, CPU = 0, 1, 2


def rne_div(a: int, b: int) -> int:
    """a / b rounded to the nearest integer, ties to even (a >= 0, b > 0)."""
    assert a >= 0 and b > 0
    q0, r = divmod(a, b)
    if 2 * r > b or (2 * r == b and q0 % 2 == 1):
        return q0 + 1
    return q0


def split_q(m: int, bw_pcie: int, bw_host: int, mode: int) -> int:
    """Number of misses sent over PCIe before capacity / fetch caps
    (snackonai, "The split policy itself"; satyajit, "Decode: the one
    equation"; backends per satyajit, "Four backends ...")."""
    if m == 0:
        return 0
    if mode == OFFLOAD:
        return m
    if mode == CPU:
        return 0
    q = rne_div(m * bw_pcie, bw_host)
    return min(max(1, q), m)


def victim_bound(max_tokens: int, k: int, E: int, n_slots: int, max_fetch: int = 0) -> int:
    K = min(max_tokens * k, E, n_slots)
    if max_fetch > 0:
        K = min(K, max_fetch)
    return K


class Residency:
    """id2slot[N], slot2id[n], slot_ts[n] and the tick; all empty at start
    (no warmup: satyajit, "Elastic memory ...", fast bootstrap)."""

    def __init__(self, n_ids: int, n_slots: int):
        self.id2slot = [-1] * n_ids
        self.slot2id = [-1] * n_slots
        self.slot_ts = [-1] * n_slots
        self.tick = 0

    @property
    def n_slots(self) -> int:
        return len(self.slot2id)

    def copy(self) -> "Residency":
        r = Residency(0, 0)
        r.id2slot = list(self.id2slot)
        r.slot2id = list(self.slot2id)
        r.slot_ts = list(self.slot_ts)
        r.tick = self.tick
        return r


@dataclass
class Plan:
    layer: int
    tick: int
    uniq: list            # ascending flattened ids routed in this call
    hits: list            # resident before the call, ascending u
    misses: list          # not resident, ascending u
    q: int                # misses filled over PCIe
    victims: list         # K slots, least recently used first, -1 padded
    fills: list           # (u, slot, evicted u or -1) for the first q misses
    cpu: list             # misses[q:], computed on the host
    slot_map: list        # [T][k]: slot id, or -1 for the CPU
    gpu: list = field(default_factory=list)  # (u, slot) evaluated on the GPU, ascending u


def plan(st: Residency, layer: int, ids, E: int, K: int, bw_pcie: int, bw_host: int,
         mode: int = HYBRID, max_fetch: int = 0) -> Plan:
    """One control step for MoE layer `layer` routed to ids [T][k]."""
    n = st.n_slots
    st.tick += 1
    tick = st.tick
    rows = [[int(e) for e in row] for row in ids]
    for row in rows:
        for e in row:
            assert 0 <= e < E

    # deduplicate the flattened ids of every routed (token, rank) of the call
    uniq = sorted({layer * E + e for row in rows for e in row})
    # classify against the residency table
    hits = [u for u in uniq if st.id2slot[u] >= 0]
    misses = [u for u in uniq if st.id2slot[u] < 0]
    m = len(misses)

    q = split_q(m, bw_pcie, bw_host, mode)
    if max_fetch > 0:
        q = min(q, max_fetch)
    q = min(q, n - len(hits))

    # a hit refreshes recency
    hit_slots = set()
    for u in hits:
        s = st.id2slot[u]
        hit_slots.add(s)
        st.slot_ts[s] = tick

    # the K least recently used slots that do not hold a current hit
    cands = sorted((st.slot_ts[s], s) for s in range(n) if s not in hit_slots)
    victims = [s for _, s in cands[:K]]
    victims += [-1] * (K - len(victims))
    assert q <= len([v for v in victims if v >= 0])

    # the first q misses are admitted into the first q victims
    fills = []
    for i in range(q):
        u, s = misses[i], victims[i]
        old = st.slot2id[s]
        if old >= 0:
            st.id2slot[old] = -1
        st.slot2id[s] = u
        st.id2slot[u] = s
        st.slot_ts[s] = tick
        fills.append((u, s, old))
    cpu = misses[q:]

    slot_map = [[st.id2slot[layer * E + e] for e in row] for row in rows]
    gpu = [(u, st.id2slot[u]) for u in uniq if st.id2slot[u] >= 0]
    return Plan(layer=layer, tick=tick, uniq=uniq, hits=hits, misses=misses, q=q,
                victims=victims, fills=fills, cpu=cpu, slot_map=slot_map, gpu=gpu)


def resize(st: Residency, n_new: int):
    """Rebuild the slot pool under a new budget without touching the host
    pool (satyajit, "Elastic memory ..."; snackonai, "Resizing the cache
    without a restart": shrinking costs throughput and nothing else).
    Reading: shrinking evicts in the same order the LRU surfaces victims,
    (tick, slot) ascending, until min(n_new, occupied) experts remain; a
    survivor below n_new stays in its slot, and the survivors at or above
    n_new move, in ascending old-slot order, into the free slots below n_new
    in ascending order, so the fewest bytes move and no move reads a slot
    another move writes.  Survivors keep their ticks; dropped ids become
    non-resident; growing appends empty slots.  Returns the moves
    [(old_slot, new_slot)]."""
    assert n_new >= 0
    n = st.n_slots
    occupied = [s for s in range(n) if st.slot2id[s] >= 0]
    lru_first = sorted(occupied, key=lambda s: (st.slot_ts[s], s))
    keep = set(lru_first[len(occupied) - min(n_new, len(occupied)):])
    for s in occupied:
        if s not in keep:
            st.id2slot[st.slot2id[s]] = -1
    new_ids = [-1] * n_new
    new_ts = [-1] * n_new
    for s in sorted(keep):
        if s < n_new:
            new_ids[s] = st.slot2id[s]
            new_ts[s] = st.slot_ts[s]
    free = [j for j in range(n_new) if new_ids[j] < 0]
    movers = [s for s in sorted(keep) if s >= n_new]
    moves = list(zip(movers, free))
    for s, j in moves:
        u = st.slot2id[s]
        new_ids[j] = u
        new_ts[j] = st.slot_ts[s]
        st.id2slot[u] = j
    st.slot2id = new_ids
    st.slot_ts = new_ts
    return moves


def prefill_admit(st: Residency, layer: int, E: int, buffers: int = 2):
    """Full-layer buffer admission for prefill (satyajit, "Prefill: hide the
    pool behind the wire"; signalovernoise essay).  Two full-layer buffers
    come out of the shared pool; reading: they are slots [0, E) and [E, 2E),
    layer l uses buffer l mod 2, expert e of layer l sits in slot b*E + e with
    one tick per prefill layer; the buffer's previous occupants are evicted
    and any other slot still holding an expert of layer l is emptied.  What
    survives seeds decode.  With the second buffer disabled (snackonai, "It
    In Action") every layer uses buffer 0.  Returns the buffer index b."""
    assert buffers in (1, 2)
    n = st.n_slots
    if n < buffers * E:
        raise ValueError("the full-layer buffers do not fit in the slot pool")
    st.tick += 1
    b = layer % buffers
    for e in range(E):
        s = b * E + e
        old = st.slot2id[s]
        if old >= 0:
            st.id2slot[old] = -1
        st.slot2id[s] = -1
        st.slot_ts[s] = -1
    for e in range(E):
        u = layer * E + e
        s = st.id2slot[u]
        if s >= 0:
            st.slot2id[s] = -1
            st.slot_ts[s] = -1
            st.id2slot[u] = -1
    for e in range(E):
        s, u = b * E + e, layer * E + e
        st.slot2id[s] = u
        st.id2slot[u] = s
        st.slot_ts[s] = st.tick
    return b


def prefill_on_demand(st: Residency, layer: int, routed, E: int):
    """On-demand prefill when the pool cannot hold the full-layer buffers
    (signalovernoise essay: it falls back to on-demand rather than
    oversubscribe; snackonai, "The Architecture, Unpacked", second decision:
    it degrades to on-demand loading instead of oversubscribing VRAM).

    Reading: only the experts of `layer` that the chunk routes to are loaded,
    after routing is known, in ascending expert order and in passes of at
    most n (the slot count) experts.  A pass behaves like a small full-layer
    buffer: one tick; slots [0, P) evict their occupants; any other slot
    holding one of the pass's IDs is emptied; expert i of the pass goes to
    slot i with the pass's tick.  Every routed expert of a pass is loaded
    from its host bank even if it was resident elsewhere.  Returns the passes
    (lists of expert indices)."""
    n = st.n_slots
    if n < 1:
        raise ValueError("on-demand prefill needs at least one slot")
    experts = sorted({int(e) for e in routed if 0 <= int(e) < E})
    passes = [experts[i:i + n] for i in range(0, len(experts), n)]
    for part in passes:
        st.tick += 1
        ids = [layer * E + e for e in part]
        for i in range(len(part)):
            old = st.slot2id[i]
            if old >= 0:
                st.id2slot[old] = -1
            st.slot2id[i] = -1
            st.slot_ts[i] = -1
        for u in ids:
            s = st.id2slot[u]
            if s >= 0:
                st.slot2id[s] = -1
                st.slot_ts[s] = -1
                st.id2slot[u] = -1
        for i, u in enumerate(ids):
            st.slot2id[i] = u
            st.id2slot[u] = i
            st.slot_ts[i] = st.tick
    return passes
