"""Pins of the residency plan: an independent recency-list model on
exhaustively enumerated tiny traces and random traces, textbook LRU through
Mattson stack distances, and structural invariants (CPU only)."""
import itertools
import random

import pytest

from oracle import plan as P
from tests.lru_sim import RecencySim


def compare(pl, sim_out, st, sim):
    assert pl.uniq == sim_out["uniq"]
    assert pl.hits == sim_out["hits"]
    assert pl.misses == sim_out["misses"]
    assert pl.q == sim_out["q"]
    assert pl.victims == sim_out["victims"]
    assert pl.fills == sim_out["fills"]
    assert pl.cpu == sim_out["cpu"]
    assert pl.slot_map == sim_out["slot_map"]
    assert st.slot2id == sim.slot2id()
    order = sorted(range(st.n_slots), key=lambda s: (st.slot_ts[s], s))
    assert order == sim.recency_order()


def check_invariants(st, pl, K):
    n = st.n_slots
    for s, u in enumerate(st.slot2id):
        if u >= 0:
            assert st.id2slot[u] == s
    for u, s in enumerate(st.id2slot):
        if s >= 0:
            assert st.slot2id[s] == u
    assert sum(1 for u in st.slot2id if u >= 0) <= n
    filled = [f[0] for f in pl.fills]
    assert sorted(pl.hits + filled + pl.cpu) == pl.uniq
    assert filled == pl.misses[:pl.q]
    real = [v for v in pl.victims if v >= 0]
    assert len(real) == len(set(real)) and len(pl.victims) == K
    hit_slots = {s for (u, s) in pl.gpu if u in set(pl.hits)}
    assert not (set(real) & hit_slots)
    for (u, s, old) in pl.fills:
        assert st.slot2id[s] == u and st.slot_ts[s] == pl.tick
    for row_ids, row_map in zip(pl.slot_map, pl.slot_map):
        for s in row_map:
            assert s == -1 or 0 <= s < n


def calls_alphabet(L, E, k, T):
    rows = list(itertools.combinations(range(E), k))
    out = []
    for l in range(L):
        for toks in itertools.product(rows, repeat=T):
            out.append((l, [list(r) for r in toks]))
    return out


@pytest.mark.parametrize("n,mode,bp,bh,T,k,depth", [
    (1, P.HYBRID, 25_000, 50_000, 1, 2, 6),
    (2, P.HYBRID, 25_000, 50_000, 1, 2, 6),
    (3, P.HYBRID, 25_000, 50_000, 1, 2, 6),
    (3, P.OFFLOAD, 1, 1, 1, 2, 6),
    (2, P.CPU, 1, 1, 1, 2, 5),
    (3, P.HYBRID, 11_800, 47_500, 2, 1, 4),
    (4, P.HYBRID, 52_700, 77_300, 2, 2, 3),
])
def test_exhaustive_tiny_traces(n, mode, bp, bh, T, k, depth):
    """Every trace up to `depth` calls over L=2 layers of E=3 experts."""
    L, E = 2, 3
    alphabet = calls_alphabet(L, E, k, T)
    K = P.victim_bound(T, k, E, n)
    nodes = 0

    def dfs(st, sim, d):
        nonlocal nodes
        if d == depth:
            return
        for layer, ids in alphabet:
            st2, sim2 = st.copy(), sim.copy()
            pl = P.plan(st2, layer, ids, E, K, bp, bh, mode)
            out = sim2.call(layer, ids, E, K, bp, bh, mode)
            compare(pl, out, st2, sim2)
            check_invariants(st2, pl, K)
            nodes += 1
            dfs(st2, sim2, d + 1)

    dfs(P.Residency(L * E, n), RecencySim(n), 0)
    assert nodes > 100


@pytest.mark.parametrize("seed", range(6))
def test_random_traces(seed):
    rng = random.Random(seed)
    L, E = rng.randint(1, 4), rng.randint(4, 16)
    k = rng.randint(1, min(4, E))
    T = rng.randint(1, 4)
    n = rng.randint(0, L * E + 2)
    mode = rng.choice([P.HYBRID, P.OFFLOAD, P.CPU])
    bp = rng.randint(1_000, 60_000)
    bh = bp + rng.randint(0, 150_000)
    max_fetch = rng.choice([0, 0, 1, 2])
    K = P.victim_bound(T, k, E, n, max_fetch)
    st, sim = P.Residency(L * E, n), RecencySim(n)
    hot = [rng.sample(range(E), k) for _ in range(L)]
    for step in range(300):
        layer = step % L
        ids = []
        for t in range(T):
            if rng.random() < 0.5:
                ids.append(list(hot[layer]))
            else:
                ids.append(rng.sample(range(E), k))
        pl = P.plan(st, layer, ids, E, K, bp, bh, mode, max_fetch)
        out = sim.call(layer, ids, E, K, bp, bh, mode, max_fetch)
        compare(pl, out, st, sim)
        check_invariants(st, pl, K)
        if rng.random() < 0.05:
            n_new = rng.randint(0, L * E + 2)
            P.resize(st, n_new)
            sim.resize(n_new)
            K = P.victim_bound(T, k, E, n_new, max_fetch)
            assert st.slot2id == sim.slot2id()
            order = sorted(range(st.n_slots), key=lambda s: (st.slot_ts[s], s))
            assert order == sim.recency_order()


def stack_distance_misses(trace, capacities):
    """Mattson et al. (1970) stack algorithm: one pass gives the LRU miss
    count of every capacity; an access misses at capacity C iff its stack
    distance exceeds C (first touches have infinite distance)."""
    stack, dists = [], []
    for u in trace:
        if u in stack:
            d = stack.index(u) + 1
            stack.remove(u)
        else:
            d = float("inf")
        stack.insert(0, u)
        dists.append(d)
    return {C: sum(1 for d in dists if d > C) for C in capacities}


@pytest.mark.parametrize("seed", range(4))
def test_textbook_lru_via_stack_distances(seed):
    """T = 1, k = 1, offload: the plan is a fully associative LRU cache."""
    rng = random.Random(100 + seed)
    L, E = 3, 7
    trace_calls = []
    for step in range(400):
        layer = rng.randrange(L)
        e = min(int(rng.paretovariate(1.2)) - 1, E - 1)
        trace_calls.append((layer, e))
    trace = [l * E + e for l, e in trace_calls]
    caps = list(range(0, 12))
    expect = stack_distance_misses(trace, caps)
    for C in caps:
        st = P.Residency(L * E, C)
        K = P.victim_bound(1, 1, E, C)
        misses = 0
        for layer, e in trace_calls:
            pl = P.plan(st, layer, [[e]], E, K, 1, 1, P.OFFLOAD)
            misses += len(pl.misses)
        assert misses == expect[C], C


def test_offload_holds_most_recent():
    """Offload mode with |U| <= n: after each call the resident ids are the
    call's ids plus the most recently used others."""
    rng = random.Random(5)
    L, E, k, n = 2, 10, 3, 7
    st = P.Residency(L * E, n)
    K = P.victim_bound(1, k, E, n)
    last = {}
    for step in range(500):
        layer = rng.randrange(L)
        ids = [rng.sample(range(E), k)]
        pl = P.plan(st, layer, ids, E, K, 1, 1, P.OFFLOAD)
        for u in pl.uniq:
            last[u] = step
        res = {u for u in st.slot2id if u >= 0}
        assert set(pl.uniq) <= res
        nonres = [u for u in last if u not in res]
        if nonres:
            assert min(last[u] for u in res) >= max(last[u] for u in nonres)


def test_empty_pool_everything_on_cpu():
    st = P.Residency(16, 0)
    K = P.victim_bound(1, 2, 8, 0)
    assert K == 0
    pl = P.plan(st, 1, [[3, 5]], 8, K, 25_000, 50_000, P.HYBRID)
    assert pl.q == 0 and pl.cpu == [11, 13] and pl.victims == []
    assert pl.slot_map == [[-1, -1]]


def test_capacity_caps_q():
    """More misses than non-hit slots: q stops at the free capacity."""
    st = P.Residency(64, 2)
    K = P.victim_bound(1, 8, 32, 2)
    pl = P.plan(st, 0, [list(range(8))], 32, K, 1, 1, P.OFFLOAD)
    assert pl.q == 2 and pl.cpu == list(range(2, 8))
    assert [f[1] for f in pl.fills] == [0, 1]
    pl = P.plan(st, 0, [[0, 1, 9]], 32, K, 1, 1, P.OFFLOAD)
    assert pl.hits == [0, 1] and pl.q == 0 and pl.cpu == [9]
    assert pl.victims == [-1, -1]


def test_max_fetch_caps_q():
    st = P.Residency(64, 32)
    K = P.victim_bound(1, 8, 32, 32, max_fetch=2)
    assert K == 2
    pl = P.plan(st, 0, [list(range(8))], 32, K, 1, 1, P.OFFLOAD, max_fetch=2)
    assert pl.q == 2 and len(pl.cpu) == 6


def test_victims_skip_hits_and_prefer_empty():
    st = P.Residency(32, 4)
    K = P.victim_bound(1, 2, 16, 4)
    P.plan(st, 0, [[0, 1]], 16, K, 1, 1, P.OFFLOAD)       # slots 0,1 <- 0,1 at tick 1
    pl = P.plan(st, 0, [[1, 2]], 16, K, 1, 1, P.OFFLOAD)  # hit 1, fill 2 into slot 2 (empty)
    assert pl.hits == [1] and pl.fills == [(2, 2, -1)]
    assert pl.victims == [2, 3]
    pl = P.plan(st, 1, [[0, 1]], 16, K, 1, 1, P.OFFLOAD)  # ids 16, 17
    assert pl.fills == [(16, 3, -1), (17, 0, 0)]


def test_resize_identity_full_pool_is_noop():
    rng = random.Random(9)
    st = P.Residency(40, 6)
    K = P.victim_bound(1, 3, 20, 6)
    for _ in range(50):
        P.plan(st, rng.randrange(2), [rng.sample(range(20), 3)], 20, K, 1, 1, P.OFFLOAD)
    assert all(u >= 0 for u in st.slot2id)
    before = st.copy()
    moves = P.resize(st, 6)
    assert all(a == b for a, b in moves)
    assert st.slot2id == before.slot2id and st.slot_ts == before.slot_ts
    assert st.id2slot == before.id2slot and st.tick == before.tick


def test_resize_keeps_most_recent_and_moves_forward():
    rng = random.Random(11)
    st = P.Residency(60, 12)
    K = P.victim_bound(1, 4, 30, 12)
    for _ in range(80):
        P.plan(st, rng.randrange(2), [rng.sample(range(30), 4)], 30, K, 1, 1, P.OFFLOAD)
    lru_first = sorted([s for s in range(12) if st.slot2id[s] >= 0],
                       key=lambda s: (st.slot_ts[s], s))
    keep_ids = {st.slot2id[s] for s in lru_first[-5:]}
    before = st.copy()
    moves = P.resize(st, 5)
    assert {u for u in st.slot2id if u >= 0} == keep_ids
    # survivors below the budget stay; only those beyond it move, into the
    # lowest free slots, sources and destinations disjoint
    assert all(s >= 5 > j for s, j in moves)
    assert [s for s, _ in moves] == sorted(s for s in range(5, 12) if before.slot2id[s] in keep_ids)
    for s in range(5):
        if before.slot2id[s] in keep_ids:
            assert st.slot2id[s] == before.slot2id[s] and st.slot_ts[s] == before.slot_ts[s]
    holes = [j for j in range(5) if before.slot2id[j] not in keep_ids]
    assert [j for _, j in moves] == holes[:len(moves)]
    P.resize(st, 9)
    assert st.slot2id[5:] == [-1] * 4 and st.slot_ts[5:] == [-1] * 4


def test_prefill_admit_buffers():
    L, E = 4, 8
    st = P.Residency(L * E, 2 * E + 3)
    K = P.victim_bound(1, 2, E, st.n_slots)
    for step in range(20):
        P.plan(st, step % L, [[step % E, (step * 3 + 1) % E]], E, K, 1, 1, P.OFFLOAD)
    for layer in range(L):
        b = P.prefill_admit(st, layer, E)
        assert b == layer % 2
        for e in range(E):
            assert st.slot2id[b * E + e] == layer * E + e
            assert st.id2slot[layer * E + e] == b * E + e
        held = [s for s, u in enumerate(st.slot2id) if u >= 0 and u // E == layer]
        assert sorted(held) == list(range(b * E, b * E + E))
        for s, u in enumerate(st.slot2id):
            if u >= 0:
                assert st.id2slot[u] == s
    with pytest.raises(ValueError):
        P.prefill_admit(P.Residency(L * E, 2 * E - 1), 0, E)


def test_prefill_admit_single_buffer():
    """With the second buffer disabled every layer lands in slots [0, E): the
    previous layer's experts there are evicted, a decode-resident expert of
    the new layer outside the buffer is emptied, slots past the buffer that
    hold other layers' experts keep them, and n = E suffices."""
    L, E = 3, 4
    st = P.Residency(L * E, E + 2)
    # decode leaves layer 1's expert 2 and layer 2's expert 0 in the extra slots
    st.tick = 5
    for s, u in ((E, 1 * E + 2), (E + 1, 2 * E + 0)):
        st.slot2id[s], st.id2slot[u], st.slot_ts[s] = u, s, 5
    assert P.prefill_admit(st, 0, E, buffers=1) == 0
    assert st.slot2id[:E] == [0, 1, 2, 3] and st.tick == 6
    assert st.slot2id[E:] == [E + 2, 2 * E]          # other layers' experts stay
    assert P.prefill_admit(st, 1, E, buffers=1) == 0
    assert st.slot2id[:E] == [E, E + 1, E + 2, E + 3]
    assert st.slot2id[E] == -1 and st.slot_ts[E] == -1  # its copy outside the buffer is emptied
    assert st.id2slot[E + 2] == 2
    assert all(st.id2slot[u] == -1 for u in range(E))    # layer 0 was evicted
    assert st.slot2id[E + 1] == 2 * E and st.slot_ts[E + 1] == 5
    for s, u in enumerate(st.slot2id):
        if u >= 0:
            assert st.id2slot[u] == s
    P.prefill_admit(P.Residency(L * E, E), 2, E, buffers=1)  # one buffer fits in n = E
    with pytest.raises(ValueError):
        P.prefill_admit(P.Residency(L * E, E - 1), 0, E, buffers=1)


def _warm(L, E, n, steps, seed):
    """A residency state left by offload decode over random routing."""
    rng = random.Random(seed)
    st = P.Residency(L * E, n)
    K = P.victim_bound(1, 2, E, n)
    for _ in range(steps):
        P.plan(st, rng.randrange(L), [rng.sample(range(E), 2)], E, K, 1, 1, P.OFFLOAD)
    return st


def test_prefill_on_demand_one_pass_is_single_buffer():
    """With every expert routed and n >= E, on-demand is one pass over all E
    experts into slots [0, E): the same tables as the one-buffer admission,
    pinned above, from the same decode-warmed state."""
    L, E = 3, 6
    for n in (E, E + 1, 2 * E - 1):
        for layer in range(L):
            a = _warm(L, E, n, 30, 100 * n + layer)
            b = a.copy()
            passes = P.prefill_on_demand(a, layer, list(range(E)) * 2, E)
            P.prefill_admit(b, layer, E, buffers=1)
            assert passes == [list(range(E))]
            assert (a.id2slot, a.slot2id, a.slot_ts, a.tick) == (b.id2slot, b.slot2id, b.slot_ts, b.tick)


def test_prefill_on_demand_passes_worked_example():
    """L = 2, E = 6, n = 2; decode left layer 1 expert 3 in slot 1 (tick 4)
    and layer 0 expert 5 in slot 0 (tick 3).  A layer-1 chunk that routes to
    experts {4, 1, 3, 1} runs passes [1, 3] and [4]: pass one (tick 5) puts
    u = 7 in slot 0 (evicting u = 5) and u = 9 in slot 1 (its own old slot,
    refreshed); pass two (tick 6) puts u = 10 in slot 0 (evicting u = 7);
    slot 1 keeps u = 9 with tick 5."""
    E = 6
    st = P.Residency(2 * E, 2)
    st.slot2id, st.slot_ts, st.tick = [5, 9], [3, 4], 4
    st.id2slot[5], st.id2slot[9] = 0, 1
    passes = P.prefill_on_demand(st, 1, [4, 1, 3, 1, -1, 6], E)
    assert passes == [[1, 3], [4]]
    assert st.tick == 6
    assert st.slot2id == [10, 9] and st.slot_ts == [6, 5]
    assert [u for u in range(2 * E) if st.id2slot[u] >= 0] == [9, 10]
    with pytest.raises(ValueError):
        P.prefill_on_demand(P.Residency(2 * E, 0), 0, [0], E)


def test_prefill_on_demand_invariants():
    """Random decode-warmed states and routed sets: the passes cover the
    routed experts in ascending order with at most n each, one tick per pass;
    the last pass's experts sit in slots [0, P) with the final tick; the
    other experts of the chunk are resident at most once, each with its pass's
    tick; slots past the first (largest) pass that held IDs outside the chunk
    keep them, and slots below it hold only the chunk's experts."""
    rng = random.Random(5)
    L, E = 3, 10
    for trial in range(200):
        n = rng.randrange(1, 2 * E)
        st = _warm(L, E, n, rng.randrange(0, 40), trial)
        before = st.copy()
        layer = rng.randrange(L)
        routed = [rng.randrange(E) for _ in range(rng.randrange(1, 3 * E))]
        passes = P.prefill_on_demand(st, layer, routed, E)
        flat = [e for p in passes for e in p]
        assert flat == sorted(set(routed))
        assert all(1 <= len(p) <= n for p in passes) and all(len(p) == n for p in passes[:-1])
        assert st.tick == before.tick + len(passes)
        last = passes[-1]
        assert st.slot2id[:len(last)] == [layer * E + e for e in last]
        assert st.slot_ts[:len(last)] == [st.tick] * len(last)
        chunk = {layer * E + e for e in flat}
        for s, u in enumerate(st.slot2id):
            if u >= 0:
                assert st.id2slot[u] == s
            if s >= len(passes[0]) and before.slot2id[s] not in chunk:
                assert (u, st.slot_ts[s]) == (before.slot2id[s], before.slot_ts[s])
            if s < len(passes[0]):
                assert u in chunk
        for u in chunk:
            s = st.id2slot[u]
            if s >= 0:
                pi = next(i for i, p in enumerate(passes) if u - layer * E in p)
                assert st.slot_ts[s] == before.tick + pi + 1


def test_resize_worked_example():
    """n = 6, slots hold u = 10..15 with ticks [5, 1, 6, 2, 7, 3]; resize to
    3 keeps the three most recent (ticks 7, 6, 5: slots 4, 2, 0).  Slots 0
    and 2 are below the budget and stay; slot 4 moves to the only free slot
    below it, 1.  Then growing to 5 appends two empty slots and moves
    nothing."""
    st = P.Residency(20, 6)
    st.slot2id = [10, 11, 12, 13, 14, 15]
    st.slot_ts = [5, 1, 6, 2, 7, 3]
    for s, u in enumerate(st.slot2id):
        st.id2slot[u] = s
    st.tick = 7
    assert P.resize(st, 3) == [(4, 1)]
    assert st.slot2id == [10, 14, 12] and st.slot_ts == [5, 7, 6]
    assert [st.id2slot[u] for u in range(10, 16)] == [0, -1, 2, -1, 1, -1]
    assert P.resize(st, 5) == []
    assert st.slot2id == [10, 14, 12, -1, -1] and st.slot_ts == [5, 7, 6, -1, -1]
