"""An independent model of the residency policy for checking the oracle.

It keeps the slots in an OrderedDict ordered from least to most recently used
(a recency list, not timestamps).  After each call the slots the call touched
move to the most-recent end in ascending slot order, which is the batch
semantics the oracle expresses with one tick per call and (tick, slot)
ordering.  Each slot also remembers the number of the call that last touched
it, only so that a resize, which renumbers slots, can put the slots one call
touched back in ascending order of their new numbers.  The split q uses
Python's round() on exact fractions.
"""
from collections import OrderedDict
from fractions import Fraction

HYBRID, OFFLOAD, CPU = 0, 1, 2


class RecencySim:
    def __init__(self, n_slots):
        self.order = OrderedDict((s, None) for s in range(n_slots))
        self.where = {}
        self.stamp = {}
        self.calls = 0

    @property
    def n(self):
        return len(self.order)

    def copy(self):
        c = RecencySim(0)
        c.order = OrderedDict(self.order)
        c.where = dict(self.where)
        c.stamp = dict(self.stamp)
        c.calls = self.calls
        return c

    def call(self, layer, ids, E, K, bp, bh, mode, max_fetch=0):
        uniq = sorted({layer * E + int(e) for row in ids for e in row})
        hits = [u for u in uniq if u in self.where]
        misses = [u for u in uniq if u not in self.where]
        m = len(misses)
        if m == 0 or mode == CPU:
            q = 0
        elif mode == OFFLOAD:
            q = m
        else:
            q = min(max(1, round(Fraction(m * bp, bh))), m)
        if max_fetch > 0:
            q = min(q, max_fetch)
        q = min(q, self.n - len(hits))
        hit_slots = {self.where[u] for u in hits}
        free_order = [s for s in self.order if s not in hit_slots]
        victims = free_order[:K] + [-1] * max(0, K - len(free_order))
        fills = []
        for i in range(q):
            s, u = victims[i], misses[i]
            old = self.order[s]
            if old is not None:
                del self.where[old]
            self.order[s] = u
            self.where[u] = s
            fills.append((u, s, -1 if old is None else old))
        self.calls += 1
        for s in sorted(hit_slots | {v for v in victims[:q]}):
            self.order.move_to_end(s)
            self.stamp[s] = self.calls
        slot_map = [[self.where.get(layer * E + int(e), -1) for e in row] for row in ids]
        return dict(uniq=uniq, hits=hits, misses=misses, q=q, victims=victims, fills=fills,
                    cpu=misses[q:], slot_map=slot_map)

    def resize(self, n_new):
        occupied = [s for s, u in self.order.items() if u is not None]   # LRU -> MRU
        keep = occupied[len(occupied) - min(n_new, len(occupied)):]
        for s in occupied:
            if s not in keep:
                del self.where[self.order[s]]
        # survivors below the budget keep their slot; the rest take the
        # lowest free slots below it, in ascending order of their old slot
        stay = {s for s in keep if s < n_new}
        holes = iter(j for j in range(n_new) if j not in stay)
        renum = {s: (s if s in stay else next(holes)) for s in sorted(keep)}
        taken = set(renum.values())
        new = OrderedDict((j, None) for j in range(n_new) if j not in taken)
        stamp = {renum[s]: self.stamp[s] for s in keep}
        for s in sorted(keep, key=lambda s: (self.stamp[s], renum[s])):
            u = self.order[s]
            new[renum[s]] = u
            self.where[u] = renum[s]
        self.order = new
        self.stamp = stamp

    def recency_order(self):
        return list(self.order.keys())

    def slot2id(self):
        return [(-1 if self.order[s] is None else self.order[s]) for s in range(self.n)]
