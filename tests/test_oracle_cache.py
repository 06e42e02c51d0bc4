"""Pins for the oracle's refinement cache (CPU only).

Reuse across decode steps follows the rag-lover.com StrataFlux summary's
explainer dialogue; the miss fallback its limitations section.  Pins: a hand trace
with known outcome, and a second, independently structured LRU (slot array with
stamps, linear scan) on random traces.
"""
import numpy as np
import pytest

from oracle.cache import LeadPool, LRUPool


def test_hand_trace():
    p = LRUPool(3)
    assert p.lookup([5, 2, 9], 0) == [False, False, False]
    assert p.fill(0) == [5, 2, 9]
    assert p.lookup([2, 7], 1) == [True, False]
    # victim among last_use < 1: units 5 and 9 (last used at 0) -> smallest id 5
    assert p.fill(1) == [7]
    assert p.resident() == {2, 7, 9}
    assert p.lookup([9, 2, 7, 4, 1], 2) == [True, True, True, False, False]
    # every resident unit used at step 2: misses dropped
    assert p.fill(2) == []
    assert p.resident() == {2, 7, 9}
    assert p.lookup([4], 3) == [False]
    # oldest: 9, 2, 7 all used at 2 -> smallest id 2
    assert p.fill(3) == [4]
    assert p.resident() == {4, 7, 9}


def test_capacity_zero_and_cap():
    p = LRUPool(0)
    p.lookup([1, 2], 0)
    assert p.fill(0) == [] and p.resident() == set()
    p = LRUPool(10)
    p.lookup([3, 1, 2, 3], 0)
    assert p.fill(0, max_fill=2) == [3, 1]
    assert p.lookup([2], 1) == [False]


class SlotLRU:
    """Independent model: fixed slot array of [unit, stamp], linear scans."""

    def __init__(self, cap):
        self.slots = [None] * cap
        self.queue = []

    def lookup(self, units, t):
        res = []
        for u in units:
            idx = [i for i, s in enumerate(self.slots) if s is not None and s[0] == u]
            if idx:
                self.slots[idx[0]][1] = t
                res.append(True)
            else:
                if u not in self.queue:
                    self.queue.append(u)
                res.append(False)
        return res

    def fill(self, t, cap=None):
        q = self.queue if cap is None else self.queue[:cap]
        self.queue = []
        for u in q:
            free = [i for i, s in enumerate(self.slots) if s is None]
            if free:
                self.slots[free[0]] = [u, t]
                continue
            cands = [(s[1], s[0], i) for i, s in enumerate(self.slots) if s[1] < t]
            if cands:
                _, _, i = min(cands)
                self.slots[i] = [u, t]

    def resident(self):
        return {s[0] for s in self.slots if s is not None}


@pytest.mark.parametrize("seed", range(8))
def test_matches_slot_model(seed):
    g = np.random.default_rng(seed)
    cap = int(g.integers(0, 12))
    a, b = LRUPool(cap), SlotLRU(cap)
    for t in range(40):
        for _ in range(int(g.integers(1, 3))):
            units = g.integers(0, 25, size=int(g.integers(0, 9))).tolist()
            assert a.lookup(units, t) == b.lookup(units, t)
        c = None if g.random() < 0.5 else int(g.integers(0, 5))
        a.fill(t, c)
        b.fill(t, c)
        assert a.resident() == b.resident()


def test_warm_full_capacity_all_hits():
    p = LRUPool(100)
    g = np.random.default_rng(3)
    seen = set()
    for t in range(6):
        sel = g.choice(100, 20, replace=False).tolist()
        hits = p.lookup(sel, t)
        # with room for every unit, exactly the units seen at earlier steps hit
        assert hits == [u in seen for u in sel]
        p.fill(t)
        seen |= set(sel)
    p.lookup(list(range(100)), 6)
    p.fill(6)
    assert all(p.lookup(list(range(100)), 7))


def test_lead_hand_trace():
    """Capacity 2, 2 ring slots: prefetched units hit without an LRU mark; the ring
    keeps what the new prediction names and empties the rest; fills go to the LRU."""
    p = LeadPool(2, 2)
    assert p.prefetch([4, 7, 9]) == [4, 7]  # 9 finds no empty ring slot
    assert p.ring == [4, 7]
    assert p.lookup([7, 9, 4], 0) == [True, False, True]
    assert p.fill(0) == [9]
    assert p.resident() == {9} and p.ring_units() == {4, 7}
    assert p.prefetch([7, 9, 1]) == [1]  # 7 stays in slot 1, 4 leaves slot 0 for 1; 9 is in the LRU
    assert p.ring == [1, 7]
    assert p.lookup([4, 1, 9, 7], 1) == [False, True, True, True]
    assert p.fill(1) == [4]  # a free LRU slot
    assert p.resident() == {9, 4}
    assert p.prefetch([5]) == [5]  # both ring slots emptied, 5 takes slot 0
    assert p.ring == [5, None]
    assert p.lookup([1, 7, 5, 4], 2) == [False, False, True, True]
    # queued 1 then 7; LRU: 4 used at 2, 9 last at 1 -> 9 goes for 1; then 7 finds
    # only 4 and 1, both used or installed at 2 -> dropped
    assert p.fill(2) == [1]
    assert p.resident() == {4, 1} and p.ring_units() == {5}
    assert p.lookup([9], 3) == [False]


def test_lead_ring_loses_to_a_later_lru_install():
    """A unit queued as a miss and prefetched before the fill ends up in its LRU slot;
    emptying its ring slot later leaves it on the device, an LRU eviction does not."""
    p = LeadPool(1, 1)
    assert p.lookup([3], 0) == [False]
    assert p.prefetch([3]) == [3]
    assert p.fill(0) == [3]
    assert p.where[3] == "lru"
    assert p.prefetch([8]) == [8]  # ring slot 0 no longer serves 3
    assert p.lookup([3, 8], 1) == [True, True]
    assert p.lookup([6], 2) == [False]
    assert p.fill(2) == [6]  # 3 (last used 1) evicted
    assert p.lookup([3, 8, 6], 3) == [False, True, True]
    with pytest.raises(ValueError):
        p.prefetch([1, 1])


@pytest.mark.parametrize("seed", range(6))
def test_lead_zero_is_the_lru(seed):
    """Without ring slots (and without prefetches) the policy is LRUPool's."""
    g = np.random.default_rng(seed)
    a, b = LRUPool(7), LeadPool(7, 0)
    for t in range(30):
        units = g.integers(0, 20, size=g.integers(1, 9)).tolist()
        assert a.lookup(units, t) == b.lookup(units, t)
        assert a.fill(t) == b.fill(t)
        assert a.resident() == b.resident()


@pytest.mark.parametrize("seed", range(6))
def test_lead_prefetched_units_hit(seed):
    """Right after a prefetch of at most `lead` new units, every unit asked for is on
    the device; the LRU state is untouched by the prefetch itself."""
    g = np.random.default_rng(100 + seed)
    p = LeadPool(5, 6)
    for t in range(20):
        want = [int(u) for u in g.choice(40, size=6, replace=False)]
        lru_before = dict(p.last_use)
        p.prefetch(want)
        assert p.last_use == lru_before
        assert all(p.lookup(want, t))
        p.lookup(g.integers(0, 40, size=4).tolist(), t)
        p.fill(t)
