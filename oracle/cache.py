"""Refinement slot cache, deterministic mode.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

rag-lover.com StrataFlux summary, explainer dialogue (解説): precision fetched
for one decode step is kept on the GPU and reused by later steps; limitations
section: a unit that is not on the GPU when it is needed stays at resident
precision.  Paper abstract (arXiv 2611.08363): generation does not wait for every
transfer.  The pages give no policy; the reading used here:

* one pool per (layer, tensor), holding at most ``capacity`` refinement units;
* a lookup at step t marks each resident unit it asks for as used at t (a hit) and
  queues each absent one (a miss, which falls back to resident precision);
* after step t the queued misses, in the order they were asked for (duplicates
  dropped), are installed: into a free slot if there is one, else in place of the
  resident unit with the smallest (last use, unit id) among those last used
  before t; if every resident unit was used at t the miss is dropped; at most
  ``max_fill`` units are installed per fill (None = no cap, units beyond the cap are
  dropped); installed units count as used at t;
* installed units are visible to lookups from step t + 1 on.
"""
from __future__ import annotations


class LRUPool:
    def __init__(self, capacity: int):
        if capacity < 0:
            raise ValueError("capacity must be >= 0")
        self.capacity = capacity
        self.last_use = {}  # unit id -> step of last use
        self.pending = []

    def resident(self):
        return set(self.last_use)

    def lookup(self, units, step: int):
        """Returns the list of booleans hit/miss, in the order of ``units``."""
        out = []
        for u in units:
            u = int(u)
            if u in self.last_use:
                self.last_use[u] = step
                out.append(True)
            else:
                if u not in self.pending:
                    self.pending.append(u)
                out.append(False)
        return out

    def fill(self, step: int, max_fill=None):
        """Install the queued misses; returns the installed unit ids in order."""
        todo = self.pending if max_fill is None else self.pending[:max_fill]
        self.pending = []
        installed = []
        for u in todo:
            if u in self.last_use:
                continue
            if len(self.last_use) >= self.capacity:
                old = [v for v, t in self.last_use.items() if t < step]
                if not old:
                    continue
                victim = min(old, key=lambda v: (self.last_use[v], v))
                del self.last_use[victim]
            if len(self.last_use) < self.capacity:
                self.last_use[u] = step
                installed.append(u)
        return installed


class LeadPool(LRUPool):
    """An LRU pool plus ``lead`` ring slots that prefetches fill (fetch lead).

    rag-lover.com StrataFlux summary, explainer dialogue (解説), fetch lead / fetch
    lag passage: the channels a block will need are predicted from the previous
    block's residual stream and fetched ahead of it.  Reading, as a cache policy:

    * ``prefetch(units)`` (distinct ids): the ring slots come to hold the latest
      prediction.  Ring units that the prediction names stay where they are; every
      other ring slot is emptied (its unit leaves the device, unless an LRU slot
      serves it); then the predicted units that are on the device nowhere, in the
      order given, take the empty ring slots in ascending slot order (those that
      find no empty slot are not fetched);
    * a lookup hits a unit in an LRU slot (marking it used) or in a ring slot (no
      mark: a prefetched unit is not an LRU entry); misses queue as in LRUPool;
    * the fill after the step installs queued misses in the LRU slots as LRUPool
      does; a unit held by both a ring slot and an LRU slot is served by the LRU
      slot (the later mapping), and an LRU eviction takes the unit off the device.

    ``where`` maps each unit on the device to "lru" or ("ring", slot).
    """

    def __init__(self, capacity: int, lead: int):
        super().__init__(capacity)
        if lead < 0:
            raise ValueError("lead must be >= 0")
        self.lead = lead
        self.ring = [None] * lead
        self.where = {}

    def ring_units(self):
        return {u for j, u in enumerate(self.ring) if u is not None and self.where.get(u) == ("ring", j)}

    def prefetch(self, units):
        """Returns the units fetched into the ring, in order."""
        units = [int(u) for u in units]
        if len(set(units)) != len(units):
            raise ValueError("prefetch ids must be distinct")
        named = set(units)
        for j, old in enumerate(self.ring):
            if old is None or (old in named and self.where.get(old) == ("ring", j)):
                continue
            if self.where.get(old) == ("ring", j):
                del self.where[old]
            self.ring[j] = None
        free = [j for j, old in enumerate(self.ring) if old is None]
        new = [u for u in units if u not in self.where][: len(free)]
        for j, u in zip(free, new):
            self.ring[j] = u
            self.where[u] = ("ring", j)
        return new

    def lookup(self, units, step: int):
        out = []
        for u in units:
            u = int(u)
            w = self.where.get(u)
            if w == "lru":
                self.last_use[u] = step
                out.append(True)
            elif w is not None:
                out.append(True)
            else:
                if u not in self.pending and u not in self.last_use:
                    self.pending.append(u)
                out.append(False)
        return out

    def fill(self, step: int, max_fill=None):
        before = set(self.last_use)
        installed = super().fill(step, max_fill)
        for v in before - set(self.last_use):
            self.where.pop(v, None)  # evicted from an LRU slot: off the device
        for u in installed:
            self.where[u] = "lru"
        return installed
