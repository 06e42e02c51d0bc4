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
