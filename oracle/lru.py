"""Strict LRU page cache with pinning (oracle; test infrastructure only).

Source: GLM5.3 sparse-attention page, HiSparse paragraph: KV entries move from
device HBM to host DRAM; the HBM part acts as an LRU cache, a top-k miss loads
from DRAM, eviction follows LRU; the loads of layer N overlap the execution of
layer N-1.  The state-snapshot page ("cat-it-di-nho-nhieu-hon", section "Lợi
ích thì đo được rõ") shows the policy's cliff: 256 slots and 500 items sent in
the same order twice give almost no reuse, random order about half.

Readings (the pages fix none of this):

* the cache unit is one page (a key such as (layer, request, logical page));
* a touch of a resident key is a hit and makes it most recent;
* a touch of an absent key is a miss: it takes a free slot if there is one,
  else the least recently touched key that is not pinned is evicted;
* keys touched for a layer stay pinned until that layer is released (the
  layer being computed and the one being fetched are both in flight);
* every key has a full backing copy in host memory, so eviction writes
  nothing back.
"""
from __future__ import annotations

from collections import OrderedDict


class LRUCache:
    def __init__(self, capacity: int):
        if capacity <= 0:
            raise ValueError("capacity must be positive")
        self.capacity = int(capacity)
        self.slots = OrderedDict()       # key -> slot, least recent first
        self.free = list(range(self.capacity - 1, -1, -1))   # pop() gives 0, 1, 2, ...
        self.pins = {}                   # tag -> set of keys
        self.pin_count = {}              # key -> number of tags pinning it
        self.hits = self.misses = self.evictions = 0

    def preload(self, keys):
        """Make ``keys`` resident in this order (first = least recent), uncounted."""
        for key in keys:
            if key in self.slots:
                self.slots.move_to_end(key)
                continue
            self._insert(key)

    def _insert(self, key):
        if self.free:
            slot = self.free.pop()
        else:
            victim = None
            for cand in self.slots:          # least recent first
                if self.pin_count.get(cand, 0) == 0:
                    victim = cand
                    break
            if victim is None:
                raise MemoryError("every resident page is pinned")
            slot = self.slots.pop(victim)
            self.evictions += 1
        self.slots[key] = slot
        return slot

    def touch(self, key, tag=None):
        """Touch one key; returns (slot, hit)."""
        if key in self.slots:
            self.slots.move_to_end(key)
            self.hits += 1
            slot, hit = self.slots[key], True
        else:
            self.misses += 1
            slot, hit = self._insert(key), False
        if tag is not None:
            s = self.pins.setdefault(tag, set())
            if key not in s:
                s.add(key)
                self.pin_count[key] = self.pin_count.get(key, 0) + 1
        return slot, hit

    def release(self, tag):
        for key in self.pins.pop(tag, ()):
            c = self.pin_count[key] - 1
            if c:
                self.pin_count[key] = c
            else:
                del self.pin_count[key]

    @property
    def hit_rate(self) -> float:
        n = self.hits + self.misses
        return self.hits / n if n else 0.0


def pages_of_positions(positions, page_size: int):
    """Distinct logical pages, ascending, touched by a set of token positions."""
    return sorted({int(p) // int(page_size) for p in positions if int(p) >= 0})


def plan_layer(cache: LRUCache, layer: int, num_req: int, pages_per_req: int, positions,
               page_size: int, tag):
    """One layer's plan under the tiered-cache policy: for each request in order, touch the
    distinct pages its positions fall in, ascending, pinned under ``tag``.  The key of page
    ``p`` of request ``r`` in ``layer`` is (layer * num_req + r) * pages_per_req + p.
    Returns the slot table [len(positions)][pages_per_req] (-1 where untouched)."""
    import numpy as np
    table = np.full((len(positions), pages_per_req), -1, dtype=np.int32)
    for r, pos in enumerate(positions):
        for page in pages_of_positions(pos, page_size):
            if page >= pages_per_req:
                continue
            key = (layer * num_req + r) * pages_per_req + page
            slot, _ = cache.touch(key, tag)
            table[r, page] = slot
    return table
