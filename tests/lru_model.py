"""A plain reference model of the bounded expert cache, for tests only.

Each size class owns its slots and one LRU list; an expert that is not resident
takes an empty slot first (the last-created empty slot goes first), else the
least recently used entry that is not pinned.  Layers are mapped to classes;
budget never moves between classes.  Sources: "RFC: stream MoE experts from disk
in from_pretrained", How the prototype works, Cache bullet (pool of slots, LRU,
per-layer expert -> slot table); "moe: expert slots in size classes", PR
description and the ExpertCache constructor in its review (own slots and LRU
per class, empty slots taken first).

The model is written from those statements alone, with Python lists, so that a
mistake in the native cache (a wrong victim, a shared budget, a lost touch)
shows up as a different slot or count.
"""
from __future__ import annotations

import numpy as np


class ClassLRU:
    def __init__(self, n_slots: int):
        self.free = list(range(n_slots))  # popped from the end: last-created first
        self.order: list = []             # most recently used first
        self.owner: dict = {}             # key -> slot
        self.hits = self.misses = self.evictions = 0

    def acquire(self, key, pinned=frozenset()):
        """Returns (slot, was_miss); raises LookupError when every slot is pinned."""
        if key in self.owner:
            self.hits += 1
            self.order.remove(key)
            self.order.insert(0, key)
            return self.owner[key], False
        if self.free:
            slot = self.free.pop()
        else:
            victim = next((k for k in reversed(self.order) if k not in pinned), None)
            if victim is None:
                raise LookupError("no free slot")
            self.order.remove(victim)
            slot = self.owner.pop(victim)
            self.evictions += 1
        self.misses += 1
        self.owner[key] = slot
        self.order.insert(0, key)
        return slot, True


class CacheModel:
    def __init__(self, class_slots: list[int], layer_class: list[int], E: int):
        self.classes = [ClassLRU(n) for n in class_slots]
        self.layer_class = list(layer_class)
        self.E = E

    def acquire(self, layer: int, expert: int, pinned=frozenset()):
        return self.classes[self.layer_class[layer]].acquire((layer, expert), pinned)

    def prepare(self, layer: int, ids) -> list[tuple[int, int, bool]]:
        """Acquire the distinct ids of one layer in order of first appearance; the
        ones acquired earlier in the same call are pinned.  Returns (expert, slot, miss)."""
        seen, out, pinned = set(), [], set()
        for e in (int(v) for v in np.asarray(ids).reshape(-1)):
            if e in seen:
                continue
            seen.add(e)
            slot, miss = self.acquire(layer, e, frozenset(pinned))
            pinned.add((layer, e))
            out.append((e, slot, miss))
        return out

    def table(self, layer: int) -> list[int]:
        owner = self.classes[self.layer_class[layer]].owner
        return [owner.get((layer, e), -1) for e in range(self.E)]

    def class_stats(self, cls: int) -> tuple[int, int, int]:
        k = self.classes[cls]
        return k.hits, k.misses, k.evictions
