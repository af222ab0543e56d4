"""A plain reference model of the bounded expert cache, for tests only.

Each size class owns its slots and one LRU list (or, per layer, one list per
layer over that layer's share of the slots); an expert that is not resident
takes an empty slot first (the last-created empty slot goes first), else the
least recently used entry that is not pinned (LFU: the least used since it
arrived, ties to the least recently used).  Layers are mapped to classes;
budget never moves between classes.  Sources: "RFC: stream MoE experts from disk
in from_pretrained", How the prototype works, Cache bullet (pool of slots, LRU,
each layer's map from expert to slot); "moe: expert slots in size classes", PR
description and the ExpertCache constructor in its review (a separate slot pool
and LRU for every class, unused slots handed out first; --per-layer gives each
layer a list of its own over an equal fraction); the RFC's Cache bullet (LRU,
optional LFU).

The model is written from those statements alone, with Python lists, so that a
mistake in the native cache (a wrong victim, a shared budget, a lost touch)
shows up as a different slot or count.
"""
from __future__ import annotations

import numpy as np


class ClassLRU:
    """One eviction order over a run of slots.  LRU evicts the least recently used
    entry that is not pinned; LFU the one used least often since it arrived (ties:
    the least recently used).  Empty slots go first."""

    def __init__(self, n_slots: int, first: int = 0, lfu: bool = False):
        self.free = list(range(first, first + n_slots))  # popped from the end: last-created first
        self.order: list = []             # most recently used first
        self.owner: dict = {}             # key -> slot
        self.uses: dict = {}              # key -> acquires since it arrived
        self.lfu = lfu
        self.hits = self.misses = self.evictions = 0

    def acquire(self, key, pinned=frozenset()):
        """Returns (slot, was_miss); raises LookupError when every slot is pinned."""
        if key in self.owner:
            self.hits += 1
            self.uses[key] += 1
            self.order.remove(key)
            self.order.insert(0, key)
            return self.owner[key], False
        if self.free:
            slot = self.free.pop()
        else:
            candidates = [k for k in reversed(self.order) if k not in pinned]  # least recent first
            if not candidates:
                raise LookupError("no free slot")
            victim = min(candidates, key=lambda k: self.uses[k]) if self.lfu else candidates[0]
            self.order.remove(victim)
            del self.uses[victim]
            slot = self.owner.pop(victim)
            self.evictions += 1
        self.misses += 1
        self.owner[key] = slot
        self.uses[key] = 1
        self.order.insert(0, key)
        return slot, True


class CacheModel:
    """Classes of slots; each class one eviction order, or (per_layer) its slots
    split between its layers in layer order, n // L each and one more for the
    first n % L layers, each run with its own order."""

    def __init__(self, class_slots: list[int], layer_class: list[int], E: int, lfu: bool = False,
                 per_layer: bool = False):
        self.layer_class = list(layer_class)
        self.E = E
        self.parts = []        # per class: list of ClassLRU
        self.layer_part = {}   # layer -> ClassLRU
        for c, n in enumerate(class_slots):
            layers = [l for l, k in enumerate(layer_class) if k == c] if per_layer else []
            P = max(len(layers), 1)
            parts, first = [], 0
            for i in range(P):
                cnt = n // P + (1 if i < n % P else 0)
                parts.append(ClassLRU(cnt, first, lfu))
                first += cnt
            self.parts.append(parts)
            for l in range(len(layer_class)):
                if layer_class[l] == c:
                    self.layer_part[l] = parts[layers.index(l)] if per_layer else parts[0]
        self.classes = [p[0] for p in self.parts]

    def acquire(self, layer: int, expert: int, pinned=frozenset()):
        return self.layer_part[layer].acquire((layer, expert), pinned)

    def prepare(self, layer: int, ids, last_first: bool = False) -> list[tuple[int, int, bool]]:
        """Acquire the distinct ids of one layer in order of first appearance (or,
        with last_first, in the reverse of that order, as the miss pipeline does);
        the ones acquired earlier in the same call are pinned.  Returns (expert,
        slot, miss)."""
        seen, order = set(), []
        for e in (int(v) for v in np.asarray(ids).reshape(-1)):
            if e not in seen:
                seen.add(e)
                order.append(e)
        if last_first:
            order.reverse()
        out, pinned = [], set()
        for e in order:
            slot, miss = self.acquire(layer, e, frozenset(pinned))
            pinned.add((layer, e))
            out.append((e, slot, miss))
        return out

    def table(self, layer: int) -> list[int]:
        owner = self.layer_part[layer].owner
        return [owner.get((layer, e), -1) for e in range(self.E)]

    def class_stats(self, cls: int) -> tuple[int, int, int]:
        ps = self.parts[cls]
        return (sum(p.hits for p in ps), sum(p.misses for p in ps), sum(p.evictions for p in ps))
