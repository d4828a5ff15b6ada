"""The bounded expert pool with LFU + recency eviction (oracle).

Test infrastructure only; see the package docstring.

Pages: hot experts stay in a bounded pool with LFU plus recency eviction, and
the reported hit rate is 43-70% (paotong.dev commentary, paragraph on the
bounded pool; cheshm.ai article, paragraph on how it works, which also names
bounded slot pools). The budget is --cache-gb, filled lazily (alphalab.site
field test, section on the 4.3 GB figure and FAQ item 1). With no cache hit a
token requests up to 480 experts, about 810 MiB (alphalab.site, section on SSD
reads).

The pages name the policy only. Reading taken here:
* slots = floor(budget / stride); the pool starts empty;
* per token, per layer, the chosen experts are visited in ascending expert
  index, global id gid = layer * E + e, and each visit advances a tick;
* hit: freq += 1, last = tick;
* miss: take the lowest-index empty slot, else evict the unpinned slot with
  the smallest (freq, last) (unique, because ticks are unique); the new
  entry gets freq = 1, last = tick;
* the experts of the current (token, layer) step are pinned until the step
  ends, so a step never evicts an expert it is about to use.
"""
from __future__ import annotations

import heapq
from typing import List, NamedTuple, Sequence

import numpy as np


class PoolStats(NamedTuple):
    accesses: int
    hits: int
    misses: int
    evictions: int
    h2d_bytes: int
    requested_bytes: int


class PoolSim:
    """Heap-based simulator of the policy above."""

    def __init__(self, n_slots: int, record_bytes: int):
        if n_slots <= 0:
            raise ValueError("pool needs at least one slot")
        self.n_slots = n_slots
        self.record_bytes = record_bytes
        self.slot_gid = [-1] * n_slots
        self.freq = [0] * n_slots
        self.last = [0] * n_slots
        self.pinned = [False] * n_slots
        self.where = {}            # gid -> slot
        self.heap = []             # (freq, last, slot) entries, stale ones skipped
        self.next_empty = 0        # slots fill in index order and never empty again
        self.tick = 0
        self.accesses = self.hits = self.misses = self.evictions = 0
        self.trace_hit: List[int] = []
        self.trace_victim: List[int] = []
        self.trace_slot: List[int] = []

    def _victim(self) -> int:
        held = []
        while True:
            f, l, s = heapq.heappop(self.heap)
            if self.freq[s] != f or self.last[s] != l or self.slot_gid[s] < 0:
                continue                      # stale entry
            if self.pinned[s]:
                held.append((f, l, s))
                continue
            for h in held:
                heapq.heappush(self.heap, h)
            return s

    def step(self, gids: Sequence[int]) -> None:
        """One (token, layer) step: visit ``gids`` in ascending order, then unpin."""
        touched = []
        for gid in sorted(int(g) for g in gids):
            self.tick += 1
            self.accesses += 1
            s = self.where.get(gid)
            if s is not None:
                self.hits += 1
                self.freq[s] += 1
                self.last[s] = self.tick
                heapq.heappush(self.heap, (self.freq[s], self.last[s], s))
                self.trace_hit.append(1)
                self.trace_victim.append(-1)
            else:
                self.misses += 1
                victim = -1
                if self.next_empty < self.n_slots:
                    s = self.next_empty
                    self.next_empty += 1
                else:
                    s = self._victim()
                    victim = self.slot_gid[s]
                    del self.where[victim]
                    self.evictions += 1
                self.slot_gid[s] = gid
                self.where[gid] = s
                self.freq[s] = 1
                self.last[s] = self.tick
                heapq.heappush(self.heap, (1, self.tick, s))
                self.trace_hit.append(0)
                self.trace_victim.append(victim)
            self.trace_slot.append(s)
            self.pinned[s] = True
            touched.append(s)
        for s in touched:
            self.pinned[s] = False

    def stats(self) -> PoolStats:
        return PoolStats(self.accesses, self.hits, self.misses, self.evictions,
                         self.misses * self.record_bytes, self.accesses * self.record_bytes)


class PoolSimNaive:
    """Brute-force twin: a full scan of every slot on each access. Used only to pin PoolSim."""

    def __init__(self, n_slots: int, record_bytes: int):
        self.n = n_slots
        self.record_bytes = record_bytes
        self.slots = [None] * n_slots      # each: [gid, freq, last]
        self.tick = 0
        self.trace_hit: List[int] = []
        self.trace_victim: List[int] = []
        self.trace_slot: List[int] = []

    def step(self, gids: Sequence[int]) -> None:
        pinned = set()
        for gid in sorted(int(g) for g in gids):
            self.tick += 1
            found = [i for i, sl in enumerate(self.slots) if sl is not None and sl[0] == gid]
            if found:
                i = found[0]
                self.slots[i][1] += 1
                self.slots[i][2] = self.tick
                self.trace_hit.append(1)
                self.trace_victim.append(-1)
            else:
                empty = [i for i, sl in enumerate(self.slots) if sl is None]
                if empty:
                    i = empty[0]
                    victim = -1
                else:
                    cands = [(sl[1], sl[2], i) for i, sl in enumerate(self.slots) if i not in pinned]
                    _, _, i = min(cands)
                    victim = self.slots[i][0]
                self.slots[i] = [gid, 1, self.tick]
                self.trace_hit.append(0)
                self.trace_victim.append(victim)
            self.trace_slot.append(i)
            pinned.add(i)


def replay(n_slots: int, record_bytes: int, idx_per_step: np.ndarray, n_experts: int,
           layers_per_token: int) -> PoolSim:
    """Replay a routing trace idx[step][k] (steps ordered token-major, layer-minor) through PoolSim."""
    sim = PoolSim(n_slots, record_bytes)
    idx_per_step = np.asarray(idx_per_step)
    for s in range(idx_per_step.shape[0]):
        layer = s % layers_per_token
        sim.step(layer * n_experts + idx_per_step[s])
    return sim
