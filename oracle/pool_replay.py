"""Replay of the bounded expert slot pool's admission and eviction decisions.

TEST INFRASTRUCTURE (same rule as ``moe_oracle``): imported only by tests,
``__graft_entry__.smoke()`` and ``bench.py``'s CPU leg.

The pages describe the pool in words only: popular experts stay in a bounded
pool of fixed-size slots, evicted by LFU combined with recency, with a hit
rate of 43-70% ([xix] how-it-works paragraph; [digest] "Core Mechanics";
[lens] "エキスパートストリーミングの仕組み").  Reading used here and by the
GPU library's pool:

* every access (one expert of one acquire call, in list order) advances a
  global tick; a hit adds one to the slot's use count and stamps the tick;
* a miss takes the lowest-numbered free slot, else evicts the resident,
  unpinned slot with the smallest (use count, last tick, layer, expert) --
  least frequently used first, least recently used among equals; the new
  expert enters with count 1 (counts restart on admission);
* an acquired slot stays pinned until released; a miss with no free or
  unpinned slot is "pool exhausted" (experts admitted earlier in the same
  call stay resident and unpinned).

Prefetch (not in the pages, which name prefetching as open room: [lens]
"結論"; this library's own rule): experts are loaded in the given order into
free slots only -- a prefetch never evicts and stops at the first expert
that finds no free slot; it is not an access (no tick, no hit or miss); a
loaded expert enters unpinned with use count 0 and the current tick, so an
expert prefetched and never used is the first victim.  Its copies count in
bytes_h2d like a miss's.

The policy affects which accesses hit, never the layer's output.
"""

from __future__ import annotations

import heapq


class PoolExhausted(RuntimeError):
    pass


class SlotBusy(RuntimeError):
    pass


class PoolReplay:
    def __init__(self, capacity: int, stride: int = 0):
        self.capacity = int(capacity)
        self.stride = int(stride)
        self.free = list(range(self.capacity))
        heapq.heapify(self.free)
        self.slot_of = {}      # (layer, expert) -> slot
        self.count = {}        # key -> uses since admission
        self.last = {}         # key -> tick of the last use
        self.pins = {}         # key -> pin count
        self.tick = 0
        self.hits = self.misses = self.evictions = self.prefetched = 0

    # -- queries
    def resident(self, layer: int, expert: int) -> bool:
        return (layer, expert) in self.slot_of

    def stats(self) -> dict:
        return {"hits": self.hits, "misses": self.misses,
                "evictions": self.evictions, "prefetched": self.prefetched,
                "bytes_h2d": (self.misses + self.prefetched) * self.stride}

    # -- operations
    def _victim(self):
        best = None
        for key in self.slot_of:
            if self.pins.get(key, 0):
                continue
            cand = (self.count[key], self.last[key], key[0], key[1])
            if best is None or cand < best:
                best = cand
        return None if best is None else (best[2], best[3])

    def _drop(self, key):
        slot = self.slot_of.pop(key)
        del self.count[key], self.last[key]
        self.pins.pop(key, None)
        heapq.heappush(self.free, slot)
        return slot

    def acquire(self, layer: int, experts):
        """Return [(slot, was_miss)] for each expert; pins each one."""
        out = []
        pinned_now = []
        for e in experts:
            key = (int(layer), int(e))
            self.tick += 1
            if key in self.slot_of:
                self.hits += 1
                self.count[key] += 1
                self.last[key] = self.tick
                out.append((self.slot_of[key], False))
            else:
                if not self.free:
                    victim = self._victim()
                    if victim is None:
                        for k in pinned_now:
                            self.pins[k] -= 1
                        raise PoolExhausted(f"no unpinned slot for {key}")
                    self._drop(victim)
                    self.evictions += 1
                slot = heapq.heappop(self.free)
                self.slot_of[key] = slot
                self.count[key] = 1
                self.last[key] = self.tick
                self.misses += 1
                out.append((slot, True))
            self.pins[key] = self.pins.get(key, 0) + 1
            pinned_now.append(key)
        return out

    def prefetch(self, layer: int, experts) -> int:
        """Load the experts not yet resident, in order, into free slots;
        returns how many were loaded."""
        loaded = 0
        for e in experts:
            key = (int(layer), int(e))
            if key in self.slot_of:
                continue
            if not self.free:
                break
            self.slot_of[key] = heapq.heappop(self.free)
            self.count[key] = 0
            self.last[key] = self.tick
            loaded += 1
        self.prefetched += loaded
        return loaded

    def release(self, layer: int, experts):
        for e in experts:
            key = (int(layer), int(e))
            if self.pins.get(key, 0) > 0:
                self.pins[key] -= 1

    def evict(self, layer: int, expert: int):
        key = (int(layer), int(expert))
        if key not in self.slot_of:
            return
        if self.pins.get(key, 0):
            raise SlotBusy(f"{key} is pinned")
        self._drop(key)
        self.evictions += 1

    def flush(self):
        if any(self.pins.get(k, 0) for k in self.slot_of):
            raise SlotBusy("flush with pinned slots")
        for key in list(self.slot_of):
            self._drop(key)
