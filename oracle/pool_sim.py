"""Reference simulator of the bounded HBM expert slot pool (TEST INFRASTRUCTURE ONLY).

The pages keep hot routed experts in a bounded pool and evict with "LFU plus
recency" (Show HN page, how-it-works list and the prior-art paragraph;
creativeainews explainer, "How Expert Streaming Works").  They name the policy
but give no formula; this simulator follows the policy as this project reads
it, in plain Python:

* per layer, ``slots`` slots; an expert is resident in at most one slot;
* every resident expert carries (count, last_use);
* aging: counts are halved (integer shift) once per ``aging_period`` steps,
  applied lazily: when a layer is first touched in epoch step // period, each
  count is shifted right by the number of epochs since the layer's last one
  (period 0 disables aging);
* acquire(layer, experts, step), experts distinct:
    1. every requested expert that is resident is a hit: count += 1,
       last_use = step, and it is pinned;
    2. the misses, in request order, each take the lowest-numbered free slot,
       else evict the unpinned resident expert with the smallest
       (count, last_use, expert id); the new expert gets count = 1,
       last_use = step and is pinned; its blob is copied into the slot;
    3. if the misses outnumber free plus unpinned slots, nothing changes and
       the call fails (pool full);
* release(layer) unpins every slot of that layer;
* evict(layer, expert) removes an unpinned resident expert (pinned: busy;
  not resident: no-op);
* prefetch(layer, experts, step), experts distinct: a best-effort early load
  of experts predicted for a later acquire (pre-gating: the next layer's
  router applied to the current layer's input).  Aging is applied first.
  Requested experts that are resident are left as they are (no count, no
  pin).  Each other requested expert, in request order, takes the
  lowest-numbered free slot, else evicts the unpinned resident expert with the
  smallest (count, last_use, expert id) among those not requested in this
  call and not loaded by it; with no such slot it is skipped.  A loaded expert
  enters unpinned with count = 0 and last_use = step, so a correct prediction
  leaves, after the acquire that hits it (count + 1, last_use = step), the
  same entry a miss would have made; its blob is copied.

Parity status: pinned by a hand-computed trace in tests/test_oracle_pool.py.
"""
from __future__ import annotations


class PoolFull(Exception):
    pass


class PoolBusy(Exception):
    pass


class PoolSim:
    def __init__(self, n_layers: int, n_experts: int, slots: int, aging_period: int, blob_bytes: int = 0):
        if n_layers <= 0 or n_experts <= 0 or slots <= 0 or aging_period < 0:
            raise ValueError("bad pool geometry")
        self.n_layers, self.n_experts, self.slots = n_layers, n_experts, slots
        self.period = aging_period
        self.blob_bytes = blob_bytes
        self.slot_of = [[-1] * n_experts for _ in range(n_layers)]
        self.expert_in = [[-1] * slots for _ in range(n_layers)]
        self.count = [[0] * slots for _ in range(n_layers)]
        self.last_use = [[0] * slots for _ in range(n_layers)]
        self.pinned = [[False] * slots for _ in range(n_layers)]
        self.epoch = [0] * n_layers
        self.hits = self.misses = self.evictions = self.bytes_h2d = self.prefetches = 0

    def _age(self, layer: int, step: int) -> None:
        if self.period == 0:
            return
        ep = step // self.period
        if ep > self.epoch[layer]:
            shift = min(ep - self.epoch[layer], 63)
            for s in range(self.slots):
                self.count[layer][s] >>= shift
            self.epoch[layer] = ep

    def acquire(self, layer: int, experts, step: int):
        """Returns a list of (expert, hit, slot, evicted_expert_or_-1) in request order."""
        experts = [int(e) for e in experts]
        if len(set(experts)) != len(experts):
            raise ValueError("experts of one call must be distinct")
        if any(e < 0 or e >= self.n_experts for e in experts):
            raise ValueError("expert id out of range")
        slot_of = self.slot_of[layer]
        misses = [e for e in experts if slot_of[e] < 0]
        requested_resident = {slot_of[e] for e in experts if slot_of[e] >= 0}
        free = sum(1 for s in range(self.slots) if self.expert_in[layer][s] < 0)
        evictable = sum(1 for s in range(self.slots)
                        if self.expert_in[layer][s] >= 0 and not self.pinned[layer][s]
                        and s not in requested_resident)
        if len(misses) > free + evictable:
            raise PoolFull(f"layer {layer}: {len(misses)} misses, {free + evictable} slots available")
        self._age(layer, step)
        result = {}
        for e in experts:
            s = slot_of[e]
            if s >= 0:
                self.count[layer][s] += 1
                self.last_use[layer][s] = step
                self.pinned[layer][s] = True
                self.hits += 1
                result[e] = (e, True, s, -1)
        for e in misses:
            victim = -1
            free_slots = [s for s in range(self.slots) if self.expert_in[layer][s] < 0]
            if free_slots:
                s = free_slots[0]
            else:
                cands = [(self.count[layer][s], self.last_use[layer][s], self.expert_in[layer][s], s)
                         for s in range(self.slots) if not self.pinned[layer][s]]
                _, _, victim, s = min(cands)
                slot_of[victim] = -1
                self.evictions += 1
            self.expert_in[layer][s] = e
            slot_of[e] = s
            self.count[layer][s] = 1
            self.last_use[layer][s] = step
            self.pinned[layer][s] = True
            self.misses += 1
            self.bytes_h2d += self.blob_bytes
            result[e] = (e, False, s, victim)
        return [result[e] for e in experts]

    def release(self, layer: int) -> None:
        self.pinned[layer] = [False] * self.slots

    def prefetch(self, layer: int, experts, step: int):
        """Returns a list of (expert, slot, evicted_expert_or_-1) for the experts it loaded, in request order."""
        experts = [int(e) for e in experts]
        if len(set(experts)) != len(experts):
            raise ValueError("experts of one call must be distinct")
        if any(e < 0 or e >= self.n_experts for e in experts):
            raise ValueError("expert id out of range")
        self._age(layer, step)
        slot_of = self.slot_of[layer]
        keep = set(experts)            # never evicted by this call
        loaded = []
        for e in experts:
            if slot_of[e] >= 0:
                continue
            victim = -1
            free_slots = [s for s in range(self.slots) if self.expert_in[layer][s] < 0]
            if free_slots:
                s = free_slots[0]
            else:
                cands = [(self.count[layer][s], self.last_use[layer][s], self.expert_in[layer][s], s)
                         for s in range(self.slots)
                         if not self.pinned[layer][s] and self.expert_in[layer][s] not in keep]
                if not cands:
                    continue
                _, _, victim, s = min(cands)
                slot_of[victim] = -1
                self.evictions += 1
            self.expert_in[layer][s] = e
            slot_of[e] = s
            self.count[layer][s] = 0
            self.last_use[layer][s] = step
            self.prefetches += 1
            self.bytes_h2d += self.blob_bytes
            loaded.append((e, s, victim))
        return loaded

    def evict(self, layer: int, expert: int) -> None:
        s = self.slot_of[layer][expert]
        if s < 0:
            return
        if self.pinned[layer][s]:
            raise PoolBusy(f"layer {layer} expert {expert} is pinned")
        self.slot_of[layer][expert] = -1
        self.expert_in[layer][s] = -1
        self.count[layer][s] = 0
        self.last_use[layer][s] = 0
        self.evictions += 1

    def stats(self):
        return dict(hits=self.hits, misses=self.misses, evictions=self.evictions, bytes_h2d=self.bytes_h2d,
                    prefetches=self.prefetches)
