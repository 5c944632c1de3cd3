"""Per-layer LRU / wave simulator.  TEST INFRASTRUCTURE (oracle).

Implements steps 1-2 of "A step: waves, page-in, merge" on the SGLang Paged
Experts docs page.  Given the experts one forward step of one layer routes
to, it forms groups ("waves") of at most K of them, the ones already holding
a slot placed first; before a wave runs, every expert of the wave that holds
no slot is given one, taken from an expert the wave does not use, the one
whose last use lies furthest back first; only those experts are copied from
the host.  There is one K-slot table per MoE layer ("The K-slot table and the
host store"), and one LRU state per layer whether the step was captured or
not ("Captured decode").

Readings where the page is silent:
- distinct experts are ordered resident-first, each part by ascending id;
- waves are consecutive chunks of K of that order;
- one wave is one use: every expert of the wave gets last_use = tick, and
  tick grows by one per wave;
- evictable slots are those whose expert is not in the wave (empty slots
  have last_use 0, below every tick, so they go first); victims are taken by
  ascending (last_use, slot index) and exactly as many as there are misses;
- the i-th missing expert (ascending id) goes to the i-th victim;
- a fresh or reset table is empty (slot_expert = -1, last_use = 0, tick = 1);
- ids outside [0, E) are ignored.
"""
from dataclasses import dataclass, field
from typing import List


@dataclass
class Wave:
    experts: List[int]          # the wave's experts, in wave order
    plan_experts: List[int]     # missing experts paged in, in plan order
    plan_slots: List[int]       # slot each one is copied into
    evicted: List[int]          # previous occupant of that slot (-1 if empty)
    slot_of: dict = field(default_factory=dict)   # expert -> slot after the wave

    @property
    def count(self) -> int:
        return len(self.plan_experts)


class LayerLRU:
    def __init__(self, num_experts: int, num_resident: int):
        if num_resident < 1 or num_resident > num_experts:
            raise ValueError("need 1 <= K <= E")
        self.E = num_experts
        self.K = num_resident
        self.reset()

    def reset(self):
        self.slot_expert = [-1] * self.K
        self.expert_slot = [-1] * self.E
        self.last_use = [0] * self.K
        self.tick = 1

    def state(self):
        return list(self.slot_expert), list(self.last_use), self.tick

    def split_waves(self, ids) -> List[List[int]]:
        """Step 1: distinct valid ids, resident ones first (each part ascending), in chunks of K."""
        distinct = sorted({int(e) for e in ids if 0 <= int(e) < self.E})
        resident = [e for e in distinct if self.expert_slot[e] >= 0]
        missing = [e for e in distinct if self.expert_slot[e] < 0]
        order = resident + missing
        return [order[i:i + self.K] for i in range(0, len(order), self.K)]

    def run_wave(self, wave: List[int]) -> Wave:
        """Step 2 for one wave: evict LRU slots outside the wave, place the misses."""
        in_wave = set(wave)
        miss = [e for e in wave if self.expert_slot[e] < 0]
        cand = sorted((self.last_use[j], j) for j in range(self.K)
                      if self.slot_expert[j] not in in_wave)
        assert len(cand) >= len(miss)
        plan_e, plan_s, evicted = [], [], []
        for r, e in enumerate(miss):
            j = cand[r][1]
            old = self.slot_expert[j]
            if old >= 0:
                self.expert_slot[old] = -1
            self.slot_expert[j] = e
            self.expert_slot[e] = j
            plan_e.append(e)
            plan_s.append(j)
            evicted.append(old)
        for e in wave:
            self.last_use[self.expert_slot[e]] = self.tick
        self.tick += 1
        return Wave(list(wave), plan_e, plan_s, evicted, {e: self.expert_slot[e] for e in wave})

    def step(self, ids) -> List[Wave]:
        """All waves of one forward step of this layer."""
        return [self.run_wave(w) for w in self.split_waves(ids)]
