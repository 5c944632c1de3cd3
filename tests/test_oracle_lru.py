"""Pins for oracle/lru.py (the per-layer LRU / wave simulator)."""
import itertools
import math

import numpy as np
import pytest

from oracle.lru import LayerLRU


class HistoryLRU:
    """Brute force in another formulation: no stored last_use.  Keeps the full
    log of waves and the slot contents; a slot's recency is recomputed each time
    by scanning the log backwards for the last wave that contained its expert."""

    def __init__(self, E, K):
        self.E, self.K = E, K
        self.slots = [None] * K
        self.log = []               # list of sets, one per wave, in order

    def recency(self, j):
        if self.slots[j] is None:
            return 0
        for n in range(len(self.log) - 1, -1, -1):
            if self.slots[j] in self.log[n]:
                return n + 1
        raise AssertionError("occupant never used")

    def step(self, ids):
        present = sorted(set(int(e) for e in ids if 0 <= e < self.E))
        held = set(s for s in self.slots if s is not None)
        order = [e for e in present if e in held] + [e for e in present if e not in held]
        out = []
        for i in range(0, len(order), self.K):
            wave = order[i:i + self.K]
            ws = set(wave)
            need = sorted(e for e in wave if e not in self.slots)
            free = sorted((j for j in range(self.K) if self.slots[j] not in ws),
                          key=lambda j: (self.recency(j), j))
            plan = []
            for e, j in zip(need, free):
                plan.append((e, j, -1 if self.slots[j] is None else self.slots[j]))
                self.slots[j] = e
            self.log.append(ws)
            out.append((wave, plan))
        return out


def _compare(E, K, trace):
    a, b = LayerLRU(E, K), HistoryLRU(E, K)
    for ids in trace:
        wa = a.step(ids)
        wb = b.step(ids)
        assert [w.experts for w in wa] == [w for w, _ in wb]
        assert [list(zip(w.plan_experts, w.plan_slots, w.evicted)) for w in wa] == [p for _, p in wb]
        assert a.slot_expert == [-1 if s is None else s for s in b.slots]


def test_exhaustive_small_vs_history_scan():
    E = 3
    for K in (1, 2, 3):
        for T in (1, 2):
            steps = list(itertools.product(range(E), repeat=T))
            for trace in itertools.product(steps, repeat=4):
                _compare(E, K, trace)


@pytest.mark.parametrize("E,K,tok,k", [(4, 1, 3, 2), (4, 2, 3, 2), (4, 3, 2, 2), (6, 2, 4, 3),
                                       (8, 4, 1, 2), (16, 5, 8, 4), (32, 7, 16, 4)])
def test_random_traces_vs_history_scan(E, K, tok, k):
    rng = np.random.default_rng(E * 100 + K)
    trace = [np.concatenate([rng.choice(E, k, replace=False) for _ in range(rng.integers(1, tok + 1))])
             for _ in range(60)]
    _compare(E, K, trace)


def _check_invariants(sim, ids, waves, resident_before):
    E, K = sim.E, sim.K
    D = sorted(set(int(e) for e in ids if 0 <= e < E))
    assert len(waves) == math.ceil(len(D) / K)
    assert sorted(e for w in waves for e in w.experts) == D
    # resident experts all sit in wave 1
    if waves:
        assert set(e for e in D if e in resident_before) <= set(waves[0].experts)
    for w in waves:
        ws = set(w.experts)
        assert len(w.experts) <= K
        assert not (set(w.evicted) & ws)                         # no eviction inside the wave
        assert w.count == len([e for e in w.experts if e not in resident_before and e in w.plan_experts])
        for e in w.experts:                                      # every routed expert is resident when used
            assert w.slot_of[e] >= 0
        assert len(set(w.plan_slots)) == len(w.plan_slots)
    # table is injective and consistent
    occ = [e for e in sim.slot_expert if e >= 0]
    assert len(occ) == len(set(occ))
    for j, e in enumerate(sim.slot_expert):
        if e >= 0:
            assert sim.expert_slot[e] == j
    for e in range(E):
        if sim.expert_slot[e] >= 0:
            assert sim.slot_expert[sim.expert_slot[e]] == e


def test_invariants_on_long_traces():
    rng = np.random.default_rng(5)
    for E, K, k, T in ((128, 40, 8, 1), (128, 26, 8, 4), (128, 92, 8, 64), (16, 4, 2, 3)):
        sim = LayerLRU(E, K)
        for s in range(200):
            ids = np.concatenate([rng.choice(E, k, replace=False) for _ in range(T)])
            before = set(e for e in sim.slot_expert if e >= 0)
            waves = sim.step(ids)
            _check_invariants(sim, ids, waves, before)
            # a single wave's misses are exactly the non-resident experts
            if len(waves) == 1:
                assert sorted(waves[0].plan_experts) == sorted(set(ids.tolist()) - before)


def test_k_equals_e_pages_each_expert_once():
    rng = np.random.default_rng(6)
    E = 16
    sim = LayerLRU(E, E)
    seen = set()
    for s in range(100):
        ids = rng.choice(E, 3, replace=False)
        waves = sim.step(ids)
        new = set(ids.tolist()) - seen
        assert sorted(waves[0].plan_experts) == sorted(new)
        assert all(v == -1 for v in waves[0].evicted)
        seen |= new


def test_working_set_within_k_stops_missing():
    rng = np.random.default_rng(7)
    E, K = 64, 10
    ws = rng.choice(E, K, replace=False)
    sim = LayerLRU(E, K)
    misses = []
    for s in range(300):
        waves = sim.step(rng.choice(ws, 3, replace=False))
        misses.append(sum(w.count for w in waves))
    assert sum(misses) == K
    assert sum(misses[100:]) == 0


def test_uniform_iid_miss_rate_is_one_minus_k_over_e():
    """i.i.d. uniform single requests: by symmetry the hit rate of any K-of-E
    table is K/E, so the miss rate is 1 - K/E (the blog's uniform baseline)."""
    rng = np.random.default_rng(8)
    for E, K in ((128, 40), (128, 92), (20, 5)):
        sim = LayerLRU(E, K)
        n = 40000
        ids = rng.integers(0, E, n)
        miss = 0
        for s in range(n):
            w = sim.step([ids[s]])
            if s >= 2 * E:
                miss += w[0].count
        m = n - 2 * E
        p = 1 - K / E
        assert abs(miss / m - p) < 5 * math.sqrt(p * (1 - p) / m)


def test_lru_evicts_least_recent_outside_wave():
    sim = LayerLRU(5, 3)
    sim.step([0])            # tick 1: slot 0 <- 0
    sim.step([1])            # tick 2: slot 1 <- 1
    sim.step([2])            # tick 3: slot 2 <- 2
    sim.step([0])            # tick 4: 0 refreshed
    w, = sim.step([3])       # LRU outside wave is expert 1 (tick 2)
    assert (w.plan_experts, w.plan_slots, w.evicted) == ([3], [1], [1])
    w, = sim.step([3, 2, 4])  # resident 2, 3 stay; victim must be slot 0 (expert 0)
    assert w.experts == [2, 3, 4]
    assert (w.plan_experts, w.plan_slots, w.evicted) == ([4], [0], [0])


def test_multi_wave_resident_first_and_ticks():
    sim = LayerLRU(10, 3)
    sim.step([7, 8])
    waves = sim.step([1, 2, 3, 7, 9])
    assert [w.experts for w in waves] == [[7, 1, 2], [3, 9]]
    # wave 1 keeps 7 (slot 0); the empty slot 2 goes first, then slot 1 (expert 8)
    assert (waves[0].plan_experts, waves[0].plan_slots, waves[0].evicted) == ([1, 2], [2, 1], [-1, 8])
    # wave 2: every slot holds a wave-1 expert with the same tick, so slot order decides
    assert (waves[1].plan_experts, waves[1].plan_slots, waves[1].evicted) == ([3, 9], [0, 1], [7, 2])
    assert sim.tick == 4


def test_reset_restores_empty_table():
    sim = LayerLRU(8, 4)
    sim.step([1, 2, 3])
    sim.reset()
    assert sim.state() == ([-1] * 4, [0] * 4, 1)
    w, = sim.step([5])
    assert w.plan_slots == [0]


def test_invalid_ids_are_ignored():
    sim = LayerLRU(8, 4)
    w, = sim.step([-1, 3, 8, 100])
    assert w.experts == [3]
