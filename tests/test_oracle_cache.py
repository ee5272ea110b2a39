"""Pins of the oracle's q* split, slot cache model and link-bound prefill."""
import json
import math
import os
import random

import numpy as np

import pytest

from oracle import cache as C

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_q_star_table1_worked_example():
    g = json.load(open(os.path.join(GOLD, "table1_bandwidths.json")))
    got = [C.q_star(10, r["B_P"], r["B_H"]) for r in g["rows"]]
    assert got == g["q_star_m10_hand"]


def test_q_star_limits():
    assert C.q_star(0, 1.0, 5.0) == 0
    assert C.q_star(12, 50.0, 50.0) == 12          # B_H -> B_P: pure fill
    assert C.q_star(12, 50.0, 40.0) == 12          # B_R = 0
    assert C.q_star(1, 1.0, 1000.0) == 1           # always fill at least one
    assert C.q_star(7, 1.0, 1000.0) == 1
    assert C.q_star(5, 1.0, 3.0, C.POLICY_HOST) == 0
    assert C.q_star(5, 1.0, 3.0, C.POLICY_OFFLOAD) == 5
    assert C.q_star(4, 1.0, 8.0) == 1              # 0.5 rounds up
    assert C.q_star(4, 3.0, 8.0) == 2              # 1.5 rounds up


@pytest.mark.parametrize("m,BP,BH", [(10, 52.7, 77.3), (7, 11.8, 47.5), (33, 51.5, 178.0)])
def test_unrounded_q_star_balances_branches(m, BP, BH):
    q = m * BP / BH
    t_fill, t_cpu = C.branch_times(m, q, 1.0, BP, BH)
    assert t_fill == pytest.approx(t_cpu, rel=1e-12)


def test_prefill_link_bound_times_match_pages():
    g = json.load(open(os.path.join(GOLD, "prefill_link.json")))
    c = g["chunk"]
    t = C.link_bound_chunk_seconds(c["pool_GB"], c["B_P_GBps"])
    assert c["printed_s_min"] <= t <= c["printed_s_max"] * 1.005
    for case in g["fp4_pool"]["cases"]:
        t = C.link_bound_chunk_seconds(g["fp4_pool"]["pool_GB"], case["GBps"])
        assert abs(t - case["printed_s"]) / case["printed_s"] < 0.2
    assert C.link_bound_chunk_seconds(140.0, g["fp4_pool"]["x8_GBps_table1_laptop"]) > g["fp4_pool"]["x8_printed_min_s"]


class BruteLRU:
    """Independent list model: residents kept as [slot] -> (layer*E+e, stamp)."""

    def __init__(self, L, E, n):
        self.E, self.n = E, n
        self.slots = [None] * n
        self.tick = 0

    def where(self, g):
        for s, v in enumerate(self.slots):
            if v is not None and v[0] == g:
                return s
        return -1

    def plan(self, layer, ids, q_fn):
        self.tick += 1
        uniq = sorted(set(ids))
        miss = []
        for e in uniq:
            s = self.where(layer * self.E + e)
            if s >= 0:
                self.slots[s] = (self.slots[s][0], self.tick)
            else:
                miss.append(e)
        q = q_fn(len(miss))
        vict = []
        for e in miss[:q]:
            cands = [s for s in range(self.n) if (self.slots[s] is None or self.slots[s][1] != self.tick)]
            if not cands:
                break
            s = min(cands, key=lambda s: ((0 if self.slots[s] is None else self.slots[s][1]), s))
            self.slots[s] = (layer * self.E + e, self.tick)
            vict.append(s)
        return miss, vict


@pytest.mark.parametrize("n_slots,policy", [(6, C.POLICY_OFFLOAD), (13, C.POLICY_HYBRID), (40, C.POLICY_OFFLOAD),
                                            (3, C.POLICY_HYBRID)])
def test_slot_cache_matches_brute_force(n_slots, policy):
    L, E, k = 3, 16, 3
    rnd = random.Random(n_slots)
    ref = BruteLRU(L, E, n_slots)
    sc = C.SlotCache(L, E, n_slots)
    for step in range(60):
        for layer in range(L):
            ids = [rnd.choice(range(E if rnd.random() < 0.5 else 5)) for _ in range(4 * k)]
            p = sc.plan(layer, ids, policy, 30.0, 70.0)
            miss, vict = ref.plan(layer, ids, lambda m: C.q_star(m, 30.0, 70.0, policy))
            assert p["misses"] == miss
            assert p["victims"] == vict
            for s in range(n_slots):
                got = sc.owner[s]
                want = -1 if ref.slots[s] is None else ref.slots[s][0]
                assert got == want
            # invariants: hits and fills resident, host set not
            for e in p["hits"] + p["F"]:
                assert sc.slot_of[layer * E + e] >= 0
            for e in p["C"]:
                assert sc.slot_of[layer * E + e] < 0


def test_lru_textbook_behaviour():
    # working set <= capacity: no misses after warm-up; cyclic set of capacity+1: every access misses
    sc = C.SlotCache(1, 32, 8)
    for i in range(100):
        p = sc.plan(0, [i % 8], C.POLICY_OFFLOAD)
        if i >= 8:
            assert p["m"] == 0
    sc = C.SlotCache(1, 32, 8)
    for i in range(100):
        p = sc.plan(0, [i % 9], C.POLICY_OFFLOAD)
        assert p["m"] == 1


def test_admit_evict():
    sc = C.SlotCache(2, 8, 4)
    v = sc.admit(1, [3, 5])
    assert v == [0, 1] and sc.slot_of[8 + 3] == 0 and sc.slot_of[8 + 5] == 1
    sc.evict(1, [3])
    assert sc.slot_of[8 + 3] == -1 and sc.owner[0] == -1 and sc.last_use[0] == 0
    v = sc.admit(0, [0, 1, 2])
    assert v == [0, 2, 3]         # empty slots (stamp 0) first, lower slot first


def test_resize_keeps_most_recent():
    """Shrinking keeps the most recently used residents (review section 2.7
    rebuild under a smaller budget, LRU order of section 2.4)."""
    sc = C.SlotCache(1, 32, 8)
    for e in range(8):
        sc.plan(0, [e], C.POLICY_OFFLOAD)
    sc.resize(3)
    assert sorted(e for e in range(32) if sc.slot_of[e] >= 0) == [5, 6, 7]
    assert sc.plan(0, [7], C.POLICY_OFFLOAD)["m"] == 0
    assert sc.plan(0, [4], C.POLICY_OFFLOAD)["m"] == 1
    # growing keeps everything and adds empty slots
    sc.resize(10)
    assert sorted(e for e in range(32) if sc.slot_of[e] >= 0) == [4, 6, 7]
    assert sc.owner[3:] == [-1] * 7


def test_resize_matches_recency_list():
    """One expert per planning call (every stamp distinct): the slot cache
    with random rebuilds equals a plain recency-ordered list, miss for miss
    and resident set for resident set."""
    from collections import OrderedDict
    rng = np.random.default_rng(12)
    L, E = 3, 10
    n = 7
    sc = C.SlotCache(L, E, n)
    lru = OrderedDict()
    for step in range(600):
        if step % 50 == 49:
            n = int(rng.integers(1, 20))
            moves = sc.resize(n)
            while len(lru) > n:
                lru.popitem(last=False)
            assert all(new <= old for old, new in moves)
        l, e = int(rng.integers(0, L)), int(rng.integers(0, E))
        miss = (l, e) not in lru
        if not miss:
            lru.move_to_end((l, e))
        else:
            if len(lru) >= n:
                lru.popitem(last=False)
            lru[(l, e)] = True
        p = sc.plan(l, [e], C.POLICY_OFFLOAD)
        assert p["m"] == int(miss)
        got = {(g // E, g % E) for g in range(L * E) if sc.slot_of[g] >= 0}
        assert got == set(lru.keys())
