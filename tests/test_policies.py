"""Host logic of the placement-policy replay (the ablation of the global LRU
residency, paper.oopus.info review of FreeToken, section 2.4): the frozen
prefill hot set, the static layer split and the fixed-placement miss count
against brute-force definitions on tiny traces, and the oracle LRU's miss
counts against what the definition of LRU fixes."""
import itertools

import numpy as np

from oracle import cache as OC
from expert_ffn_execution_router_amd import policies as P


def _trace(seed, S, L, T, E, k, reuse=0.7):
    """ids [S, L, T, k]: distinct experts per token; each (layer, token) keeps
    its previous step's set with probability `reuse`."""
    rng = np.random.default_rng(seed)
    tr = np.empty((S, L, T, k), dtype=np.int32)
    pop = 1.0 / np.arange(1, E + 1) ** 1.1
    pop /= pop.sum()
    for s in range(S):
        for l in range(L):
            for t in range(T):
                if s > 0 and rng.random() < reuse:
                    tr[s, l, t] = tr[s - 1, l, t]
                else:
                    tr[s, l, t] = rng.choice(E, size=k, replace=False, p=pop)
    return tr


def _oracle_lru(trace, E, n_slots, warmup):
    S, L = trace.shape[:2]
    c = OC.SlotCache(L, E, n_slots)
    miss = uniq = 0
    for s in range(S):
        for l in range(L):
            r = c.plan(l, trace[s, l].reshape(-1), OC.POLICY_OFFLOAD)
            if s >= warmup:
                miss += r["m"]
                uniq += len(r["unique"])
    return miss, uniq


def test_prefill_hot_set_brute_force():
    rng = np.random.default_rng(1)
    L, E, Tp, k = 3, 6, 5, 2
    pre = np.stack([np.stack([rng.choice(E, k, replace=False) for _ in range(Tp)]) for _ in range(L)])
    counts = {}
    for l in range(L):
        for t in range(Tp):
            for e in pre[l, t]:
                counts[(l, int(e))] = counts.get((l, int(e)), 0) + 1
    pairs = [(l, e) for l in range(L) for e in range(E)]
    for n in range(L * E + 1):
        best = sorted(pairs, key=lambda p: (-counts.get(p, 0), p[0], p[1]))[:n]
        want = np.zeros(L * E, dtype=bool)
        for l, e in best:
            want[l * E + e] = True
        assert (P.prefill_hot_set(pre.astype(np.int32), E, n) == want).all(), n


def test_static_split_is_a_layer_prefix():
    L, E = 4, 5
    for n in range(L * E + 2):
        m = P.static_split(L, E, n)
        assert m.sum() == min(n, L * E)
        got = [(i // E, i % E) for i in np.flatnonzero(m)]
        assert got == list(itertools.islice(((l, e) for l in range(L) for e in range(E)), min(n, L * E)))


def test_fixed_replay_brute_force():
    L, E, k = 3, 10, 3
    tr = _trace(2, 12, L, 2, E, k)
    rng = np.random.default_rng(4)
    for trial in range(5):
        res = rng.random(L * E) < 0.4
        miss = uniq = 0
        for s in range(3, 12):
            for l in range(L):
                u = set(int(e) for e in tr[s, l].ravel())
                uniq += len(u)
                miss += sum(1 for e in u if not res[l * E + e])
        assert P.fixed_replay(res, tr, 3) == (miss, uniq)
    assert P.fixed_replay(np.ones(L * E, bool), tr, 0)[0] == 0
    m, u = P.fixed_replay(np.zeros(L * E, bool), tr, 0)
    assert m == u


def test_lru_full_capacity_misses_only_first_touches():
    """With a slot for every (layer, expert) nothing is evicted: the misses
    are exactly the first touches of each pair."""
    L, E, k = 3, 12, 3
    tr = _trace(5, 20, L, 2, E, k)
    seen, first = set(), 0
    for s in range(20):
        for l in range(L):
            for e in set(int(v) for v in tr[s, l].ravel()):
                if (l, e) not in seen:
                    seen.add((l, e))
                    first += 1
    assert _oracle_lru(tr, E, L * E, 0)[0] == first


def test_lru_brute_force_recency():
    """Tiny LRU replay against a direct recency simulation: each step-layer
    refreshes its routed pairs; each miss evicts the pair touched longest ago
    (ties: lowest slot, which here is the pair installed first)."""
    L, E, k, n_slots = 2, 6, 2, 5
    tr = _trace(7, 30, L, 1, E, k, reuse=0.5)
    resident = []          # (last_touch, install_order, pair)
    order = 0
    miss_ref = 0
    tick = 0
    for s in range(30):
        for l in range(L):
            tick += 1
            U = sorted(set(int(v) for v in tr[s, l].ravel()))
            cur = {p: (t, o) for t, o, p in resident}
            miss = [e for e in U if (l, e) not in cur]
            for e in U:
                if (l, e) in cur:
                    cur[(l, e)] = (tick, cur[(l, e)][1])
            miss_ref += len(miss)
            # slot ids: install order maps to slots 0.. until full, then victims reuse their slot
            resident = [(t, o, p) for p, (t, o) in cur.items()]
            for e in miss:
                if len(resident) < n_slots:
                    resident.append((tick, order, (l, e)))
                    order += 1
                else:
                    elig = [r for r in resident if r[0] != tick]
                    v = min(elig, key=lambda r: (r[0], r[1]))
                    resident.remove(v)
                    resident.append((tick, v[1], (l, e)))
    assert _oracle_lru(tr, E, n_slots, 0)[0] == miss_ref


def test_policy_ordering_on_a_skewed_trace():
    """On a popularity-skewed trace with reuse, LRU misses least and the
    routing-agnostic split most (the ordering the ablation reports)."""
    L, E, k = 4, 32, 4
    tr = _trace(11, 60, L, 1, E, k)
    pre = _trace(12, 1, L, 64, E, k, reuse=0.0)[0]
    n = int(0.3 * L * E)
    lru = _oracle_lru(tr, E, n, 10)
    hot = P.fixed_replay(P.prefill_hot_set(pre, E, n), tr, 10)
    static = P.fixed_replay(P.static_split(L, E, n), tr, 10)
    assert lru[1] == hot[1] == static[1]
    assert lru[0] < hot[0] < static[0]
