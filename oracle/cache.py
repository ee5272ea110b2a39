"""Reference model of the expert slot cache, the miss split and the link-bound
prefill time.

TEST INFRASTRUCTURE ONLY: nothing on the product path imports this module.

Sources (paper.oopus.info review of FreeToken):
  * section 2: one slot holds every tensor of one (layer, expert); residency
    and lookup use only the logical id; the cache never changes the output;
  * section 2.2: two full-layer buffers taken from the same slot pool; the
    next layer's complete expert set is copied while the current one computes;
    chunk time equals pool bytes over the link bandwidth when compute hides;
  * section 2.4: one global LRU shared by all MoE layers: a hit refreshes the
    expert's recency, a miss admits the expert and evicts the least recently
    needed one;
  * section 2.5: the miss set M splits into a fill set F and a host set C,
    q = |F|; with B_R = max(B_H - B_P, 0), T_fill = qS/B_P and
    T_cpu = (m-q)S/(B_H-B_P) balance at q* = m B_P / B_H; q* is rounded to
    the nearest integer and at least one expert is always filled; which
    misses enter F is left to the replacement policy; C does not change
    residency;
  * section 2.6: one pass finds K least-recently-used candidate slots and the
    miss path takes the first q of them;
  * section 2.7: at a scheduler safe point the GPU expert cache is rebuilt
    under a revised memory budget without restarting or reloading the host
    pool; the output never depends on the cache size (section 2).
Readings where the pages leave a step open:
  * "rounded to the nearest integer" = floor(x + 0.5) (round half up);
  * B_H <= B_P leaves no residual host bandwidth, so q = m;
  * F = the q misses with the smallest expert ids;
  * victims: slots not stamped in the current tick, smallest last-use stamp
    first, ties to the lower slot; empty slots carry stamp 0 so they go
    first; the i-th smallest expert of F goes to the i-th victim;
  * one tick per planning call; hits and fills are stamped with it;
  * if fewer slots are eligible than q, q shrinks to the eligible count and
    the rest of M joins C (capacity cap);
  * a rebuild to n' slots keeps the n' most recently used residents (last-use
    stamp descending, ties to the lower slot), with their stamps; survivors
    are packed into slots 0, 1, ... in the order of their old slots; the
    clock keeps running.
"""
from __future__ import annotations

import math

POLICY_OFFLOAD, POLICY_HOST, POLICY_HYBRID = 0, 1, 2


def q_star(m: int, B_P: float, B_H: float, policy: int = POLICY_HYBRID) -> int:
    """Number of misses to fill over the link (section 2.5 of the review)."""
    if m <= 0:
        return 0
    if policy == POLICY_OFFLOAD:
        return m
    if policy == POLICY_HOST:
        return 0
    if B_H <= B_P:          # B_R = 0: the host has nothing left after the link
        return m
    q = math.floor(m * B_P / B_H + 0.5)
    return max(1, min(m, q))


def branch_times(m: int, q: int, S: float, B_P: float, B_H: float):
    """(T_fill, T_cpu) in seconds for bandwidths in bytes/s (section 2.5)."""
    t_fill = q * S / B_P
    B_R = max(B_H - B_P, 0.0)
    t_cpu = 0.0 if m - q == 0 else ((m - q) * S / B_R if B_R > 0 else math.inf)
    return t_fill, t_cpu


def link_bound_chunk_seconds(pool_bytes: float, B_P: float) -> float:
    """Prefill chunk time when expert compute hides behind the full-layer copy
    (section 2.2): every routed expert crosses the link once per chunk."""
    return pool_bytes / B_P


class SlotCache:
    """Global LRU over n_slots slots shared by all layers (logical id l*E+e)."""

    def __init__(self, L: int, E: int, n_slots: int):
        self.L, self.E, self.n_slots = L, E, n_slots
        self.slot_of = [-1] * (L * E)
        self.owner = [-1] * n_slots
        self.last_use = [0] * n_slots
        self.tick = 0

    # -- helpers ---------------------------------------------------------
    def resident(self, layer: int) -> dict:
        return {e: self.slot_of[layer * self.E + e] for e in range(self.E) if self.slot_of[layer * self.E + e] >= 0}

    def _eligible(self):
        return sorted((s for s in range(self.n_slots) if self.last_use[s] != self.tick),
                      key=lambda s: (self.last_use[s], s))

    def _install(self, layer, experts, victims):
        evicted = []
        for e, s in zip(experts, victims):
            if self.owner[s] >= 0:
                evicted.append(self.owner[s])
                self.slot_of[self.owner[s]] = -1
            self.owner[s] = layer * self.E + e
            self.slot_of[layer * self.E + e] = s
            self.last_use[s] = self.tick
        return evicted

    # -- one planning call per (step, layer) -----------------------------
    def plan(self, layer: int, ids, policy=POLICY_HYBRID, B_P=1.0, B_H=1.0) -> dict:
        self.tick += 1
        U = sorted(set(int(e) for e in list(ids)))
        hits, misses = [], []
        for e in U:
            s = self.slot_of[layer * self.E + e]
            if s >= 0:
                hits.append(e)
                self.last_use[s] = self.tick
            else:
                misses.append(e)
        m = len(misses)
        q = q_star(m, B_P, B_H, policy)
        elig = self._eligible()
        q = min(q, len(elig))
        F, C = misses[:q], misses[q:]
        victims = elig[:q]
        evicted = self._install(layer, F, victims)
        return dict(tick=self.tick, unique=U, hits=hits, misses=misses, m=m, q=q, F=F, C=C,
                    victims=victims, evicted=evicted)

    def admit(self, layer: int, experts) -> list:
        """Install the given experts (already-resident ones only refreshed)."""
        self.tick += 1
        need = []
        for e in sorted(set(int(v) for v in experts)):
            s = self.slot_of[layer * self.E + e]
            if s >= 0:
                self.last_use[s] = self.tick
            else:
                need.append(e)
        elig = self._eligible()
        if len(elig) < len(need):
            raise RuntimeError("not enough slots")
        victims = elig[:len(need)]
        self._install(layer, need, victims)
        return victims

    def resize(self, n_slots: int) -> list:
        """Rebuild with n_slots slots; returns the (old slot, new slot) moves."""
        used = [s for s in range(self.n_slots) if self.owner[s] >= 0]
        keep = sorted(used, key=lambda s: (-self.last_use[s], s))[:n_slots]
        keep.sort()
        owner = [-1] * n_slots
        last_use = [0] * n_slots
        self.slot_of = [-1] * (self.L * self.E)
        moves = []
        for new, old in enumerate(keep):
            owner[new] = self.owner[old]
            last_use[new] = self.last_use[old]
            self.slot_of[self.owner[old]] = new
            moves.append((old, new))
        self.owner, self.last_use, self.n_slots = owner, last_use, n_slots
        return moves

    def evict(self, layer: int, experts) -> None:
        for e in experts:
            g = layer * self.E + int(e)
            s = self.slot_of[g]
            if s >= 0:
                self.slot_of[g] = -1
                self.owner[s] = -1
                self.last_use[s] = 0
