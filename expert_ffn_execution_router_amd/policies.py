"""Replay of routing traces through expert placement policies (miss rates).

The policies compared by the ablation of the global LRU residency
(paper.oopus.info review of FreeToken, section 2.4 and the ablation list
that repeats it), each at the same number of expert slots:

* global LRU over every layer's experts: a hit refreshes recency, every miss
  is admitted and evicts the least recently needed expert.  Replayed through
  the library's device cache-control kernel under the OFFLOAD policy (q = m);
* a placement frozen at prefill: the slots hold the (layer, expert) pairs
  routed most often in a prefill chunk, fixed for the whole decode (reading:
  ties go to the lower layer, then the lower expert id);
* a routing-agnostic static split: whole layers in order from layer 0 until
  the slots run out, the last layer partly with its lowest expert ids
  (reading of an assignment made when the model is loaded).

A trace holds the routed expert ids of every (step, layer): int32
[steps, L, T, k].  A miss is a routed (layer, expert) pair of a step that is
not resident when the step needs it; rates are misses over the distinct
routed pairs of the counted steps.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B


def route_rows(rt, x, router_w, bias) -> np.ndarray:
    """Routed ids int32 [n, k] of hidden rows x [n, H] (bf16 bits as int16, on
    the device) through the library's router and top-k, in chunks of the
    runtime's max_tokens."""
    n = x.shape[0]
    step = rt.cfg.max_tokens
    ids = torch.empty(n, rt.cfg.k, dtype=torch.int32, device=x.device)
    w = torch.empty(n, rt.cfg.k, dtype=torch.float32, device=x.device)
    for a in range(0, n, step):
        b = min(n, a + step)
        rt.route(x[a:b], router_w, bias, ids[a:b], w[a:b])
    return ids.cpu().numpy()


def lru_replay(rt, trace: np.ndarray, warmup: int) -> tuple[int, int]:
    """(misses, distinct routed pairs) over steps >= warmup, replaying the
    trace through the device LRU of runtime `rt` (cold start, OFFLOAD: every
    miss admitted).  rt must have the trace's L, E, k; its expert size is
    irrelevant (planning copies nothing)."""
    S, L = trace.shape[:2]
    rt.reset_cache()
    rt.set_policy(B.MOE_POLICY_OFFLOAD)
    dev = torch.from_numpy(np.ascontiguousarray(trace, dtype=np.int32)).to(rt.device)
    misses = uniq = 0
    for s in range(S):
        for l in range(L):
            info, _, _ = rt.plan(l, dev[s, l])
            if s >= warmup:
                misses += info.m
                uniq += info.n_unique
    return misses, uniq


def prefill_hot_set(prefill_ids: np.ndarray, E: int, n_slots: int) -> np.ndarray:
    """Resident mask bool [L*E]: the n_slots (layer, expert) pairs with the most
    routed tokens in the prefill chunk prefill_ids int32 [L, Tp, k]."""
    L = prefill_ids.shape[0]
    counts = np.stack([np.bincount(prefill_ids[l].ravel(), minlength=E) for l in range(L)]).ravel()
    order = np.lexsort((np.arange(L * E), -counts))      # most routed first, then lower (layer, expert)
    mask = np.zeros(L * E, dtype=bool)
    mask[order[:min(n_slots, L * E)]] = True
    return mask


def static_split(L: int, E: int, n_slots: int) -> np.ndarray:
    """Resident mask bool [L*E]: layers 0, 1, ... whole, the next one partly."""
    mask = np.zeros(L * E, dtype=bool)
    mask[:min(n_slots, L * E)] = True
    return mask


def fixed_replay(resident: np.ndarray, trace: np.ndarray, warmup: int) -> tuple[int, int]:
    """(misses, distinct routed pairs) over steps >= warmup for a placement
    that never changes."""
    S, L = trace.shape[:2]
    E = resident.size // L
    misses = uniq = 0
    for s in range(warmup, S):
        for l in range(L):
            u = np.unique(trace[s, l])
            uniq += u.size
            misses += int((~resident[l * E + u]).sum())
    return misses, uniq
