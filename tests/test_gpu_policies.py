"""GPU side of the placement-policy replay: the LRU replay through the device
cache-control kernel equals the oracle's slot model miss for miss, and the
chunked routing of a trace equals the oracle's top-k."""
import numpy as np
import pytest
import torch

from oracle import moe as M
from expert_ffn_execution_router_amd import policies as P
from gpu_util import Setup, shape
from test_policies import _oracle_lru, _trace

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_slots,T", [(24, 1), (40, 1), (96, 3), (192, 2)])
def test_lru_replay_matches_slot_model(n_slots, T):
    print(f"lru replay n_slots={n_slots} T={T}", flush=True)
    L, E, k = 6, 32, 4
    cfg = shape(1, L=L, E=E, k=k, H=256, I=128)
    s = Setup(cfg, seed=3, n_slots=n_slots, max_tokens=64)
    try:
        tr = _trace(n_slots + T, 40, L, T, E, k)
        got = P.lru_replay(s.rt, tr, 8)
        assert got == _oracle_lru(tr, E, n_slots, 8)
        assert P.lru_replay(s.rt, tr, 8) == got          # reset_cache gives a cold start again
    finally:
        s.close()


def test_route_rows_chunks_match_oracle():
    print("route_rows chunked", flush=True)
    cfg = shape(2, L=2, H=512, I=128)
    s = Setup(cfg, seed=9, n_slots=0, max_tokens=64)
    try:
        x, xd = s.hidden(150, tag=4)                      # chunks of 64, 64, 22
        for l in range(cfg.L):
            got = P.route_rows(s.rt, xd, s.R_d[l], s.b_d[l])
            z = M.router_logits(x, s.R[l], s.b[l]).astype(np.float32).astype(np.float64)
            ref = M.select_topk(z, cfg.k)
            ok = M.topk_margin(z, cfg.k) > 1e-4
            assert ok.sum() > 140
            assert (np.sort(got[ok], 1) == np.sort(ref[ok], 1)).all()
    finally:
        s.close()
