"""A captured HIP graph of moe_layer_forward calls replays to the eager result,
bit for bit, on every replay, with eager work and synchronisations between
the replays (small-batch and tiled kernels, two layers per graph)."""
import numpy as np
import pytest
import torch

from gpu_util import Setup, compare, shape

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T", [1, 5, 64, 300])
def test_graph_replay_matches_eager(T):
    print(f"graph replay T={T}", flush=True)
    cfg = shape(1, L=2, E=32, k=4, H=1024, I=384)
    s = Setup(cfg, seed=31, max_tokens=512)
    try:
        for layer in range(cfg.L):
            s.admit_all(layer)
        xs, xds = zip(*[s.hidden(T, tag=100 + l) for l in range(cfg.L)])
        rows = [s.slot_row(l) for l in range(cfg.L)]
        eager = []
        for l in range(cfg.L):
            o = torch.empty(T, cfg.H, dtype=torch.bfloat16, device="cuda")
            s.rt.forward(l, xds[l], s.R_d[l], s.b_d[l], rows[l], o)
            eager.append(o)
        torch.cuda.synchronize()
        for l in range(cfg.L):
            compare(s, l, xs[l], eager[l])
        outs = [torch.zeros(T, cfg.H, dtype=torch.bfloat16, device="cuda") for _ in range(cfg.L)]
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        with torch.cuda.graph(g, stream=cap):
            for l in range(cfg.L):
                s.rt.forward(l, xds[l], s.R_d[l], s.b_d[l], rows[l], outs[l])
        other_x, other_xd = s.hidden(T, tag=999)
        scratch = torch.empty(T, cfg.H, dtype=torch.bfloat16, device="cuda")
        for rep in range(4):
            for o in outs:
                o.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for l in range(cfg.L):
                assert torch.equal(outs[l].view(torch.int16), eager[l].view(torch.int16)), (rep, l)
            # eager work between replays reuses the same workspace
            s.rt.forward(0, other_xd, s.R_d[0], s.b_d[0], rows[0], scratch)
            torch.cuda.synchronize()
        assert s.rt.check_device_error() == 0
        compare(s, 0, other_x, scratch)
    finally:
        s.close()
