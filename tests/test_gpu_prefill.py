"""GPU tests of the full-layer double-buffered prefill streamer: outputs match
the oracle, and are bit-identical with the double buffer on, off, with every
expert already resident, and on the on-demand fallback."""
import numpy as np
import pytest
import torch

from expert_ffn_execution_router_amd import binding as B
from gpu_util import Setup, compare, shape

pytestmark = pytest.mark.gpu


def _cfg(fmt=0):
    if fmt == 0:
        return shape(1, L=4, E=8, k=2, H=256, I=128)
    return shape(1, L=3, E=8, k=2, H=512, I=256, fmt=fmt)


def _prefill(cfg, n_slots, T, double_buffer=True, seed=2, act=None):
    s = Setup(cfg, seed=seed, n_slots=n_slots, max_tokens=T)
    if act:
        s.set_act(act)
    outs, xs, rcs = [], [], []
    comp, copy = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(comp):
        for layer in range(cfg.L):
            x, xd = s.hidden(T, tag=layer)
            out = torch.empty(T, cfg.H, dtype=torch.bfloat16, device="cuda")
            rcs.append(s.rt.prefill_layer(layer, xd, s.R_d[layer], s.b_d[layer], out, stream=comp,
                                          copy_stream=copy, double_buffer=double_buffer))
            outs.append(out)
            xs.append(x)
    torch.cuda.synchronize()
    return s, outs, xs, rcs


@pytest.mark.parametrize("fmt,act", [(0, None), (1, None), (2, None), (2, "mxfp6")])
def test_prefill_matches_oracle_and_is_buffer_invariant(fmt, act):
    print(f"prefill fmt={fmt} act={act}", flush=True)
    cfg = _cfg(fmt)
    T = 300
    s, outs, xs, rcs = _prefill(cfg, 2 * cfg.E, T, act=act)
    try:
        assert rcs == [0] * cfg.L
        assert s.rt.check_device_error() == 0
        for layer in range(cfg.L):
            compare(s, layer, xs[layer], outs[layer])
        ref = [o.view(torch.int16).cpu().numpy() for o in outs]
        # survivors: the last two layers stay resident for decode
        t = s.rt.slot_table().cpu().numpy().reshape(cfg.L, cfg.E)
        assert (t[cfg.L - 1] >= 0).all() and (t[cfg.L - 2] >= 0).all()
    finally:
        s.close()
    for n_slots, dbuf, want_rc in [(2 * cfg.E, False, 0), (cfg.L * cfg.E, True, 0), (cfg.E, True, 2),
                                   (2 * cfg.E - 1, True, 2)]:
        print(f"  variant n_slots={n_slots} double_buffer={dbuf}", flush=True)
        s, outs, xs, rcs = _prefill(cfg, n_slots, T, double_buffer=dbuf, act=act)
        try:
            assert rcs == [want_rc] * cfg.L
            for a, b in zip(ref, outs):
                assert np.array_equal(a, b.view(torch.int16).cpu().numpy())
        finally:
            s.close()
    # fewer than E slots: the layer in expert ranges of n_slots on the GPU
    # (the ranges' sums add in a different order: within tolerance, not bit
    # for bit); 3 slots leave a short last range
    for n_slots in (cfg.E // 2, 3):
        print(f"  variant in ranges n_slots={n_slots}", flush=True)
        s, outs, xs, rcs = _prefill(cfg, n_slots, T, act=act)
        try:
            assert rcs == [1] * cfg.L
            assert s.rt.check_device_error() == 0
            for layer in range(cfg.L):
                compare(s, layer, xs[layer], outs[layer])
        finally:
            s.close()


def test_prefill_then_decode_uses_survivors():
    cfg = _cfg()
    s, outs, xs, rcs = _prefill(cfg, 3 * cfg.E, 64)
    try:
        s.rt.set_policy(B.MOE_POLICY_OFFLOAD)
        x, xd = s.hidden(1, tag=77)
        out = torch.empty(1, cfg.H, dtype=torch.bfloat16, device="cuda")
        info = s.rt.decode_layer(cfg.L - 1, xd, s.R_d[cfg.L - 1], s.b_d[cfg.L - 1], out)
        torch.cuda.synchronize()
        assert info.m == 0 and info.n_hit == info.n_unique
        compare(s, cfg.L - 1, x, out)
    finally:
        s.close()
