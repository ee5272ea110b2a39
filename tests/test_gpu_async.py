"""The decode layer with device-resident cache control (no host read of the
plan, indexed fill kernel, host branch as a stream callback): bit-identical to
the synchronous decode layer on the same inputs and cache history, its plan
totals equal to the oracle's slot model, and a captured HIP graph of a whole
step replays to the same results with eager work between the replays."""
import numpy as np
import pytest
import torch

from oracle import cache as OC
from oracle import moe as M
from expert_ffn_execution_router_amd import binding as B
from gpu_util import exact_bound, MARGIN, TOL, Setup, bf16_to_np, compare, rel_err, shape

pytestmark = pytest.mark.gpu

BP, BH = 30.0, 70.0


def _pair(cfg, n_slots, policy, seed=5):
    a = Setup(cfg, seed=seed, n_slots=n_slots, max_tokens=64)
    b = Setup(cfg, seed=seed, n_slots=n_slots, max_tokens=64, pool=a.pool)
    for s in (a, b):
        s.rt.set_policy(policy, BP, BH)
    return a, b


def _bits(t):
    return t.view(torch.int16).cpu().numpy()


def _device_ids(s, layer, xd):
    T = xd.shape[0]
    ids = torch.empty(T, s.cfg.k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, s.cfg.k, dtype=torch.float32, device="cuda")
    s.rt.route(xd, s.R_d[layer], s.b_d[layer], ids, w)
    torch.cuda.synchronize()
    return ids.cpu().numpy()


def _check_oracle(s, layer, x, out, host_set):
    """The mirrored oracle with the plan's host set evaluated exactly (the
    host branch keeps fp32 and the weights' exact values)."""
    T = len(x)
    ref = M.moe_layer(x, s.R[layer], s.b[layer], s.cfg.k, s.weights(layer), fmt=s.cfg.fmt, mode="both",
                      host_set=host_set, act=s.act_of(T))
    rows = np.nonzero(ref["margin"] >= MARGIN)[0]
    assert len(rows) > 0
    got = bf16_to_np(out)
    assert rel_err(got, ref["out"], rows) <= TOL[s.cfg.fmt]
    e_q = rel_err(ref["out"], ref["out_exact"], rows)
    assert rel_err(got, ref["out_exact"], rows) <= exact_bound(s, T, e_q, TOL[s.cfg.fmt])


@pytest.mark.parametrize("fmt,n_slots,policy,T", [(0, 12, B.MOE_POLICY_HYBRID, 5), (0, 12, B.MOE_POLICY_OFFLOAD, 3),
                                                  (0, 20, B.MOE_POLICY_OFFLOAD, 1), (0, 12, B.MOE_POLICY_HOST, 4),
                                                  (1, 10, B.MOE_POLICY_HYBRID, 2), (2, 10, B.MOE_POLICY_OFFLOAD, 6),
                                                  (3, 10, B.MOE_POLICY_HYBRID, 3)])
def test_async_equals_sync_decode(fmt, n_slots, policy, T):
    print(f"async decode fmt={fmt} n_slots={n_slots} policy={policy} T={T}", flush=True)
    cfg = shape(1, L=3, E=16, k=4, H=256, I=128, fmt=fmt)
    a, b = _pair(cfg, n_slots, policy)
    try:
        copy = torch.cuda.Stream()
        hs = torch.cuda.Stream()
        model = OC.SlotCache(cfg.L, cfg.E, n_slots)
        infos = []
        for step in range(4):
            for layer in range(cfg.L):
                x, xd = a.hidden(T, tag=2000 + step * 11 + layer)
                ref = model.plan(layer, _device_ids(b, layer, xd).reshape(-1), policy, BP, BH)
                oa = torch.empty(T, cfg.H, dtype=torch.bfloat16, device="cuda")
                ob = torch.empty(T, cfg.H, dtype=torch.bfloat16, device="cuda")
                info = b.rt.decode_layer(layer, xd, b.R_d[layer], b.b_d[layer], ob, copy_stream=copy)
                infos.append(info)
                assert (info.m, info.q, info.n_host) == (ref["m"], ref["q"], len(ref["C"]))
                a.rt.decode_layer_async(layer, xd, a.R_d[layer], a.b_d[layer], oa, host_stream=hs)
                torch.cuda.synchronize()
                assert np.array_equal(_bits(oa), _bits(ob)), (step, layer)
                if step >= 2:
                    _check_oracle(a, layer, x, oa, ref["C"])
        tot = a.rt.plan_stats()
        assert a.rt.check_device_error() == 0
        assert tot["calls"] == len(infos)
        for f in ("n_unique", "n_hit", "m", "q", "n_host", "n_evict"):
            assert tot[f] == sum(getattr(i, f) for i in infos), f
        assert tot["m"] > 0
        assert list(a.rt.slot_table().cpu().numpy()) == list(b.rt.slot_table().cpu().numpy()) == model.slot_of
    finally:
        a.close()
        b.close()


@pytest.mark.parametrize("policy,n_slots", [(B.MOE_POLICY_HYBRID, 12), (B.MOE_POLICY_OFFLOAD, 20)])
def test_async_step_graph_replays(policy, n_slots):
    """One captured graph per step shape; each replay plans afresh (the LRU
    clock lives on the device), so replays with new inputs follow the same
    cache history as synchronous calls."""
    print(f"async graph policy={policy} n_slots={n_slots}", flush=True)
    cfg = shape(1, L=3, E=16, k=4, H=256, I=128)
    T = 2
    a, b = _pair(cfg, n_slots, policy, seed=8)
    try:
        copy = torch.cuda.Stream()
        hs = torch.cuda.Stream()
        cap = torch.cuda.Stream()
        xin = torch.zeros(cfg.L, T, cfg.H, dtype=torch.int16, device="cuda")
        outs = torch.zeros(cfg.L, T, cfg.H, dtype=torch.bfloat16, device="cuda")

        def step_inputs(tag):
            return [a.hidden(T, tag=tag * 10 + l) for l in range(cfg.L)]

        def ref_step(inputs):
            res = []
            for l, (x, xd) in enumerate(inputs):
                o = torch.empty(T, cfg.H, dtype=torch.bfloat16, device="cuda")
                b.rt.decode_layer(l, xd, b.R_d[l], b.b_d[l], o, copy_stream=copy)
                res.append(o)
            torch.cuda.synchronize()
            return res

        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for l in range(cfg.L):
                a.rt.decode_layer_async(l, xin[l], a.R_d[l], a.b_d[l], outs[l], stream=cap, host_stream=hs)
        torch.cuda.synchronize()
        assert a.rt.plan_stats(reset=True)["calls"] == 0      # capture plans nothing
        scratch = torch.empty(T, cfg.H, dtype=torch.bfloat16, device="cuda")
        for rep in range(4):
            inputs = step_inputs(100 + rep)
            for l, (_, xd) in enumerate(inputs):
                xin[l].copy_(xd)
            outs.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            ref = ref_step(inputs)
            for l in range(cfg.L):
                assert np.array_equal(_bits(outs[l]), _bits(ref[l])), (rep, l)
            # eager asynchronous work between replays, same context and cache
            x, xd = a.hidden(T, tag=900 + rep)
            a.rt.decode_layer_async(1, xd, a.R_d[1], a.b_d[1], scratch, host_stream=hs)
            o = torch.empty(T, cfg.H, dtype=torch.bfloat16, device="cuda")
            b.rt.decode_layer(1, xd, b.R_d[1], b.b_d[1], o, copy_stream=copy)
            torch.cuda.synchronize()
            assert np.array_equal(_bits(scratch), _bits(o)), rep
        compare(a, 1, x, scratch)
        tot = a.rt.plan_stats()
        assert tot["calls"] == 4 * (cfg.L + 1)
        assert tot["m"] > 0
        assert a.rt.check_device_error() == 0
        assert list(a.rt.slot_table().cpu().numpy()) == list(b.rt.slot_table().cpu().numpy())
    finally:
        a.close()
        b.close()
