"""GPU tests of the slot cache path: the device LRU kernel against the oracle's
slot model (bit-exact table), decode layers through the cache against the
oracle, and the invariants the pages fix: the output does not depend on the
cache size or on slot assignment, and a GPU + host split equals the all-GPU
result."""
import time

import numpy as np
import pytest
import torch

from oracle import cache as OC
from oracle import moe as M
from expert_ffn_execution_router_amd import binding as B
from gpu_util import Setup, bf16_to_np, compare, rel_err, shape

pytestmark = pytest.mark.gpu

CFG = dict(base=1, L=3, E=16, k=4, H=256, I=128)


def _cfg(**kw):
    d = dict(CFG)
    d.update(kw)
    base = d.pop("base")
    return shape(base, **d)


def _route(s, layer, xd):
    T = xd.shape[0]
    ids = torch.empty(T, s.cfg.k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, s.cfg.k, dtype=torch.float32, device="cuda")
    s.rt.route(xd, s.R_d[layer], s.b_d[layer], ids, w)
    torch.cuda.synchronize()
    return ids.cpu().numpy()


@pytest.mark.parametrize("n_slots,policy", [(12, B.MOE_POLICY_OFFLOAD), (12, B.MOE_POLICY_HYBRID),
                                            (20, B.MOE_POLICY_HOST), (7, B.MOE_POLICY_HYBRID),
                                            (48, B.MOE_POLICY_OFFLOAD)])
def test_plan_kernel_matches_slot_model(n_slots, policy):
    print(f"plan n_slots={n_slots} policy={policy}", flush=True)
    cfg = _cfg()
    s = Setup(cfg, seed=21, n_slots=n_slots, max_tokens=16)
    try:
        BP, BH = 30.0, 70.0
        s.rt.set_policy(policy, BP, BH)
        model = OC.SlotCache(cfg.L, cfg.E, n_slots)
        rng = np.random.default_rng(n_slots)
        for step in range(12):
            for layer in range(cfg.L):
                T = int(rng.integers(1, 6))
                x, xd = s.hidden(T, tag=step * 10 + layer)
                ids = _route(s, layer, xd)
                ids_d = torch.from_numpy(ids).cuda()
                mask = torch.zeros(8, dtype=torch.int32, device="cuda")
                info, fe, fs = s.rt.plan(layer, ids_d, mask)
                ref = model.plan(layer, ids.reshape(-1), policy, BP, BH)
                assert (info.m, info.q, info.n_hit, info.n_unique) == (ref["m"], ref["q"], len(ref["hits"]),
                                                                       len(ref["unique"]))
                assert fe == ref["F"] and fs == ref["victims"]
                table = s.rt.slot_table().cpu().numpy()
                assert list(table) == model.slot_of
                m = mask.cpu().numpy().view(np.uint32)
                got_c = [e for e in range(cfg.E) if (m[e >> 5] >> (e & 31)) & 1]
                assert got_c == ref["C"]
    finally:
        s.close()


@pytest.mark.parametrize("policy", [B.MOE_POLICY_OFFLOAD, B.MOE_POLICY_HYBRID])
def test_plan_kernel_many_slots(policy):
    """More slots than the kernel has threads (victims and stamp ties across
    1024-slot blocks) and up to ~128 misses per layer (q beyond one wave)."""
    print(f"plan many slots policy={policy}", flush=True)
    cfg = _cfg(L=24, E=128, k=8, H=256, I=128)
    n_slots = 2500
    s = Setup(cfg, seed=23, n_slots=n_slots, max_tokens=64)
    try:
        BP, BH = 30.0, 70.0
        s.rt.set_policy(policy, BP, BH)
        model = OC.SlotCache(cfg.L, cfg.E, n_slots)
        rng = np.random.default_rng(3)
        for step in range(4):
            for layer in range(cfg.L):
                T = int(rng.integers(8, 41))
                x, xd = s.hidden(T, tag=step * 100 + layer)
                ids = _route(s, layer, xd)
                ids_d = torch.from_numpy(ids).cuda()
                mask = torch.zeros(8, dtype=torch.int32, device="cuda")
                info, fe, fs = s.rt.plan(layer, ids_d, mask)
                ref = model.plan(layer, ids.reshape(-1), policy, BP, BH)
                assert (info.m, info.q, info.n_hit, info.n_unique) == (ref["m"], ref["q"], len(ref["hits"]),
                                                                       len(ref["unique"]))
                assert fe == ref["F"] and fs == ref["victims"]
                m = mask.cpu().numpy().view(np.uint32)
                got_c = [e for e in range(cfg.E) if (m[e >> 5] >> (e & 31)) & 1]
                assert got_c == ref["C"]
        assert list(s.rt.slot_table().cpu().numpy()) == model.slot_of
    finally:
        s.close()


def _decode_run(cfg, n_slots, policy, steps, T, seed=5, BP=30.0, BH=70.0, reverse_admit=False):
    s = Setup(cfg, seed=seed, n_slots=n_slots, max_tokens=64)
    outs = []
    infos = []
    try:
        s.rt.set_policy(policy, BP, BH)
        copy = torch.cuda.Stream()
        if reverse_admit:
            # a different slot assignment: layers in reverse, odd experts before even ones
            for layer in reversed(range(cfg.L)):
                s.rt.admit(layer, list(range(1, cfg.E, 2)))
                s.rt.admit(layer, list(range(0, cfg.E, 2)))
            torch.cuda.synchronize()
        for step in range(steps):
            for layer in range(cfg.L):
                x, xd = s.hidden(T, tag=1000 + step * 7 + layer)
                out = torch.empty(T, cfg.H, dtype=torch.bfloat16, device="cuda")
                info = s.rt.decode_layer(layer, xd, s.R_d[layer], s.b_d[layer], out, copy_stream=copy)
                infos.append(info.as_dict())
                outs.append((layer, x, out))
        torch.cuda.synchronize()
        assert s.rt.check_device_error() == 0
        return s, outs, infos
    except Exception:
        s.close()
        raise


@pytest.mark.parametrize("policy", [B.MOE_POLICY_OFFLOAD, B.MOE_POLICY_HOST, B.MOE_POLICY_HYBRID])
def test_decode_through_cache_matches_oracle(policy):
    print(f"decode policy={policy}", flush=True)
    cfg = _cfg()
    s, outs, infos = _decode_run(cfg, 12, policy, steps=4, T=5)
    try:
        for layer, x, out in outs:
            compare(s, layer, x, out)
        m = sum(i["m"] for i in infos)
        assert m > 0
        if policy == B.MOE_POLICY_HOST:
            assert sum(i["q"] for i in infos) == 0 and sum(i["n_host"] for i in infos) == m
        if policy == B.MOE_POLICY_OFFLOAD:
            # every miss that fits is filled; only the capacity overflow goes to the host
            assert all(i["q"] == min(i["m"], 12 - i["n_hit"]) for i in infos)
        if policy == B.MOE_POLICY_HYBRID:
            assert all(i["q"] >= 1 for i in infos if i["m"] > 0)
            assert sum(i["n_host"] for i in infos) > 0
    finally:
        s.close()


def test_output_independent_of_cache_size_and_slot_assignment():
    """Bit-identical outputs for full / fraction / 2E / k slots and for a
    different initial slot assignment (OFFLOAD: every expert runs on the GPU)."""
    cfg = _cfg()
    ref_outs = None
    for n_slots, T, rev in [(cfg.L * cfg.E, 1, False), (12, 1, False), (2 * cfg.E, 1, False), (cfg.k, 1, False),
                            (cfg.L * cfg.E, 1, True)]:
        print(f"invariance n_slots={n_slots} reverse={rev}", flush=True)
        s, outs, _ = _decode_run(cfg, n_slots, B.MOE_POLICY_OFFLOAD, steps=3, T=T, reverse_admit=rev)
        try:
            cur = [o.view(torch.int16).cpu().numpy() for _, _, o in outs]
            if ref_outs is None:
                ref_outs = cur
                for layer, x, out in outs:
                    compare(s, layer, x, out)
            else:
                for a, b in zip(ref_outs, cur):
                    assert np.array_equal(a, b)
        finally:
            s.close()


def test_split_equals_all_gpu():
    cfg = _cfg()
    outs_by = {}
    for policy in (B.MOE_POLICY_OFFLOAD, B.MOE_POLICY_HYBRID, B.MOE_POLICY_HOST):
        s, outs, _ = _decode_run(cfg, 12, policy, steps=3, T=6)
        try:
            outs_by[policy] = [bf16_to_np(o) for _, _, o in outs]
        finally:
            s.close()
    for policy in (B.MOE_POLICY_HYBRID, B.MOE_POLICY_HOST):
        for a, b in zip(outs_by[B.MOE_POLICY_OFFLOAD], outs_by[policy]):
            assert rel_err(b, a) <= 1e-2


def test_identical_experts_equal_single_ffn():
    cfg = _cfg(L=1)
    from expert_ffn_execution_router_amd.runtime import HostPool
    import synth
    S = cfg.expert_bytes
    pool = HostPool(cfg.L * cfg.E * S)
    arr = pool.array().reshape(cfg.E, S)
    arr[:] = synth.expert_blob(cfg, 9, 0, 0)[None, :]
    s = Setup(cfg, seed=9, n_slots=cfg.E, pool=pool)
    try:
        s.admit_all(0)
        T = 16
        x, xd = s.hidden(T)
        out = torch.empty(T, cfg.H, dtype=torch.bfloat16, device="cuda")
        s.rt.forward(0, xd, s.R_d[0], s.b_d[0], s.slot_row(0), out)
        torch.cuda.synchronize()
        from oracle.formats import bf16_to_f64
        single = M.expert_ffn(bf16_to_f64(x), *s.weights(0)(0))
        assert rel_err(bf16_to_np(out), single) <= 1e-2
    finally:
        s.close()
        pool.free()


def test_admit_evict_api():
    cfg = _cfg(L=2)
    s = Setup(cfg, seed=4, n_slots=10)
    try:
        s.rt.admit(1, [3, 5, 7])
        torch.cuda.synchronize()
        t = s.rt.slot_table().cpu().numpy()
        assert list(t[cfg.E + np.array([3, 5, 7])]) == [0, 1, 2]
        s.rt.evict(1, [5])
        t = s.rt.slot_table().cpu().numpy()
        assert t[cfg.E + 5] == -1 and t[cfg.E + 3] == 0
        # the filled slot holds the host bytes of (1, 7)
        torch.cuda.synchronize()
        got = s.rt.slots[2 * cfg.expert_bytes:3 * cfg.expert_bytes].cpu().numpy()
        assert np.array_equal(got, s.pool_np[cfg.E + 7])
        with pytest.raises(B.MoeError):
            s.rt.admit(0, list(range(cfg.E)))      # more than the 10 slots
    finally:
        s.close()


def test_calibrate_bandwidths():
    """Both rates positive; the copy targets are left empty and the table
    stays consistent."""
    print("calibrate", flush=True)
    cfg = _cfg(L=2)
    s = Setup(cfg, seed=6, n_slots=10)
    try:
        bp, bh = s.rt.calibrate()
        assert bp > 0.1 and bh > bp
        tab = s.rt.slot_table().cpu().numpy()
        assert (tab == -1).all()
        s.rt.admit(0, list(range(8)))
        torch.cuda.synchronize()
        assert (s.rt.slot_table().cpu().numpy()[:8] >= 0).all()
        assert s.rt.check_device_error() == 0
    finally:
        s.close()


def test_calibrate_reproducible_on_deployed_shape():
    """The calibration on the decode shape's experts (9.4 MB each) is
    reproducible: two calibrations in one process agree within 15% on B_P
    and within 25% on B_H, and the fill counts q* = round(m B_P / B_H) they
    give for m = 1 .. 2k misses differ by at most one; B_P lies within the
    copy engine's own range (a 256 MB pinned -> device copy timed here);
    every median lies inside its min/max and B_H = B_P + the residual host
    rate.  The host branch streams host DRAM, whose rate on a shared host
    drifts between calibrations a second apart (medians of 40 calls measured
    at 215 and 184 GB/s in one process), so B_H gets the wider bound; a
    wrong byte or expert count would put it off by a factor."""
    print("calibrate deployed shape", flush=True)
    cfg = shape(2, L=4)
    s = Setup(cfg, seed=1, n_slots=16, max_tokens=64, host_threads=8)
    try:
        a = s.rt.calibrate_ex(1)
        b = s.rt.calibrate_ex(1)
        print("calibration", a, b, flush=True)
        for m in (a, b):
            assert m["n_copy"] == 5 and m["n_host_alone"] == 40
            assert m["B_P_min"] <= m["B_P"] <= m["B_P_max"]
            assert m["host_alone_min"] <= m["host_alone"] <= m["host_alone_max"]
            assert m["B_H"] == pytest.approx(m["B_P"] + m["B_R"])
            # t(n) = t0 + n S / B_R passes through the medians of the calls on
            # 1 and k experts (the series the split uses)
            conc = m["n_host_conc"] >= 3
            r1, rk = (m["host_conc_1"], m["host_conc"]) if conc else (m["host_alone_1"], m["host_alone"])
            S = s.rt.S
            t1, tk = S / (r1 * 1e3), cfg.k * S / (rk * 1e3)          # us
            if m["host_t0_us"] > 0:
                assert m["host_t0_us"] + S / (m["B_R"] * 1e3) == pytest.approx(t1, rel=1e-9)
                assert m["host_t0_us"] + cfg.k * S / (m["B_R"] * 1e3) == pytest.approx(tk, rel=1e-9)
            else:
                assert m["B_R"] == pytest.approx(rk)
            assert m["B_R"] >= rk * (1 - 1e-9)         # further experts stream at least as fast as whole calls
        # the calibration's outputs (what q* uses) agree; the standalone host
        # rate is a reported diagnostic
        assert abs(a["B_P"] - b["B_P"]) <= 0.15 * max(a["B_P"], b["B_P"])
        assert abs(a["B_H"] - b["B_H"]) <= 0.25 * max(a["B_H"], b["B_H"])
        for m in range(1, 2 * cfg.k + 1):
            qa, qb = (OC.q_star(m, x["B_P"], x["B_H"]) for x in (a, b))
            assert abs(qa - qb) <= 1, (m, qa, qb)
        src = torch.empty(256 << 20, dtype=torch.uint8, pin_memory=True)
        dst = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        rates = []
        for _ in range(4):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            dst.copy_(src, non_blocking=True)
            torch.cuda.synchronize()
            rates.append(src.numel() / (time.perf_counter() - t0) / 1e9)
        ce = sorted(rates)[1:]
        print(f"copy engine {ce} GB/s", flush=True)
        assert 0.7 * min(ce) <= a["B_P"] <= 1.3 * max(ce)
        assert (s.rt.slot_table().cpu().numpy() == -1).all()
    finally:
        s.close()
