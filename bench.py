"""Benchmark of the routed MoE-layer forward on one MI355X.

Default run (python bench.py): the decode-shaped workload (48 layers, E=128
experts, top-8, H=2048, I=768, bf16, T=64 tokens per step, Zipf router bias,
0.7 reuse of the previous step's rows) with every expert resident in HBM,
timed over --steps steps of 48 layers after --warmup steps.  One JSON line on
stdout; progress on stderr.

  value    MoE-layer tokens/s = tokens x layers processed / wall time
  roofline the grouped gate/up GEMM (the dominant kernel) against HBM
  cpu_baseline the float64 oracle on a bounded sample of the same workload

Extra objects in the same line: per-stage GPU times, the same decode steps
through the 40% slot cache with the q* miss split (PCIe and host included,
never the value), and one 8192-token prefill chunk streamed through the
full-layer double buffer (with the ablation without it).

--phases selects a subset (decode, e2e, prefill, cpu) for profiling runs, or
adds the optional ones: formats (fp8 / MXFP4 / NVFP4 shapes, a subset with
--format-shapes), policies (miss rates
of expert placements replayed over synthetic routing), elastic (cache
rebuilds between decode steps), fallback (prefill with fewer than two
layers of slots, and the prefill-to-decode hand-off), mxfp4_serving (the
MXFP4 shape's pool: a prefill chunk, then 512 decode steps through a 25%
cache) and fp8_serving (the fp8 shape's pool: a 4096-token prefill chunk,
then decode at T=1 and 32 through a 30% cache);
--copy-probe only runs a 1 GiB device copy (calibrates the byte counters).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np


def profile_end(rt):
    """Stage timings of a profiled region; every launch must have been timed
    (a region that outgrew its event capacity would undercount)."""
    prof = rt.profile_end()
    if prof["dropped"]:
        raise RuntimeError("profiling dropped launches: raise the event capacity of profile_begin")
    return prof


def log(*a):
    print(*a, file=sys.stderr, flush=True)


METRIC = "MoE-layer tokens/s (decode T≤64, prefill 8k); % HBM BW / % MFMA peak"
HBM_PEAK = 8.0e12
BF16_PEAK = 2.5e15
FP8_PEAK = 5.0e15
FP4_PEAK = 10.1e15
ROOT = os.path.dirname(os.path.abspath(__file__))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--T", type=int, default=64)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--layers", type=int, default=48)
    ap.add_argument("--phases", default="decode,e2e,prefill,cpu")
    ap.add_argument("--no-e2e", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--small-T", type=lambda v: [int(t) for t in v.split(",") if t], default=[1, 8, 32],
                    help="extra resident decode batch sizes timed on the same runtime (comma list, empty: none)")
    ap.add_argument("--e2e-T", type=int, default=1, help="tokens per step through the slot cache")
    ap.add_argument("--e2e-Ts", type=lambda v: [int(t) for t in v.split(",") if t], default=[8, 32, 64],
                    help="further batch sizes through the slot cache, short runs (comma list, empty: none)")
    ap.add_argument("--e2e-T-steps", type=int, default=8, help="timed steps of each --e2e-Ts run")
    ap.add_argument("--e2e-warmup", type=int, default=16)
    ap.add_argument("--high-hit-frac", type=float, default=0.9,
                    help="cache fraction of the high-hit sync-vs-graph decode comparison (0: skip)")
    ap.add_argument("--e2e-steps", type=int, default=32)
    ap.add_argument("--prefill-T", type=int, default=8192)
    ap.add_argument("--prefill-Ts", type=lambda v: [int(t) for t in v.split(",") if t], default=[4096, 16384],
                    help="further prefill chunk sizes timed with and without the second buffer (comma list)")
    ap.add_argument("--prefill-runs", type=int, default=2, help="double-buffered chunks timed (best is kept)")
    ap.add_argument("--cpu-layers", type=int, default=20, help="decode layers the oracle times (~0.5 s each)")
    ap.add_argument("--host-threads", type=int, default=13,
                    help="host FFN pool threads: the 16 host cores of one GPU's share less three, for the calling "
                         "thread (it launches, copies and synchronises while the pool runs) and the HIP runtime's "
                         "(the pool's workers poll for their next job between jobs)")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of one graph per step")
    ap.add_argument("--format-shapes", default="fp8,mxfp4,nvfp4", help="shapes of the formats phase")
    ap.add_argument("--format-layers", type=int, default=4,
                    help="layers of the fp8 and MXFP4 pools in the formats phase")
    ap.add_argument("--policy-steps", type=int, default=256, help="decode steps counted by the policies phase")
    ap.add_argument("--serving-steps", type=int, default=512, help="decode steps of the mxfp4 serving phase")
    ap.add_argument("--serving-layers", type=int, default=11, help="layers of the mxfp4 serving phase's pool")
    ap.add_argument("--fp8-serving-layers", type=int, default=6, help="layers of the fp8 serving phase's pool")
    ap.add_argument("--fp8-serving-steps", type=int, default=256, help="T=1 decode steps of the fp8 serving phase "
                    "(a quarter as many at T=32)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only copy 1 GiB device->device 3 times (calibrates HBM byte counters)")
    a = ap.parse_args()
    ph = set(p for p in a.phases.split(",") if p)
    for flag, name in ((a.no_e2e, "e2e"), (a.no_prefill, "prefill"), (a.no_cpu, "cpu")):
        if flag:
            ph.discard(name)
    a.phase_set = ph
    return a


def counted_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None when the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "decode_T64_bf16_gemm_hbm_counters.md")
    src = os.path.join(ROOT, "expert_ffn_execution_router_amd", "csrc", "gemm_dec.hip")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and line[0] not in "|#`":
            k, v = line.strip().split("=", 1)
            vals[k] = v
    cur = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    if vals.get("source_sha256_16[gemm_dec.hip]") != cur:
        return None
    v = vals.get(f"traffic_bytes[{kernel}]")
    return None if v is None else float(v)


def copy_probe():
    """A plain copy kernel of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = 1 << 30
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        t0 = time.perf_counter()
        b.copy_(a)
        torch.cuda.synchronize()
        log(f"copy {n} bytes: {2 * n / (time.perf_counter() - t0) / 1e9:.0f} GB/s (read+write)")


class Workload:
    """Seeded inputs of the decode/prefill shapes, resident on the device."""

    def __init__(self, args):
        import torch
        import synth
        from expert_ffn_execution_router_amd.runtime import HostPool
        self.args = args
        self.cfg = synth.CONFIGS[2].with_layers(args.layers)
        c = self.cfg
        self.dev = torch.device("cuda:0")
        t0 = time.time()
        self.pool = HostPool(c.L * c.E * c.expert_bytes)
        log(f"pinned host pool {c.L * c.E * c.expert_bytes / 1e9:.1f} GB allocated in {time.time() - t0:.1f}s")
        t0 = time.time()
        synth.fill_pool(self.pool.ptr, c, args.seed)
        log(f"host pool filled in {time.time() - t0:.1f}s")
        self.R = [torch.from_numpy(synth.router_weights(c, args.seed, l)).to(self.dev) for l in range(c.L)]
        self.bias = [torch.from_numpy(synth.router_bias(c, args.seed, l)).to(self.dev) for l in range(c.L)]
        W, K, T = args.warmup, args.steps, args.T
        keys = synth.decode_row_keys(c, args.seed, W + K, T)
        self.hid_np = synth.hidden_rows(c, keys.reshape(-1)).reshape(W + K, c.L, T, c.H)
        self.hidden = torch.from_numpy(self.hid_np.view(np.int16)).to(self.dev)   # in HBM before timing
        self.outs = torch.empty(c.L, T, c.H, dtype=torch.bfloat16, device=self.dev)

    def runtime(self, n_slots, max_tokens):
        from expert_ffn_execution_router_amd.runtime import MoeRuntime
        c = self.cfg
        return MoeRuntime(c.L, c.E, c.k, c.H, c.I, c.fmt, n_slots, max_tokens, self.pool,
                          host_threads=self.args.host_threads)


def phase_decode(w: Workload):
    """The value: decode steps with every expert resident in HBM."""
    import torch
    args, c = w.args, w.cfg
    L, E, k, H, I, T, S = c.L, c.E, c.k, c.H, c.I, args.T, c.expert_bytes
    K, W = args.steps, args.warmup
    rt = w.runtime(L * E, max(T, 64))
    t0 = time.time()
    for l in range(L):
        rt.admit(l, list(range(E)))
    torch.cuda.synchronize()
    log(f"resident pool: {L * E} experts copied to HBM in {time.time() - t0:.1f}s")
    table = rt.slot_table()
    rows = [table[l * E:(l + 1) * E] for l in range(L)]
    # routing of every timed (step, layer), for the algorithmic byte counts
    ids = torch.empty(T, k, dtype=torch.int32, device=w.dev)
    wts = torch.empty(T, k, dtype=torch.float32, device=w.dev)
    n_active = np.zeros((K, L), dtype=np.int64)
    for s in range(K):
        for l in range(L):
            rt.route(w.hidden[W + s, l], w.R[l], w.bias[l], ids, wts)
            n_active[s, l] = len(torch.unique(ids).cpu())
    torch.cuda.synchronize()

    def step(s):
        for l in range(L):
            rt.forward(l, w.hidden[s, l], w.R[l], w.bias[l], rows[l], w.outs[l])

    for s in range(W):
        step(s)
    torch.cuda.synchronize()
    # per-stage breakdown: one eager pass over the timed steps with every stage timed (not the value)
    rt.profile_begin(K * L * 8 + 16)
    for s in range(K):
        step(W + s)
    prof_all = profile_end(rt)
    # eager timed pass: GEMM 1 bracketed by HIP events on its stream (the
    # roofline's kernel duration); events inside a captured graph cannot be timed
    rt.profile_begin(K * L + 16, stages=["gemm1"])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        step(W + s)
    torch.cuda.synchronize()
    elapsed_eager = time.perf_counter() - t0
    prof = profile_end(rt)
    # graph timed pass (the value): one HIP graph per step (48 layers of
    # launches), as the pages replay a captured decode step
    use_graph = not args.eager
    graphs = []
    if use_graph:
        try:
            cap = torch.cuda.Stream()
            for s in range(K):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    step(W + s)
                graphs.append(g)
        except Exception as ex:       # capture unavailable: the eager pass is the value
            log(f"graph capture failed ({ex}); the value is the eager pass")
            use_graph = False
    torch.cuda.synchronize()
    elapsed = elapsed_eager
    if use_graph:
        graphs[0].replay()            # first replay uploads the graph
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(K):
            graphs[s].replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    assert rt.check_device_error() == 0
    value = K * L * T / elapsed
    log(f"decode resident: eager {elapsed_eager / K * 1e3:.3f} ms/step, "
        f"{'graph' if use_graph else 'eager'} {elapsed / K * 1e3:.3f} ms/step, {value:.0f} MoE-layer tokens/s")
    # algorithmic bytes (each active expert's weights read once; routed rows and outputs once)
    tk = T * k
    g1_bytes = (n_active * 2 * I * H * 2 + tk * H * 2 + tk * I * 2).sum()
    g2_bytes = (n_active * H * I * 2 + tk * I * 2 + tk * H * 2).sum()
    layer_bytes = (n_active * S + E * H * 4 + 2 * T * H * 2).sum()
    n_calls = K * L
    stage_ms = {n: v["ms"] / v["launches"] for n, v in prof_all.items() if isinstance(v, dict) and v["launches"]}
    g1_ms = prof["gemm1"]["ms"] / max(prof["gemm1"]["launches"], 1)   # inside the timed region
    g2_ms = stage_ms["gemm2"]
    gpu_layer_ms = sum(stage_ms.values())
    g1_achieved = g1_bytes / n_calls / (g1_ms * 1e-3)
    roofline = {
        "bound": "hbm", "kernel": "gemm_dec (bf16 gate/up + SwiGLU, small-batch grouped GEMM)",
        "achieved": g1_achieved / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
        "frac": g1_achieved / HBM_PEAK,
        "traffic": counted_traffic("void gemm_dec<0, true, 2>") if T > 8 else None,
        "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated)",
        "bytes_per_launch": float(g1_bytes / n_calls), "avg_launch_us": g1_ms * 1e3,
    }
    detail = {
        "launch": "hip graph per step" if use_graph else "eager",
        "eager_ms_per_step": elapsed_eager / K * 1e3,
        "gemm1_launches_timed": prof["gemm1"]["launches"],
        "ms_per_step": elapsed / K * 1e3, "layer_wall_us": elapsed / n_calls * 1e6,
        "stage_us": {n: v * 1e3 for n, v in stage_ms.items()},
        "gpu_layer_us": gpu_layer_ms * 1e3,
        "layer_hbm_frac_of_gpu_time": float(layer_bytes / n_calls / (gpu_layer_ms * 1e-3) / HBM_PEAK),
        "layer_hbm_frac_of_wall": float(layer_bytes / elapsed / HBM_PEAK),
        "gemm2_GBps": float(g2_bytes / n_calls / (g2_ms * 1e-3) / 1e9),
        "mean_active_experts": float(n_active.mean()),
        "layer_bytes_MB": float(layer_bytes / n_calls / 1e6),
    }
    log(json.dumps(roofline))
    log(json.dumps(detail))
    if args.small_T:
        detail["small_T"] = {str(t): decode_resident_at(w, rt, rows, t) for t in args.small_T}
    rt.close()
    del rt
    torch.cuda.empty_cache()
    return value, elapsed, roofline, detail


def decode_resident_at(w: Workload, rt, rows, T):
    """Resident decode at a smaller batch on the same runtime: seeded rows of
    the locality model, one HIP graph per 48-layer step (the value's launch
    mode), then an eager pass with every launch timed for the stage split."""
    import torch
    import synth
    args, c = w.args, w.cfg
    L, E, k, H, I, S = c.L, c.E, c.k, c.H, c.I, c.expert_bytes
    K, W = args.steps, args.warmup
    keys = synth.decode_row_keys(c, args.seed + 100 + T, W + K, T)
    hid = torch.from_numpy(synth.hidden_rows(c, keys.reshape(-1)).reshape(W + K, L, T, H).view(np.int16)).to(w.dev)
    outs = torch.empty(L, T, H, dtype=torch.bfloat16, device=w.dev)
    ids = torch.empty(T, k, dtype=torch.int32, device=w.dev)
    wts = torch.empty(T, k, dtype=torch.float32, device=w.dev)
    n_active = np.zeros((K, L), dtype=np.int64)
    for s in range(K):
        for l in range(L):
            rt.route(hid[W + s, l], w.R[l], w.bias[l], ids, wts)
            n_active[s, l] = len(torch.unique(ids).cpu())

    def step(s):
        for l in range(L):
            rt.forward(l, hid[s, l], w.R[l], w.bias[l], rows[l], outs[l])

    for s in range(W):
        step(s)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    graphs = []
    for s in range(K):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            step(W + s)
        graphs.append(g)
    graphs[0].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        graphs[s].replay()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    rt.profile_begin(K * L * 10 + 16)
    for s in range(K):
        step(W + s)
    prof = profile_end(rt)
    assert rt.check_device_error() == 0
    stage_us = {n: v["ms"] / v["launches"] * 1e3 for n, v in prof.items() if isinstance(v, dict) and v["launches"]}
    launches = {n: v["launches"] / (K * L) for n, v in prof.items() if isinstance(v, dict) and v["launches"]}
    gpu_layer_us = sum(stage_us[n] * launches[n] for n in stage_us)
    layer_bytes = float((n_active * S + E * H * 4 + 2 * T * H * 2).sum() / (K * L))
    res = {
        "T": T, "launch": "hip graph per step", "ms_per_step": el / K * 1e3,
        "moe_layer_tokens_per_s": K * L * T / el, "layer_wall_us": el / (K * L) * 1e6,
        "layer_bytes_MB": layer_bytes / 1e6, "mean_active_experts": float(n_active.mean()),
        "layer_hbm_frac_of_wall": layer_bytes / (el / (K * L)) / HBM_PEAK,
        "gpu_layer_us": gpu_layer_us, "layer_hbm_frac_of_gpu_time": layer_bytes / (gpu_layer_us * 1e-6) / HBM_PEAK,
        "launches_per_layer": launches, "stage_us": stage_us,
    }
    log(f"decode resident T={T}: {json.dumps(res)}")
    return res


def phase_e2e(w: Workload):
    """Decode steps through the 40% slot cache (LRU, HYBRID miss split with the
    bandwidths measured at startup), cold start: PCIe and host included."""
    import torch
    import synth
    from expert_ffn_execution_router_amd import binding as B
    args, c = w.args, w.cfg
    L, T = c.L, args.e2e_T
    W, K = args.e2e_warmup, args.e2e_steps
    keys = synth.decode_row_keys(c, args.seed + 1, W + K, T)
    hid = torch.from_numpy(synth.hidden_rows(c, keys.reshape(-1)).reshape(W + K, L, T, c.H).view(np.int16)).to(w.dev)
    outs = torch.empty(L, T, c.H, dtype=torch.bfloat16, device=w.dev)
    rc = w.runtime(c.n_slots, max(T, 64))
    cal = rc.calibrate_ex(T)
    bp, bh = cal["B_P"], cal["B_H"]
    log(f"calibration: {json.dumps(cal)}")
    rc.set_policy(B.MOE_POLICY_HYBRID, bp, bh)
    copy = torch.cuda.Stream()
    infos = []

    def e2e_step(s, record):
        for l in range(L):
            info = rc.decode_layer(l, hid[s, l], w.R[l], w.bias[l], outs[l], copy_stream=copy)
            if record:
                infos.append(info.as_dict())

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(W):
        e2e_step(s, False)
    torch.cuda.synchronize()
    warm_el = time.perf_counter() - t0
    rc.plan_stats(reset=True)
    t0 = time.perf_counter()
    for s in range(K):
        e2e_step(W + s, True)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    tot = rc.plan_stats(reset=True)           # host-branch time of the timed steps, from the pool
    assert rc.check_device_error() == 0
    uq = sum(i["n_unique"] for i in infos)
    # per-stage GPU times over the timed steps' rows again (after the timed
    # region, cache state carried on; not part of the step time)
    n_rec = len(infos)
    rc.profile_begin(K * L * 12 + 16)
    for s in range(K):
        e2e_step(W + s, False)
    prof = profile_end(rc)
    torch.cuda.synchronize()
    stage_us = {n: v["ms"] / v["launches"] * 1e3 for n, v in prof.items() if isinstance(v, dict) and v["launches"]}
    del infos[n_rec:]
    res = {
        "note": "PCIe and host included; not the value",
        "T": T, "n_slots": c.n_slots, "policy": "hybrid", "B_P_GBps": bp, "B_H_GBps": bh,
        "B_R_GBps": bh - bp, "calibration": cal,
        "q_star_over_m": bp / bh, "warmup_steps": W, "warmup_ms_per_step": warm_el / max(W, 1) * 1e3,
        "steps": K, "moe_layer_tokens_per_s": K * L * T / el, "ms_per_step": el / K * 1e3,
        "hit_rate": sum(i["n_hit"] for i in infos) / max(uq, 1),
        "misses_per_layer": sum(i["m"] for i in infos) / len(infos),
        "fills_per_layer": sum(i["q"] for i in infos) / len(infos),
        "host_per_layer": sum(i["n_host"] for i in infos) / len(infos),
        "t_fill_pred_us_per_layer": sum(i["t_fill_pred_us"] for i in infos) / len(infos),
        "t_host_pred_us_per_layer": sum(i["t_host_pred_us"] for i in infos) / len(infos),
        # the host branches as they ran (pool time, timed steps), against the prediction above
        "host_branch_us_per_layer": tot["host_ms"] * 1e3 / len(infos),
        "host_branch_GBps": tot["n_host"] * c.expert_bytes / max(tot["host_ms"] * 1e-3, 1e-12) / 1e9,
        "stage_us_per_launch": stage_us,
    }
    res["host_pred_over_measured"] = res["t_host_pred_us_per_layer"] / max(res["host_branch_us_per_layer"], 1e-9)
    res["device_cache_control"] = e2e_async(w, rc, hid, outs)
    log(json.dumps(res))
    rc.close()
    del rc
    torch.cuda.empty_cache()
    if args.e2e_Ts:
        res["by_T"] = {str(t): e2e_at(w, t, bp, bh) for t in args.e2e_Ts}
    if args.high_hit_frac > 0:
        res["high_hit"] = e2e_high_hit(w, bp, bh, args.high_hit_frac)
    return res


def e2e_high_hit(w: Workload, bp, bh, frac):
    """The synchronous decode layer (a host read of each layer's plan) against
    the device-resident one (one captured graph per step, no host read) where
    misses are rare: T=1 through a cache of `frac` of the pool, the same rows
    and the same cold start for both, 64 warm-up and 32 timed steps."""
    import torch
    import synth
    from expert_ffn_execution_router_amd import binding as B
    args, c = w.args, w.cfg
    L, T, W, K = c.L, 1, 64, 32
    n_slots = int(frac * L * c.E)
    keys = synth.decode_row_keys(c, args.seed + 3, W + K, T)
    hid = torch.from_numpy(synth.hidden_rows(c, keys.reshape(-1)).reshape(W + K, L, T, c.H).view(np.int16)).to(w.dev)
    outs = torch.empty(L, T, c.H, dtype=torch.bfloat16, device=w.dev)
    rc = w.runtime(n_slots, 64)
    rc.set_policy(B.MOE_POLICY_HYBRID, bp, bh)

    def totals(t):
        n = max(t["calls"], 1)
        return {"hit_rate": t["n_hit"] / max(t["n_unique"], 1), "misses_per_layer": t["m"] / n,
                "fills_per_layer": t["q"] / n, "host_per_layer": t["n_host"] / n}
    copy = torch.cuda.Stream()
    res = {"T": T, "n_slots": n_slots, "cache_frac": frac, "warmup_steps": W, "steps": K}
    for s in range(W):
        for l in range(L):
            rc.decode_layer(l, hid[s, l], w.R[l], w.bias[l], outs[l], copy_stream=copy)
    torch.cuda.synchronize()
    rc.plan_stats(reset=True)
    t0 = time.perf_counter()
    for s in range(K):
        for l in range(L):
            rc.decode_layer(l, hid[W + s, l], w.R[l], w.bias[l], outs[l], copy_stream=copy)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    res["sync"] = dict(ms_per_step=el / K * 1e3, **totals(rc.plan_stats(reset=True)))
    hs, cap = torch.cuda.Stream(), torch.cuda.Stream()
    xin = torch.empty_like(hid[0])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        for l in range(L):
            rc.decode_layer_async(l, xin[l], w.R[l], w.bias[l], outs[l], stream=cap, host_stream=hs)
    rc.reset_cache()
    torch.cuda.synchronize()
    for s in range(W):
        xin.copy_(hid[s])
        g.replay()
    torch.cuda.synchronize()
    rc.plan_stats(reset=True)
    t0 = time.perf_counter()
    for s in range(K):
        xin.copy_(hid[W + s])
        g.replay()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    assert rc.check_device_error() == 0
    res["graph"] = dict(ms_per_step=el / K * 1e3, **totals(rc.plan_stats(reset=True)))
    log(f"high-hit decode: {json.dumps(res)}")
    rc.close()
    del rc, g
    torch.cuda.empty_cache()
    return res


def e2e_at(w: Workload, T, bp, bh):
    """Decode at a larger batch through the same 40% cache (HYBRID with the
    same calibrated bandwidths), cold start, a short run: --e2e-T-steps
    timed steps after half as many warm-up steps, each on its own rows."""
    import torch
    import synth
    from expert_ffn_execution_router_amd import binding as B
    args, c = w.args, w.cfg
    L = c.L
    K = args.e2e_T_steps
    W = max(1, K // 2)
    keys = synth.decode_row_keys(c, args.seed + 2 + T, W + K, T)
    hid = torch.from_numpy(synth.hidden_rows(c, keys.reshape(-1)).reshape(W + K, L, T, c.H).view(np.int16)).to(w.dev)
    outs = torch.empty(L, T, c.H, dtype=torch.bfloat16, device=w.dev)
    rc = w.runtime(c.n_slots, max(T, 64))
    rc.set_policy(B.MOE_POLICY_HYBRID, bp, bh)
    copy = torch.cuda.Stream()
    infos = []
    for s in range(W + K):
        if s == W:
            torch.cuda.synchronize()
            rc.plan_stats(reset=True)
            t0 = time.perf_counter()
        for l in range(L):
            info = rc.decode_layer(l, hid[s, l], w.R[l], w.bias[l], outs[l], copy_stream=copy)
            if s >= W:
                infos.append(info.as_dict())
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    tot = rc.plan_stats(reset=True)
    assert rc.check_device_error() == 0
    uq = sum(i["n_unique"] for i in infos)
    n = len(infos)
    res = {
        "T": T, "warmup_steps": W, "steps": K, "ms_per_step": el / K * 1e3,
        "moe_layer_tokens_per_s": K * L * T / el,
        "hit_rate": sum(i["n_hit"] for i in infos) / max(uq, 1),
        "unique_experts_per_layer": uq / n, "misses_per_layer": sum(i["m"] for i in infos) / n,
        "fills_per_layer": sum(i["q"] for i in infos) / n, "host_per_layer": sum(i["n_host"] for i in infos) / n,
        "t_fill_pred_us_per_layer": sum(i["t_fill_pred_us"] for i in infos) / n,
        "t_host_pred_us_per_layer": sum(i["t_host_pred_us"] for i in infos) / n,
        "host_branch_us_per_layer": tot["host_ms"] * 1e3 / n,
    }
    log(f"decode through the cache at T={T}: {json.dumps(res)}")
    rc.close()
    del rc
    torch.cuda.empty_cache()
    return res


def e2e_async(w: Workload, rc, hid, outs):
    """The same decode steps (cold cache, same rows) with no host read of the
    plan: eager launches of moe_decode_layer_async, then one captured HIP
    graph per step (the host branch a host node) replayed over a static input
    buffer refreshed inside the timed region."""
    import torch
    args, c = w.args, w.cfg
    L, T = c.L, args.e2e_T
    W, K = args.e2e_warmup, args.e2e_steps
    hs = torch.cuda.Stream()
    out = {}

    def totals(t):
        n = max(t["calls"], 1)
        return {"hit_rate": t["n_hit"] / max(t["n_unique"], 1), "misses_per_layer": t["m"] / n,
                "fills_per_layer": t["q"] / n, "host_per_layer": t["n_host"] / n,
                "host_branch_us_per_layer": t["host_ms"] * 1e3 / n}

    # eager launches
    rc.reset_cache()
    rc.plan_stats(reset=True)
    for s in range(W):
        for l in range(L):
            rc.decode_layer_async(l, hid[s, l], w.R[l], w.bias[l], outs[l], host_stream=hs)
    torch.cuda.synchronize()
    rc.plan_stats(reset=True)
    t0 = time.perf_counter()
    for s in range(K):
        for l in range(L):
            rc.decode_layer_async(l, hid[W + s, l], w.R[l], w.bias[l], outs[l], host_stream=hs)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    out["eager"] = dict(ms_per_step=el / K * 1e3, moe_layer_tokens_per_s=K * L * T / el, **totals(rc.plan_stats()))
    # per-stage times of the eager launches (fill kernel included), cache state carried on
    rc.plan_stats(reset=True)
    rc.profile_begin(K * L * 14 + 16)
    for s in range(K):
        for l in range(L):
            rc.decode_layer_async(l, hid[W + s, l], w.R[l], w.bias[l], outs[l], host_stream=hs)
    prof = profile_end(rc)
    out["eager"]["stage_us_per_launch"] = {n: v["ms"] / v["launches"] * 1e3 for n, v in prof.items()
                                           if isinstance(v, dict) and v["launches"]}
    fl = prof.get("fill", {"launches": 0})
    if fl["launches"]:
        st = rc.plan_stats(reset=True)
        out["eager"]["fill_kernel_GBps"] = st["q"] * rc.S / (fl["ms"] * 1e-3) / 1e9
    # one graph per step
    try:
        cap = torch.cuda.Stream()
        xin = torch.empty_like(hid[0])
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for l in range(L):
                rc.decode_layer_async(l, xin[l], w.R[l], w.bias[l], outs[l], stream=cap, host_stream=hs)
    except Exception as ex:
        out["graph"] = {"error": str(ex)}
        return out
    rc.reset_cache()
    torch.cuda.synchronize()
    for s in range(W):
        xin.copy_(hid[s])
        g.replay()
    torch.cuda.synchronize()
    rc.plan_stats(reset=True)
    t0 = time.perf_counter()
    for s in range(K):
        xin.copy_(hid[W + s])
        g.replay()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    assert rc.check_device_error() == 0
    out["graph"] = dict(ms_per_step=el / K * 1e3, moe_layer_tokens_per_s=K * L * T / el, **totals(rc.plan_stats()))
    log(f"device cache control: {json.dumps(out)}")
    return out


def phase_elastic(w: Workload):
    """Rebuilds of the expert cache at step boundaries (decode T=1, HYBRID,
    one captured graph per step, captured again after every rebuild): 40% of
    the pool, shrink in place to 20%, grow into a new pool of 57.8%.  Reports
    each rebuild's wall time and each segment's step time and hit rate."""
    import torch
    import synth
    from expert_ffn_execution_router_amd import binding as B
    args, c = w.args, w.cfg
    L, T, E = c.L, 1, c.E
    W, K = 8, 16
    segs = [("40%", 0.4, None), ("20% in place", 0.2, True), ("57.8% new pool", 0.578, False)]
    keys = synth.decode_row_keys(c, args.seed + 2, len(segs) * (W + K), T)
    hid = torch.from_numpy(synth.hidden_rows(c, keys.reshape(-1)).reshape(-1, L, T, c.H).view(np.int16)).to(w.dev)
    outs = torch.empty(L, T, c.H, dtype=torch.bfloat16, device=w.dev)
    rc = w.runtime(int(round(0.4 * L * E)), 64)
    bp, bh = rc.calibrate()
    rc.set_policy(B.MOE_POLICY_HYBRID, bp, bh)
    hs, cap = torch.cuda.Stream(), torch.cuda.Stream()
    xin = torch.empty_like(hid[0])
    res = {"T": T, "policy": "hybrid", "steps_per_segment": K, "warmup_per_segment": W}
    row = 0
    for name, frac, in_place in segs:
        n = int(round(frac * L * E))
        if in_place is not None:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            rc.resize(n, in_place=in_place)
            dt = time.perf_counter() - t0
        else:
            dt = None
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for l in range(L):
                rc.decode_layer_async(l, xin[l], w.R[l], w.bias[l], outs[l], stream=cap, host_stream=hs)
        for s in range(W):
            xin.copy_(hid[row])
            row += 1
            g.replay()
        torch.cuda.synchronize()
        rc.plan_stats(reset=True)
        t0 = time.perf_counter()
        for s in range(K):
            xin.copy_(hid[row])
            row += 1
            g.replay()
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        st = rc.plan_stats(reset=True)
        res[name] = {"n_slots": n, "rebuild_s": dt, "ms_per_step": el / K * 1e3,
                     "hit_rate": st["n_hit"] / max(st["n_unique"], 1), "misses_per_layer": st["m"] / max(st["calls"], 1)}
        log(f"elastic {name}: {json.dumps(res[name])}")
        del g
    assert rc.check_device_error() == 0
    rc.close()
    del rc
    torch.cuda.empty_cache()
    return res


def phase_prefill(w: Workload):
    """Prefill chunks through the full-layer double buffer, and without it,
    at each chunk size of --prefill-Ts (the 8192-token chunk is the headline
    prefill figure; the others are listed under by_T)."""
    import torch
    import synth
    args, c = w.args, w.cfg
    L = c.L
    Ts = sorted(set(args.prefill_Ts + [args.prefill_T]))
    pcfg = synth.CONFIGS[3].with_layers(L)
    rp = w.runtime(pcfg.n_slots, max(Ts))
    by_T = {Tp: prefill_at(w, rp, pcfg, Tp) for Tp in Ts}
    rp.close()
    del rp
    torch.cuda.empty_cache()
    res = dict(by_T[args.prefill_T])
    res["by_T"] = {str(Tp): r for Tp, r in by_T.items() if Tp != args.prefill_T}
    return res


def prefill_at(w: Workload, rp, pcfg, Tp):
    """One chunk of Tp tokens through the 48 layers: best of --prefill-runs
    double-buffered runs, then one run with the second buffer off."""
    import torch
    import synth
    args, c = w.args, w.cfg
    L, E, k, H, I, S = c.L, c.E, c.k, c.H, c.I, c.expert_bytes
    comp, copy = torch.cuda.Stream(), torch.cuda.Stream()
    hp = torch.empty(Tp, H, dtype=torch.int16, device=w.dev)
    out_p = torch.empty(Tp, H, dtype=torch.bfloat16, device=w.dev)
    pk = synth.keys_range(synth.key(args.seed, pcfg.config_id, 4, 0xF111), 0, Tp)
    hp.copy_(torch.from_numpy(synth.hidden_rows(pcfg, pk).view(np.int16)))
    torch.cuda.synchronize()
    runs = {}
    for dbuf in [True] * max(1, args.prefill_runs - 1) + [False, True]:
        rp.reset_cache()
        torch.cuda.synchronize()
        rp.profile_begin(L * 16 + 16)
        t0 = time.perf_counter()
        with torch.cuda.stream(comp):
            for l in range(L):
                rp.prefill_layer(l, hp, w.R[l], None, out_p, stream=comp, copy_stream=copy, double_buffer=dbuf)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        runs.setdefault(dbuf, []).append((el, profile_end(rp)))
    el_on, pprof = min(runs[True], key=lambda r: r[0])
    el_off = runs[False][0][0]
    flops = 6.0 * Tp * k * H * I * L
    # the overflow rows' small-batch GEMMs (and their sums) count as GEMM time
    gemm_ms = pprof["gemm1"]["ms"] + pprof["gemm2"]["ms"] + pprof["tail"]["ms"]
    res = {
        "T": Tp, "layers": L, "chunk_s": el_on, "tokens_per_s": Tp / el_on,
        "h2d_GBps": L * E * S / el_on / 1e9,
        "gemm_ms_per_layer": gemm_ms / L,
        "mfma_frac_bf16": flops / (gemm_ms * 1e-3) / BF16_PEAK,
        "stage_ms_per_layer": {n: v["ms"] / L for n, v in pprof.items() if isinstance(v, dict) and v["launches"]},
        "chunk_s_double_buffer_off": el_off,
        "loss_without_double_buffer": 1.0 - el_on / el_off,
    }
    log(json.dumps(res))
    return res


def phase_fallback(w: Workload):
    """The prefill regimes below two full layers of slots, and the hand-off
    from a prefill chunk to decode: (a) 8192-token chunk with 1.5 layers of
    slots (full layers through one buffer), (b) with half a layer of slots
    (on demand, capacity overflow on the host; two layers only), (c) decode
    T=1 steps right after a double-buffered chunk against the same steps
    from a cold cache (40% of the pool, HYBRID)."""
    import torch
    import synth
    from expert_ffn_execution_router_amd import binding as B
    args, c = w.args, w.cfg
    L, E, H = c.L, c.E, c.H
    Tp = args.prefill_T
    pcfg = synth.CONFIGS[3].with_layers(L)
    hp = torch.empty(Tp, H, dtype=torch.int16, device=w.dev)
    pk = synth.keys_range(synth.key(args.seed, pcfg.config_id, 4, 0xF111), 0, Tp)
    hp.copy_(torch.from_numpy(synth.hidden_rows(pcfg, pk).view(np.int16)))
    out_p = torch.empty(Tp, H, dtype=torch.bfloat16, device=w.dev)
    comp, copy = torch.cuda.Stream(), torch.cuda.Stream()
    res = {"T": Tp}

    def chunk(rt, layers):
        rcs = []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(comp):
            for l in range(layers):
                rcs.append(rt.prefill_layer(l, hp, w.R[l], None, out_p, stream=comp, copy_stream=copy))
        torch.cuda.synchronize()
        return time.perf_counter() - t0, rcs

    rt = w.runtime(E + E // 2, Tp)
    el, rcs = chunk(rt, L)
    res["single_buffer"] = {"n_slots": E + E // 2, "chunk_s": el, "status": sorted(set(rcs)),
                            "h2d_GBps": L * E * c.expert_bytes / el / 1e9}
    log(f"fallback single buffer: {json.dumps(res['single_buffer'])}")
    rt.close()
    rt = w.runtime(E // 2, Tp)
    rt.set_policy(B.MOE_POLICY_OFFLOAD)
    el, rcs = chunk(rt, 2)
    res["on_demand"] = {"n_slots": E // 2, "layers": 2, "s_per_layer": el / 2, "status": sorted(set(rcs))}
    log(f"fallback on demand: {json.dumps(res['on_demand'])}")
    rt.close()
    # hand-off
    rt = w.runtime(pcfg.n_slots, Tp)
    bp, bh = rt.calibrate()
    rt.set_policy(B.MOE_POLICY_HYBRID, bp, bh)
    K = 4
    keys = synth.decode_row_keys(c, args.seed + 3, K, 1)
    hid = torch.from_numpy(synth.hidden_rows(c, keys.reshape(-1)).reshape(K, L, 1, H).view(np.int16)).to(w.dev)
    o1 = torch.empty(1, H, dtype=torch.bfloat16, device=w.dev)

    def decode_steps():
        out = []
        for s_ in range(K):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            infos = [rt.decode_layer(l, hid[s_, l], w.R[l], w.bias[l], o1, copy_stream=copy) for l in range(L)]
            torch.cuda.synchronize()
            out.append({"ms": (time.perf_counter() - t0) * 1e3,
                        "hit_rate": sum(i.n_hit for i in infos) / max(sum(i.n_unique for i in infos), 1)})
        return out

    rt.reset_cache()
    chunk(rt, L)
    warm = decode_steps()
    rt.reset_cache()
    torch.cuda.synchronize()
    cold = decode_steps()
    res["handoff"] = {"n_slots": pcfg.n_slots, "after_prefill": warm, "cold": cold}
    log(f"hand-off: {json.dumps(res['handoff'])}")
    assert rt.check_device_error() == 0
    rt.close()
    torch.cuda.empty_cache()
    return res


def serve(args, c, name, Tp, decode):
    """One shape end to end as its workload states it: a Tp-token prefill
    chunk through the full-layer double buffer, then decode steps through the
    slot cache with the q* split on the bandwidths calibrated at startup, one
    captured graph per step and batch size (decode: [(T, steps)], run in
    order, each after 8 warm-up steps and on the cache the previous left)."""
    import torch
    import synth
    from expert_ffn_execution_router_amd import binding as B
    from expert_ffn_execution_router_amd.runtime import HostPool, MoeRuntime
    L, E, k, H, I, S = c.L, c.E, c.k, c.H, c.I, c.expert_bytes
    dev = torch.device("cuda:0")
    t0 = time.time()
    pool = HostPool(L * E * S)
    synth.fill_pool(pool.ptr, c, args.seed)
    log(f"{name} pool {L * E * S / 1e9:.1f} GB pinned and filled in {time.time() - t0:.1f}s")
    R = [torch.from_numpy(synth.router_weights(c, args.seed, l)).to(dev) for l in range(L)]
    bias = [None if b is None else torch.from_numpy(b).to(dev)
            for b in (synth.router_bias(c, args.seed, l) for l in range(L))]
    W = 8
    rt = MoeRuntime(L, E, k, H, I, c.fmt, c.n_slots, max([Tp] + [t for t, _ in decode]), pool,
                    host_threads=args.host_threads)
    bp, bh = rt.calibrate()
    rt.set_policy(B.MOE_POLICY_HYBRID, bp, bh)
    rt.reset_cache()
    hp = torch.from_numpy(synth.hidden(c, args.seed, Tp, 0x5E5).view(np.int16)).to(dev)
    out_p = torch.empty(Tp, H, dtype=torch.bfloat16, device=dev)
    comp, copy = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(comp):
        for l in range(L):
            rt.prefill_layer(l, hp, R[l], bias[l], out_p, stream=comp, copy_stream=copy)
    torch.cuda.synchronize()
    el_p = time.perf_counter() - t0
    del hp, out_p
    res = {"workload": f"{name}: {L} layers, E={E} top-{k}, H={H}, I={I}, {L * E * S / 1e9:.1f} GB pool, "
                       f"{c.n_slots} slots ({100.0 * c.n_slots / (L * E):.0f}%)",
           "prefill": {"T": Tp, "chunk_s": el_p, "tokens_per_s": Tp / el_p, "h2d_GBps": L * E * S / el_p / 1e9},
           "B_P_GBps": bp, "B_H_GBps": bh}
    for T, K in decode:
        keys = synth.decode_row_keys(c, args.seed + T, W + K, T)
        hid = torch.from_numpy(synth.hidden_rows(c, keys.reshape(-1)).reshape(W + K, L, T, H).view(np.int16)).to(dev)
        outs = torch.empty(L, T, H, dtype=torch.bfloat16, device=dev)
        xin = torch.empty_like(hid[0])
        hs, cap = torch.cuda.Stream(), torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for l in range(L):
                rt.decode_layer_async(l, xin[l], R[l], bias[l], outs[l], stream=cap, host_stream=hs)
        for s_ in range(W):
            xin.copy_(hid[s_])
            g.replay()
        torch.cuda.synchronize()
        rt.plan_stats(reset=True)
        t0 = time.perf_counter()
        for s_ in range(K):
            xin.copy_(hid[W + s_])
            g.replay()
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        st = rt.plan_stats()
        assert rt.check_device_error() == 0
        n = max(st["calls"], 1)
        res[f"decode_T{T}"] = {
            "T": T, "steps": K, "warmup": W, "ms_per_step": el / K * 1e3,
            "moe_layer_tokens_per_s": K * L * T / el,
            "hit_rate": st["n_hit"] / max(st["n_unique"], 1), "misses_per_layer": st["m"] / n,
            "fills_per_layer": st["q"] / n, "host_per_layer": st["n_host"] / n,
            "host_branch_us_per_layer": st["host_ms"] * 1e3 / n}
        log(f"{name} decode T={T}: {json.dumps(res[f'decode_T{T}'])}")
        del g, hid, outs, xin
    log(f"{name} serving: {json.dumps(res)}")
    rt.close()
    del rt
    torch.cuda.empty_cache()
    pool.free()
    return res


def phase_mxfp4_serving(args):
    """The MXFP4 shape (E=256 top-8, H=6144, I=2048, a slot cache of 25% of
    the pool): one 16384-token prefill chunk, then 512 decode steps at T=1
    (Zipf bias, 0.7 row reuse).  --serving-layers of its 16 layers (the whole
    82 GB pool is more than one process can pin here; per-layer work and the
    cache fraction are unchanged)."""
    import synth
    c = synth.CONFIGS[5].with_layers(args.serving_layers)
    return serve(args, c, "mxfp4", 16384, [(1, args.serving_steps)])


def phase_fp8_serving(args):
    """The fp8 shape (E=256 top-6, H=4096, I=2048, fp32 scale per 128x128
    block, a slot cache of 30% of the pool): one 4096-token prefill chunk,
    then decode at T=1 and T=32 through the cache.  --fp8-serving-layers of
    its 43 layers (the 277 GB pool cannot be pinned by one process; per-layer
    work and the cache fraction are unchanged)."""
    import synth
    c = synth.CONFIGS[4].with_layers(args.fp8_serving_layers)
    return serve(args, c, "fp8_e4m3_b128", 4096, [(1, args.fp8_serving_steps), (32, args.fp8_serving_steps // 4)])


def phase_formats(args):
    """The fp8 (43-layer E=256 top-6 H=4096 I=2048 shape), MXFP4 (16-layer
    E=256 top-8 H=6144 I=2048 shape) and NVFP4 (the 48-layer E=128 top-8
    H=2048 I=768 decode shape) paths with every expert resident:
    decode steps at the small token counts, and one prefill-shaped batch per
    layer.  Layers are cut to --format-layers so the pools fit host memory;
    per-layer work is unchanged."""
    import torch
    import synth
    from expert_ffn_execution_router_amd.runtime import HostPool, MoeRuntime
    out = {}
    dev = torch.device("cuda:0")
    import dataclasses
    shapes = set(args.format_shapes.split(","))
    for cid, dec_T, pf_T, pf_bound in ((4, (1, 32), 4096, "hbm"), (5, (1,), 16384, "mfma"),
                                       (6, (1, 32, 64), 8192, "mfma")):
        if {4: "fp8", 5: "mxfp4", 6: "nvfp4"}[cid] not in shapes:
            continue
        if cid == 6:       # the decode shape with NVFP4 experts (the pages' laptop build of that model)
            c = dataclasses.replace(synth.CONFIGS[2], name="decode_nvfp4", fmt=synth.FMT_NVFP4)
            c = c.with_layers(args.format_layers)
        else:
            c = synth.CONFIGS[cid].with_layers(args.format_layers)
        L, E, k, H, I, S = c.L, c.E, c.k, c.H, c.I, c.expert_bytes
        name = {4: "fp8_e4m3_b128", 5: "mxfp4", 6: "nvfp4"}[cid]
        pool = HostPool(L * E * S)
        synth.fill_pool(pool.ptr, c, args.seed)
        R = [torch.from_numpy(synth.router_weights(c, args.seed, l)).to(dev) for l in range(L)]
        bias = [None if b is None else torch.from_numpy(b).to(dev)
                for b in (synth.router_bias(c, args.seed, l) for l in range(L))]
        rt = MoeRuntime(L, E, k, H, I, c.fmt, L * E, max(max(dec_T), pf_T), pool, host_threads=args.host_threads)
        for l in range(L):
            rt.admit(l, list(range(E)))
        torch.cuda.synchronize()
        table = rt.slot_table()
        rows = [table[l * E:(l + 1) * E] for l in range(L)]
        res = {"workload": f"{name}: E={E} top-{k} H={H} I={I}, {L} layers resident", "expert_bytes": S}
        wgu = 2 * S / 3                          # gate + up bytes of one expert (scales included)
        for T in dec_T:
            K, W = 16, 4
            keys = synth.decode_row_keys(c, args.seed, W + K, T)
            hid = torch.from_numpy(synth.hidden_rows(c, keys.reshape(-1)).reshape(W + K, L, T, H).view(np.int16)).to(dev)
            o = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
            ids = torch.empty(T, k, dtype=torch.int32, device=dev)
            wts = torch.empty(T, k, dtype=torch.float32, device=dev)
            n_active = np.zeros((K, L))
            for s in range(K):
                for l in range(L):
                    rt.route(hid[W + s, l], R[l], bias[l], ids, wts)
                    n_active[s, l] = len(torch.unique(ids).cpu())
            for s in range(W):
                for l in range(L):
                    rt.forward(l, hid[s, l], R[l], bias[l], rows[l], o)
            torch.cuda.synchronize()
            rt.profile_begin(K * L * 12 + 16)
            for s in range(K):
                for l in range(L):
                    rt.forward(l, hid[W + s, l], R[l], bias[l], rows[l], o)
            prof = profile_end(rt)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for s in range(K):
                for l in range(L):
                    rt.forward(l, hid[W + s, l], R[l], bias[l], rows[l], o)
            torch.cuda.synchronize()
            wall = (time.perf_counter() - t0) / (K * L)
            assert rt.check_device_error() == 0
            st = {n: v["ms"] / v["launches"] * 1e3 for n, v in prof.items() if isinstance(v, dict) and v["launches"]}
            xb, ab = (2, 2) if cid == 6 else (1, 4)        # token and A bytes per value
            g1_bytes = float(n_active.mean() * wgu + T * k * H * xb + T * k * I * ab)
            layer_bytes = float(n_active.mean() * S + E * H * 4 + 2 * T * H * 2)
            gpu_us = sum(st.values())
            res[f"decode_T{T}"] = {
                "tokens_per_s_eager": T / wall, "layer_wall_us": wall * 1e6, "gpu_layer_us": gpu_us,
                "stage_us": st, "mean_active_experts": float(n_active.mean()),
                "gemm1_GBps": g1_bytes / (st["gemm1"] * 1e-6) / 1e9,
                "gemm1_hbm_frac": g1_bytes / (st["gemm1"] * 1e-6) / HBM_PEAK,
                "layer_hbm_frac_of_gpu_time": layer_bytes / (gpu_us * 1e-6) / HBM_PEAK,
            }
            log(f"{name} decode T={T}: {json.dumps(res[f'decode_T{T}'])}")
            del hid
        # prefill-shaped batch: one forward per layer
        hp = torch.from_numpy(synth.hidden(c, args.seed, pf_T, 7).view(np.int16)).to(dev)
        op = torch.empty(pf_T, H, dtype=torch.bfloat16, device=dev)

        # the NVFP4 experts sit on the decode shape, whose router bias is the
        # decode workload's Zipf prior; its prefill batch takes the prefill
        # shape's unbiased routing (nearly every expert ~512 rows at 8192)
        pbias = [None] * L if cid == 6 else bias

        def prefill_pass(key, kernel, peak):
            rt.forward(0, hp, R[0], pbias[0], rows[0], op)
            torch.cuda.synchronize()
            rt.profile_begin(L * 16 + 16)
            for l in range(L):
                rt.forward(l, hp, R[l], pbias[l], rows[l], op)
            prof = profile_end(rt)
            torch.cuda.synchronize()
            assert rt.check_device_error() == 0
            # per layer (one forward each): the tiled GEMMs, the streaming
            # kernels' sums and the overflow rows' GEMMs
            st = {n: v["ms"] / L * 1e3 for n, v in prof.items() if isinstance(v, dict) and v["launches"]}
            gemm_us = st["gemm1"] + st["gemm2"] + st.get("fixup", 0.0) + st.get("tail", 0.0)
            flops = 6.0 * pf_T * k * H * I
            res[key] = {
                "bound": pf_bound, "gemm_us": gemm_us, "gpu_layer_us": sum(st.values()), "stage_us": st,
                "weights_hbm_frac": E * S / (gemm_us * 1e-6) / HBM_PEAK,
                "mfma_frac": flops / (gemm_us * 1e-6) / peak, "mfma_peak_TFLOPs": peak / 1e12, "kernel": kernel,
            }
            log(f"{name} {key}: {json.dumps(res[key])}")

        peak = {4: FP8_PEAK, 5: FP4_PEAK, 6: BF16_PEAK}[cid]
        prefill_pass(f"prefill_T{pf_T}", "gemm_pf16 (LDS-tiled fp16-MFMA grouped GEMM, NVFP4 dequantised in "
                     "registers)" if cid == 6 else "gemm_pf_q8 (LDS-tiled scaled-MFMA grouped GEMM)", peak)
        if cid == 5:     # MXFP6 activations: E2M1 x E2M3 at the 6/4-bit MFMA rate
            from expert_ffn_execution_router_amd import binding as B
            rt.set_activations(B.MOE_ACT_MXFP6)
            prefill_pass(f"prefill_T{pf_T}_mxfp6", "gemm_pf_q8 (E2M1 weights x MXFP6 activations)", FP4_PEAK)
            rt.set_activations(B.MOE_ACT_DEFAULT)
        out[name] = res
        rt.close()
        del rt, hp, op
        torch.cuda.empty_cache()
        pool.free()
    return out


def phase_policies(args):
    """Miss rates of three expert placements at matched slot counts, replayed
    over synthetic decode routing (T=1, the 0.7-reuse locality model) of the
    decode-shaped (48 layers, E=128 top-8, Zipf bias) and large-pool (43
    layers, E=256 top-6, log-normal router scales) generators: the device
    global LRU, a hot set frozen from a 2048-token prefill chunk's routing,
    and a static layer split.  Routing runs through the library's router."""
    import torch
    import synth
    from expert_ffn_execution_router_amd import policies as P
    from expert_ffn_execution_router_amd.runtime import HostPool, MoeRuntime
    dev = torch.device("cuda:0")
    W, K, Tp = 16, args.policy_steps, 2048
    caps = (0.11, 0.2, 0.3, 0.37, 0.4, 0.5, 0.578)
    out = {}
    for cid in (2, 4):
        c = synth.CONFIGS[cid]
        L, E, k, H = c.L, c.E, c.k, c.H
        t0 = time.time()
        # routing context: one layer's shapes, router weights passed per call
        rpool = HostPool(E * synth.expert_bytes(0, H, 128))
        rrt = MoeRuntime(1, E, k, H, 128, 0, 0, 4096, rpool)
        keys = synth.decode_row_keys(c, args.seed, W + K, 1)
        trace = np.empty((W + K, L, 1, k), dtype=np.int32)
        prefill = np.empty((L, Tp, k), dtype=np.int32)
        for l in range(L):
            R = torch.from_numpy(synth.router_weights(c, args.seed, l)).to(dev)
            b = synth.router_bias(c, args.seed, l)
            b = None if b is None else torch.from_numpy(b).to(dev)
            x = torch.from_numpy(synth.hidden_rows(c, keys[:, l].reshape(-1)).view(np.int16)).to(dev)
            trace[:, l] = P.route_rows(rrt, x, R, b).reshape(W + K, 1, k)
            xp = torch.from_numpy(synth.hidden(c, args.seed, Tp, 0x9F0000 + l).view(np.int16)).to(dev)
            prefill[l] = P.route_rows(rrt, xp, R, b)
        rrt.close()
        rpool.free()
        log(f"policies C{cid}: routed {W + K} decode steps and a {Tp}-token prefill in {time.time() - t0:.1f}s")
        # LRU context: the same L, E, k; planning never touches expert bytes
        S = synth.expert_bytes(0, 256, 128)
        lpool = HostPool(L * E * S)
        res = {"workload": f"{c.name}: {L} layers, E={E} top-{k}, decode T=1, {W} warm-up + {K} counted steps, "
                           f"prefill chunk {Tp} tokens",
               "mean_unique_per_layer": float(np.mean([len(np.unique(trace[s, l])) for s in range(W, W + K)
                                                       for l in range(L)]))}
        for cap in caps:
            n = max(k, int(round(cap * L * E)))
            lrt = MoeRuntime(L, E, k, 256, 128, 0, n, 64, lpool)
            t1 = time.time()
            lm, lu = P.lru_replay(lrt, trace, W)
            lrt.close()
            hm, hu = P.fixed_replay(P.prefill_hot_set(prefill, E, n), trace, W)
            sm, su = P.fixed_replay(P.static_split(L, E, n), trace, W)
            assert lu == hu == su
            res[f"{cap:.3f}"] = {"n_slots": n, "lru": lm / lu, "prefill_hot_set": hm / hu, "static_split": sm / su}
            log(f"policies C{cid} capacity {cap:.3f} ({n} slots): {json.dumps(res[f'{cap:.3f}'])} "
                f"[{time.time() - t1:.1f}s]")
        lpool.free()
        out[f"config{cid}"] = res
        torch.cuda.empty_cache()
    return out


def phase_cpu(w: Workload):
    """The float64 oracle on a bounded sample of the decode workload."""
    from threadpoolctl import threadpool_info
    from oracle import moe as M
    args, c = w.args, w.cfg
    L, E, k, H, I, T, S = c.L, c.E, c.k, c.H, c.I, args.T, c.expert_bytes
    cores = len(os.sched_getaffinity(0))
    blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    pool_np = w.pool.array().reshape(L * E, S)
    nl = min(args.cpu_layers, L)
    t0 = time.perf_counter()
    for l in range(nl):
        wcache = {}

        def wf(e, l=l):
            if e not in wcache:
                wcache[e] = M.dequant_expert(pool_np[l * E + e], c.fmt, H, I)
            return wcache[e]
        M.moe_layer(w.hid_np[args.warmup, l], w.R[l].cpu().numpy(), w.bias[l].cpu().numpy(), k, wf, fmt=c.fmt,
                    mode="exact")
    el = time.perf_counter() - t0
    # the same oracle with its BLAS held to one thread, on fewer layers
    from threadpoolctl import threadpool_limits
    n1 = max(1, min(args.cpu_layers // 5, L))
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for l in range(n1):
            wcache = {}

            def wf1(e, l=l):
                if e not in wcache:
                    wcache[e] = M.dequant_expert(pool_np[l * E + e], c.fmt, H, I)
                return wcache[e]
            M.moe_layer(w.hid_np[args.warmup, l], w.R[l].cpu().numpy(), w.bias[l].cpu().numpy(), k, wf1,
                        fmt=c.fmt, mode="exact")
        el1 = time.perf_counter() - t0
    res = {
        "value": nl * T / el, "unit": "MoE-layer tokens/s", "cores": int(blas_threads), "kind": "oracle",
        "sample": f"layers 0-{nl - 1} of the first timed decode step (T={T}), float64 NumPy oracle, "
                  f"{cores} host cores visible",
        "seconds": el,
        "one_thread": {"value": n1 * T / el1, "cores": 1, "seconds": el1,
                       "sample": f"layers 0-{n1 - 1} of the same step, BLAS limited to one thread"},
    }
    log(json.dumps(res))
    return res


def main():
    args = parse()
    if args.copy_probe:
        copy_probe()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path has no multi-GPU mode",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    from expert_ffn_execution_router_amd import binding as B
    B.lib()   # fail loudly when the library is missing
    synth.lib()
    torch.cuda.init()
    needs_w = bool(args.phase_set & {"decode", "e2e", "prefill", "cpu", "elastic", "fallback"})
    w = Workload(args) if needs_w else None
    c = w.cfg if needs_w else synth.CONFIGS[2].with_layers(args.layers)
    line = {
        "metric": METRIC, "value": None, "unit": "MoE-layer tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"decode, {c.L} MoE layers, E={c.E} top-{c.k}, H={c.H}, I={c.I}, bf16 experts, "
                               f"T={args.T} tokens per step, Zipf(1.1) router bias, 0.7 row reuse, every expert "
                               f"resident in HBM",
                   "global_batch": args.T, "layers": c.L, "parallelism": "single GPU"},
    }
    if "decode" in args.phase_set:
        value, elapsed, roofline, detail = phase_decode(w)
        line["value"] = value
        line["ms_per_step"] = elapsed / args.steps * 1e3
        line["roofline"] = roofline
        line["decode_resident"] = detail
    if "e2e" in args.phase_set:
        line["decode_cache40_e2e"] = phase_e2e(w)
    if "prefill" in args.phase_set:
        line["prefill_chunk"] = phase_prefill(w)
    if "elastic" in args.phase_set:
        line["elastic_cache"] = phase_elastic(w)
    if "fallback" in args.phase_set:
        line["prefill_fallback_and_handoff"] = phase_fallback(w)
    if "cpu" in args.phase_set:
        line["cpu_baseline"] = phase_cpu(w)
    if "formats" in args.phase_set:
        line["formats_resident"] = phase_formats(args)
    if "policies" in args.phase_set:
        line["placement_miss_rates"] = phase_policies(args)
    if "mxfp4_serving" in args.phase_set:
        line["mxfp4_serving"] = phase_mxfp4_serving(args)
    if "fp8_serving" in args.phase_set:
        line["fp8_serving"] = phase_fp8_serving(args)
    print(json.dumps(line), flush=True)
    if w is not None:
        w.pool.free()


if __name__ == "__main__":
    main()
