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
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np


def log(*a):
    print(*a, file=sys.stderr, flush=True)


METRIC = "MoE-layer tokens/s (decode T≤64, prefill 8k); % HBM BW / % MFMA peak"
HBM_PEAK = 8.0e12
BF16_PEAK = 2.5e15


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--T", type=int, default=64)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--layers", type=int, default=48)
    ap.add_argument("--no-e2e", action="store_true", help="skip the slot-cache decode phase")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill phase")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--prefill-T", type=int, default=8192)
    ap.add_argument("--cpu-layers", type=int, default=3)
    ap.add_argument("--host-threads", type=int, default=16)
    ap.add_argument("--copy-probe", action="store_true",
                    help="only copy 1 GiB device->device 3 times (calibrates HBM byte counters)")
    return ap.parse_args()


def counted_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None when the kernel source changed since it was taken."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", "decode_T64_bf16_gemm_hbm_counters.md")
    src = os.path.join(root, "expert_ffn_execution_router_amd", "csrc", "gemm_dec.hip")
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
    from expert_ffn_execution_router_amd.runtime import HostPool, MoeRuntime

    B.lib()   # fail loudly when the library is missing
    synth.lib()
    cfg = synth.CONFIGS[2].with_layers(args.layers)
    L, E, k, H, I, T = cfg.L, cfg.E, cfg.k, cfg.H, cfg.I, args.T
    S = cfg.expert_bytes
    K, W = args.steps, args.warmup
    torch.cuda.init()
    dev = torch.device("cuda:0")

    # ------------------------------------------------------------------ inputs
    t0 = time.time()
    pool = HostPool(L * E * S)
    log(f"pinned host pool {L * E * S / 1e9:.1f} GB allocated in {time.time() - t0:.1f}s")
    t0 = time.time()
    synth.fill_pool(pool.ptr, cfg, args.seed)
    log(f"host pool filled in {time.time() - t0:.1f}s")
    R = [torch.from_numpy(synth.router_weights(cfg, args.seed, l)).to(dev) for l in range(L)]
    bias = [torch.from_numpy(synth.router_bias(cfg, args.seed, l)).to(dev) for l in range(L)]
    keys = synth.decode_row_keys(cfg, args.seed, W + K, T)
    hid_np = synth.hidden_rows(cfg, keys.reshape(-1)).reshape(W + K, L, T, H)
    hidden = torch.from_numpy(hid_np.view(np.int16)).to(dev)          # resident in HBM before timing
    outs = torch.empty(L, T, H, dtype=torch.bfloat16, device=dev)
    result = {}

    # ------------------------------------------------ resident pool: the value
    rt = MoeRuntime(L, E, k, H, I, cfg.fmt, L * E, max(T, 64), pool, host_threads=args.host_threads)
    t0 = time.time()
    for l in range(L):
        rt.admit(l, list(range(E)))
    torch.cuda.synchronize()
    log(f"resident pool: {L * E} experts copied to HBM in {time.time() - t0:.1f}s")
    table = rt.slot_table()
    rows = [table[l * E:(l + 1) * E] for l in range(L)]
    # routing of every timed (step, layer), for the algorithmic byte counts
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    wts = torch.empty(T, k, dtype=torch.float32, device=dev)
    n_active = np.zeros((K, L), dtype=np.int64)
    for s in range(K):
        for l in range(L):
            rt.route(hidden[W + s, l], R[l], bias[l], ids, wts)
            n_active[s, l] = len(torch.unique(ids).cpu())
    torch.cuda.synchronize()

    def step(s):
        for l in range(L):
            rt.forward(l, hidden[s, l], R[l], bias[l], rows[l], outs[l])

    for s in range(W):
        step(s)
    torch.cuda.synchronize()
    rt.profile_begin(K * L * 8 + 16)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        step(W + s)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    prof = rt.profile_end()
    assert rt.check_device_error() == 0
    value = K * L * T / elapsed
    log(f"decode resident: {elapsed / K * 1e3:.3f} ms/step, {value:.0f} MoE-layer tokens/s")

    # algorithmic bytes (each active expert's weights read once; routed rows and outputs once)
    tk = T * k
    g1_bytes = (n_active * 2 * I * H * 2 + tk * H * 2 + tk * I * 2).sum()
    g2_bytes = (n_active * H * I * 2 + tk * I * 2 + tk * H * 2).sum()
    layer_bytes = (n_active * S + E * H * 4 + 2 * T * H * 2).sum()
    n_calls = K * L
    g1_ms = prof["gemm1"]["ms"] / max(prof["gemm1"]["launches"], 1)
    g2_ms = prof["gemm2"]["ms"] / max(prof["gemm2"]["launches"], 1)
    stage_ms = {n: v["ms"] / max(v["launches"], 1) for n, v in prof.items() if isinstance(v, dict) and v["launches"]}
    gpu_layer_ms = sum(stage_ms.values())
    g1_achieved = g1_bytes / n_calls / (g1_ms * 1e-3)
    result["roofline"] = {
        "bound": "hbm", "kernel": "gemm_dec_bf16 (grouped gate/up + SwiGLU)",
        "achieved": g1_achieved / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
        "frac": g1_achieved / HBM_PEAK,
        "traffic": counted_traffic("void gemm_dec<0, true, 2>") if T > 8 else None,
        "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated)",
        "bytes_per_launch": float(g1_bytes / n_calls), "avg_launch_us": g1_ms * 1e3,
    }
    result["decode_resident"] = {
        "ms_per_step": elapsed / K * 1e3, "layer_wall_us": elapsed / n_calls * 1e6,
        "stage_us": {n: v * 1e3 for n, v in stage_ms.items()},
        "gpu_layer_us": gpu_layer_ms * 1e3,
        "layer_hbm_frac_of_gpu_time": float(layer_bytes / n_calls / (gpu_layer_ms * 1e-3) / HBM_PEAK),
        "layer_hbm_frac_of_wall": float(layer_bytes / elapsed / HBM_PEAK),
        "gemm2_GBps": float(g2_bytes / n_calls / (g2_ms * 1e-3) / 1e9),
        "mean_active_experts": float(n_active.mean()),
        "layer_bytes_MB": float(layer_bytes / n_calls / 1e6),
    }
    log(json.dumps(result["roofline"]))
    log(json.dumps(result["decode_resident"]))
    rt.close()
    del rt
    torch.cuda.empty_cache()

    # --------------------------------------- the same steps through the cache
    if not args.no_e2e:
        n_slots = cfg.n_slots
        rc = MoeRuntime(L, E, k, H, I, cfg.fmt, n_slots, max(T, 64), pool, host_threads=args.host_threads)
        bp, bh = rc.calibrate()
        rc.set_policy(B.MOE_POLICY_HYBRID, bp, bh)
        copy = torch.cuda.Stream()
        ke = max(2, K // 2)
        infos = []

        def e2e_step(s, record):
            for l in range(L):
                info = rc.decode_layer(l, hidden[s % (W + K), l], R[l], bias[l], outs[l], copy_stream=copy)
                if record:
                    infos.append(info.as_dict())

        for s in range(W):
            e2e_step(s, False)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(ke):
            e2e_step(W + s, True)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        assert rc.check_device_error() == 0
        uq = sum(i["n_unique"] for i in infos)
        result["decode_cache40_e2e"] = {
            "note": "PCIe and host included; not the value",
            "n_slots": n_slots, "policy": "hybrid", "B_P_GBps": bp, "B_H_GBps": bh,
            "q_star_over_m": bp / bh, "steps": ke,
            "moe_layer_tokens_per_s": ke * L * T / el, "ms_per_step": el / ke * 1e3,
            "hit_rate": sum(i["n_hit"] for i in infos) / max(uq, 1),
            "misses_per_layer": sum(i["m"] for i in infos) / len(infos),
            "fills_per_layer": sum(i["q"] for i in infos) / len(infos),
            "host_per_layer": sum(i["n_host"] for i in infos) / len(infos),
            "t_fill_pred_us_per_layer": sum(i["t_fill_pred_us"] for i in infos) / len(infos),
            "t_host_pred_us_per_layer": sum(i["t_host_pred_us"] for i in infos) / len(infos),
        }
        log(json.dumps(result["decode_cache40_e2e"]))
        rc.close()
        del rc
        torch.cuda.empty_cache()

    # ------------------------------------------------ prefill, double buffered
    if not args.no_prefill:
        Tp = args.prefill_T
        pcfg = synth.CONFIGS[3].with_layers(L)
        rp = MoeRuntime(L, E, k, H, I, pcfg.fmt, pcfg.n_slots, Tp, pool, host_threads=args.host_threads)
        comp, copy = torch.cuda.Stream(), torch.cuda.Stream()
        hp = torch.empty(Tp, H, dtype=torch.int16, device=dev)
        out_p = torch.empty(Tp, H, dtype=torch.bfloat16, device=dev)
        pk = synth.keys_range(synth.key(args.seed, pcfg.config_id, 4, 0xF111), 0, Tp)
        hp.copy_(torch.from_numpy(synth.hidden_rows(pcfg, pk).view(np.int16)))
        torch.cuda.synchronize()
        runs = {}
        for dbuf in (True, False, True):
            rp.reset_cache()
            torch.cuda.synchronize()
            rp.profile_begin(L * 8 + 16)
            t0 = time.perf_counter()
            with torch.cuda.stream(comp):
                for l in range(L):
                    rp.prefill_layer(l, hp, R[l], None, out_p, stream=comp, copy_stream=copy, double_buffer=dbuf)
            torch.cuda.synchronize()
            el = time.perf_counter() - t0
            pprof = rp.profile_end()
            runs.setdefault(dbuf, []).append((el, pprof))
        el_on, pprof = min(runs[True], key=lambda r: r[0])
        el_off, _ = runs[False][0]
        flops = 6.0 * Tp * k * H * I * L
        gemm_ms = pprof["gemm1"]["ms"] + pprof["gemm2"]["ms"]
        pool_bytes = L * E * S
        result["prefill_chunk"] = {
            "T": Tp, "layers": L, "chunk_s": el_on, "tokens_per_s": Tp / el_on,
            "h2d_GBps": pool_bytes / el_on / 1e9,
            "gemm_ms_per_layer": gemm_ms / L,
            "mfma_frac_bf16": flops / (gemm_ms * 1e-3) / BF16_PEAK,
            "gpu_ms_per_layer": sum(v["ms"] for v in pprof.values() if isinstance(v, dict)) / L,
            "chunk_s_double_buffer_off": el_off,
            "loss_without_double_buffer": 1.0 - el_on / el_off,
        }
        log(json.dumps(result["prefill_chunk"]))
        rp.close()
        del rp
        torch.cuda.empty_cache()

    # ------------------------------------------- CPU baseline (the oracle)
    if not args.no_cpu:
        from threadpoolctl import threadpool_info
        from oracle import moe as M
        cores = len(os.sched_getaffinity(0))
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        pool_np = pool.array().reshape(L * E, S)
        nl = min(args.cpu_layers, L)
        t0 = time.perf_counter()
        for l in range(nl):
            wcache = {}

            def wf(e, l=l):
                if e not in wcache:
                    wcache[e] = M.dequant_expert(pool_np[l * E + e], cfg.fmt, H, I)
                return wcache[e]
            M.moe_layer(hid_np[W, l], R[l].cpu().numpy(), bias[l].cpu().numpy(), k, wf, fmt=cfg.fmt,
                        mode="exact")
        el = time.perf_counter() - t0
        result["cpu_baseline"] = {
            "value": nl * T / el, "unit": "MoE-layer tokens/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"layers 0-{nl - 1} of the first timed decode step (T={T}), float64 NumPy oracle, "
                      f"{cores} host cores visible",
        }
        log(json.dumps(result["cpu_baseline"]))

    line = {
        "metric": METRIC, "value": value, "unit": "MoE-layer tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": elapsed / K * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"decode, {L} MoE layers, E={E} top-{k}, H={H}, I={I}, bf16 experts, T={T} tokens "
                               f"per step, Zipf(1.1) router bias, 0.7 row reuse, every expert resident in HBM",
                   "global_batch": T, "layers": L, "parallelism": "single GPU"},
    }
    line.update(result)
    print(json.dumps(line), flush=True)
    pool.free()


if __name__ == "__main__":
    main()
