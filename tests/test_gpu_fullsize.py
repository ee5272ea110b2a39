"""Parity at the workloads' full per-layer sizes, in the launch configurations
the bench times, on sampled tokens the oracle computes one by one (each
token's output depends only on its own routing, so a subset of rows is an
exact check of those rows)."""
import numpy as np
import pytest
import torch

import synth
from oracle import moe as M
from gpu_util import MARGIN, TOL, Setup, bf16_to_np, rel_err

pytestmark = pytest.mark.gpu


def _check_rows(s, layer, x, out_t, n_sample, seed):
    z = M.router_logits(x, s.R[layer], s.b[layer])
    margin = M.topk_margin(z, s.cfg.k)
    cand = np.nonzero(margin >= MARGIN)[0]
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(cand, size=min(n_sample, len(cand)), replace=False))
    cfg = s.cfg

    def wf(e):   # no caching: one expert's float64 weights at a time
        return M.dequant_expert(s.pool_np[layer * cfg.E + e], cfg.fmt, cfg.H, cfg.I)
    act = s.act if s.tiled(len(x)) else None
    ref = M.moe_layer(x[rows], s.R[layer], s.b[layer], cfg.k, wf, fmt=cfg.fmt, mode="mirrored", act=act)
    got = bf16_to_np(out_t)[rows]
    err = rel_err(got, ref["out"])
    print(f"  sampled rows {list(rows)} err vs mirrored {err:.2e}")
    assert err <= TOL[cfg.fmt]


def _fullsize(cfg_id, L=1):
    return synth.CONFIGS[cfg_id].with_layers(L)


def test_decode_config2_shape_T64():
    """48-layer decode shape (one layer here), T=64 with the locality model's rows."""
    print("decode config-2 shape", flush=True)
    cfg = _fullsize(2, L=2)
    s = Setup(cfg, seed=0, max_tokens=64, host_threads=8)
    try:
        for layer in range(cfg.L):
            s.admit_all(layer)
        keys = synth.decode_row_keys(cfg, 0, 2, 64)
        for step in range(2):
            for layer in range(cfg.L):
                x = synth.hidden_rows(cfg, keys[step, layer])
                xd = torch.from_numpy(x.view(np.int16)).cuda()
                out = torch.empty(64, cfg.H, dtype=torch.bfloat16, device="cuda")
                s.rt.forward(layer, xd, s.R_d[layer], s.b_d[layer], s.slot_row(layer), out)
                torch.cuda.synchronize()
                _check_rows(s, layer, x, out, 6, step * 10 + layer)
        assert s.rt.check_device_error() == 0
    finally:
        s.close()


@pytest.mark.parametrize("T", [2048, 8192])
def test_prefill_config3_shape(T):
    """Prefill shape through the full-layer double buffer, T tokens, tiled GEMMs."""
    print(f"prefill config-3 shape T={T}", flush=True)
    cfg = _fullsize(3, L=2)
    s = Setup(cfg, seed=1, n_slots=2 * cfg.E, max_tokens=T, host_threads=8)
    try:
        comp, copy = torch.cuda.Stream(), torch.cuda.Stream()
        xs, outs = [], []
        with torch.cuda.stream(comp):
            for layer in range(cfg.L):
                x, xd = s.hidden(T, tag=layer)
                out = torch.empty(T, cfg.H, dtype=torch.bfloat16, device="cuda")
                assert s.rt.prefill_layer(layer, xd, s.R_d[layer], s.b_d[layer], out, stream=comp,
                                          copy_stream=copy) == 0
                xs.append(x)
                outs.append(out)
        torch.cuda.synchronize()
        assert s.rt.check_device_error() == 0
        for layer in range(cfg.L):
            _check_rows(s, layer, xs[layer], outs[layer], 6, layer)
    finally:
        s.close()


@pytest.mark.parametrize("T", [1, 32, 512, 4096])
def test_fp8_config4_shape(T):
    print(f"fp8 config-4 shape T={T}", flush=True)
    cfg = _fullsize(4, L=1)
    s = Setup(cfg, seed=2, max_tokens=max(T, 64), host_threads=8)
    try:
        s.admit_all(0)
        x, xd = s.hidden(T, tag=T)
        out = torch.empty(T, cfg.H, dtype=torch.bfloat16, device="cuda")
        s.rt.forward(0, xd, s.R_d[0], s.b_d[0], s.slot_row(0), out)
        torch.cuda.synchronize()
        assert s.rt.check_device_error() == 0
        _check_rows(s, 0, x, out, 4, T)
    finally:
        s.close()


@pytest.mark.parametrize("T", [1, 16, 2048])
def test_mxfp4_config5_shape(T):
    print(f"mxfp4 config-5 shape T={T}", flush=True)
    cfg = _fullsize(5, L=1)
    s = Setup(cfg, seed=3, max_tokens=max(T, 64), host_threads=8)
    try:
        s.admit_all(0)
        x, xd = s.hidden(T, tag=T)
        out = torch.empty(T, cfg.H, dtype=torch.bfloat16, device="cuda")
        s.rt.forward(0, xd, s.R_d[0], s.b_d[0], s.slot_row(0), out)
        torch.cuda.synchronize()
        assert s.rt.check_device_error() == 0
        _check_rows(s, 0, x, out, 3, T)
    finally:
        s.close()


@pytest.mark.parametrize("T", [2048, 16384])
def test_mxfp4_config5_shape_mxfp6(T):
    """MXFP6 activations on the MXFP4 shape, up to the prefill chunk the bench
    times (16384 tokens, ~512 rows per expert)."""
    print(f"mxfp4 config-5 shape, MXFP6 activations, T={T}", flush=True)
    cfg = _fullsize(5, L=1)
    s = Setup(cfg, seed=3, max_tokens=T, host_threads=8)
    try:
        s.admit_all(0)
        s.set_act("mxfp6")
        x, xd = s.hidden(T, tag=T + 1)
        out = torch.empty(T, cfg.H, dtype=torch.bfloat16, device="cuda")
        s.rt.forward(0, xd, s.R_d[0], s.b_d[0], s.slot_row(0), out)
        torch.cuda.synchronize()
        assert s.rt.check_device_error() == 0
        _check_rows(s, 0, x, out, 3, T)
    finally:
        s.close()


@pytest.mark.parametrize("T", [1, 64, 1024])
def test_nvfp4_decode_shape(T):
    """The decode shape with NVFP4 experts at the sizes the formats bench
    times (T=1 and 64) and a large batch through the same weight stream."""
    import dataclasses
    print(f"nvfp4 decode shape T={T}", flush=True)
    cfg = dataclasses.replace(_fullsize(2, L=1), fmt=synth.FMT_NVFP4)
    s = Setup(cfg, seed=4, max_tokens=max(T, 64), host_threads=8)
    try:
        s.admit_all(0)
        x, xd = s.hidden(T, tag=T)
        out = torch.empty(T, cfg.H, dtype=torch.bfloat16, device="cuda")
        s.rt.forward(0, xd, s.R_d[0], s.b_d[0], s.slot_row(0), out)
        torch.cuda.synchronize()
        assert s.rt.check_device_error() == 0
        _check_rows(s, 0, x, out, 6, T)
    finally:
        s.close()
