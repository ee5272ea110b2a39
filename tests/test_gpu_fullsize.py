"""Parity at the workloads' full per-layer sizes, in the launch configurations
the bench times.  Each token's output depends only on its own routing, so the
oracle computes a subset of rows exactly; the subset is chosen to cover the
whole launch: in every expert's grouped rows, one row at every multiple of 64
and the last row (every m-tile of every tiled or small-batch item holds at
least 64 rows or ends an expert, and an expert's overflow rows are its last
ones), moved forward to the next row whose token is away from a top-k tie.
Checked against the mirrored oracle (the path's tolerance) and the exact one
(the same tolerance with 16-bit activations; plus the quantisation's own cost
with 8-bit ones)."""
import numpy as np
import pytest
import torch

import synth
from oracle import moe as M
from gpu_util import MARGIN, TOL, Setup, bf16_to_np, exact_bound, rel_err

pytestmark = pytest.mark.gpu


def covering_rows(s, layer, x, stride=64):
    """Tokens covering every `stride`-row block (and the last row) of every
    expert's grouped rows, among tokens whose top-k margin is >= MARGIN."""
    z = M.router_logits(x, s.R[layer], s.b[layer])
    k, E = s.cfg.k, s.cfg.E
    margin = M.topk_margin(z, k)
    ok = margin >= MARGIN
    # top-k by argpartition then a stable order (ties are excluded by the margin)
    part = np.argpartition(-z, k - 1, axis=1)[:, :k]
    tok = np.repeat(np.arange(len(x)), k)
    ex = part.reshape(-1)
    order = np.lexsort((tok, ex))                  # grouped order: expert, then token
    tok_g, ex_g = tok[order], ex[order]
    counts = np.bincount(ex_g, minlength=E)
    offs = np.concatenate([[0], np.cumsum(counts)])
    rows = set()
    for e in range(E):
        c = counts[e]
        for r0 in list(range(0, c, stride)) + ([c - 1] if c else []):
            for r in range(r0, min(r0 + stride, c)):   # first usable row of the block
                t = tok_g[offs[e] + r]
                if ok[t]:
                    rows.add(int(t))
                    break
    return np.array(sorted(rows)), counts


def _check_rows(s, layer, x, out_t, stride=64):
    rows, counts = covering_rows(s, layer, x, stride)
    cfg = s.cfg

    def wf(e):   # no caching: one expert's float64 weights at a time
        return M.dequant_expert(s.pool_np[layer * cfg.E + e], cfg.fmt, cfg.H, cfg.I)
    T = len(x)
    ref = M.moe_layer(x[rows], s.R[layer], s.b[layer], cfg.k, wf, fmt=cfg.fmt, mode="both", act=s.act_of(T))
    got = bf16_to_np(out_t)[rows]
    e_m = rel_err(got, ref["out"])
    e_x = rel_err(got, ref["out_exact"])
    e_q = rel_err(ref["out"], ref["out_exact"])
    print(f"  {len(rows)} rows covering {int((counts > 0).sum())} experts: err vs mirrored {e_m:.2e}, "
          f"vs exact {e_x:.2e} (activation rule {s.act_of(T)}, its own cost {e_q:.2e})", flush=True)
    assert e_m <= TOL[cfg.fmt]
    assert e_x <= exact_bound(s, T, e_q, TOL[cfg.fmt])
    return rows


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
                _check_rows(s, layer, x, out)
        assert s.rt.check_device_error() == 0
    finally:
        s.close()


@pytest.mark.parametrize("T", [1, 3, 4, 8, 16])
def test_decode_config2_shape_small_T(T):
    """The decode shape at the smallest batches (up to 8 tokens: the
    matrix-vector kernels; 16: the MFMA kernel), every item covered."""
    print(f"decode config-2 shape T={T}", flush=True)
    cfg = _fullsize(2, L=1)
    s = Setup(cfg, seed=5, max_tokens=64, host_threads=8)
    try:
        s.admit_all(0)
        keys = synth.decode_row_keys(cfg, 5, 1, T)
        x = synth.hidden_rows(cfg, keys[0, 0])
        xd = torch.from_numpy(x.view(np.int16)).cuda()
        out = torch.empty(T, cfg.H, dtype=torch.bfloat16, device="cuda")
        s.rt.forward(0, xd, s.R_d[0], s.b_d[0], s.slot_row(0), out)
        torch.cuda.synchronize()
        assert s.rt.check_device_error() == 0
        _check_rows(s, 0, x, out)
    finally:
        s.close()


@pytest.mark.timeout(400)
@pytest.mark.parametrize("T", [2048, 4096, 8192, 16384])
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
            _check_rows(s, layer, xs[layer], outs[layer])
    finally:
        s.close()


@pytest.mark.timeout(400)
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
        _check_rows(s, 0, x, out)
    finally:
        s.close()


@pytest.mark.timeout(400)
@pytest.mark.parametrize("T", [1, 16, 2048, 16384])
def test_mxfp4_config5_shape(T):
    print(f"mxfp4 config-5 shape T={T}", flush=True)
    cfg = _fullsize(5, L=1)
    s = Setup(cfg, seed=3, max_tokens=max(T, 64), host_threads=8)
    try:
        s.admit_all(0)
        if T >= 2048:
            assert s.tiled(T)          # MXFP8 activations; 288-token tiles at 16384 (T*k > 160*E)
        x, xd = s.hidden(T, tag=T)
        out = torch.empty(T, cfg.H, dtype=torch.bfloat16, device="cuda")
        s.rt.forward(0, xd, s.R_d[0], s.b_d[0], s.slot_row(0), out)
        torch.cuda.synchronize()
        assert s.rt.check_device_error() == 0
        _check_rows(s, 0, x, out)
    finally:
        s.close()


@pytest.mark.timeout(400)
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
        _check_rows(s, 0, x, out)
    finally:
        s.close()


@pytest.mark.timeout(400)
@pytest.mark.parametrize("T", [1, 64, 1024, 8192])
def test_nvfp4_decode_shape(T):
    """The decode shape with NVFP4 experts at the sizes the formats bench
    times (T=1 and 64 through the weight stream, 8192 through the tiled
    kernel) and a batch of 1024 (tiled, ~64 rows per expert)."""
    import dataclasses
    print(f"nvfp4 decode shape T={T}", flush=True)
    cfg = dataclasses.replace(_fullsize(2, L=1), fmt=synth.FMT_NVFP4)
    s = Setup(cfg, seed=4, max_tokens=max(T, 64), host_threads=8)
    try:
        s.admit_all(0)
        assert s.tiled(T) == (T >= 1024)
        x, xd = s.hidden(T, tag=T)
        out = torch.empty(T, cfg.H, dtype=torch.bfloat16, device="cuda")
        s.rt.forward(0, xd, s.R_d[0], s.b_d[0], s.slot_row(0), out)
        torch.cuda.synchronize()
        assert s.rt.check_device_error() == 0
        _check_rows(s, 0, x, out)
    finally:
        s.close()
