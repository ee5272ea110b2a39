"""Shared set-up for the GPU parity tests: seeded inputs from synth, the
library context, and the oracle on the same bytes."""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import synth
from oracle import moe as M

TOL = {0: 1e-2, 1: 3e-2, 2: 5e-2, 3: 1e-2}   # max|diff| / max|ref| per weight format
MARGIN = 1e-4                         # tokens closer to a top-k tie are excluded


def shape(base=1, **kw):
    return dataclasses.replace(synth.CONFIGS[base], **kw)


class Setup:
    """Host pool filled from synth, a runtime, and per-layer router tensors."""

    def __init__(self, cfg, seed=0, n_slots=None, max_tokens=64, host_threads=4, pool=None):
        from expert_ffn_execution_router_amd.runtime import HostPool, MoeRuntime
        self.cfg, self.seed = cfg, seed
        S = cfg.expert_bytes
        if pool is None:
            pool = HostPool(cfg.L * cfg.E * S)
            synth.fill_pool(pool.ptr, cfg, seed)
        self.pool = pool
        self.pool_np = pool.array().reshape(cfg.L * cfg.E, S)
        n_slots = cfg.L * cfg.E if n_slots is None else n_slots
        self.rt = MoeRuntime(cfg.L, cfg.E, cfg.k, cfg.H, cfg.I, cfg.fmt, n_slots, max_tokens, pool,
                             host_threads=host_threads)
        self.R = [synth.router_weights(cfg, seed, l) for l in range(cfg.L)]
        self.b = [synth.router_bias(cfg, seed, l) for l in range(cfg.L)]
        self.R_d = [torch.from_numpy(r).cuda() for r in self.R]
        self.b_d = [None if b is None else torch.from_numpy(b).cuda() for b in self.b]
        self._w = {}
        self.act = None

    def set_act(self, act):
        """MXFP4 activation variant: None (MXFP8) or "mxfp6" (large-batch GEMMs)."""
        from expert_ffn_execution_router_amd import binding as B
        self.rt.set_activations(B.MOE_ACT_MXFP6 if act == "mxfp6" else B.MOE_ACT_DEFAULT)
        self.act = act

    def tiled(self, T):
        """Whether a forward of T tokens runs the large-batch GEMMs."""
        c = self.cfg
        return T > 64 and T * c.k >= 48 * c.E

    def weights(self, layer):
        def get(e):
            key = (layer, e)
            if key not in self._w:
                self._w[key] = M.dequant_expert(self.pool_np[layer * self.cfg.E + e], self.cfg.fmt, self.cfg.H,
                                                self.cfg.I)
            return self._w[key]
        return get

    def hidden(self, T, tag=0):
        x = synth.hidden(self.cfg, self.seed, T, tag)
        return x, torch.from_numpy(x.view(np.int16)).cuda()

    def act_of(self, T):
        """Activation rule of a call of T tokens: the large-batch kernels
        quantise fp8 / MXFP4 activations (E4M3 per 128, MXFP8, or MXFP6 when
        selected); the small-batch kernels take bf16 activations."""
        if self.tiled(T):
            return self.act
        return "bf16" if self.cfg.fmt in (1, 2) else None

    def oracle(self, layer, x_bits, mode="mirrored", rows=None, T=None):
        """T: tokens of the GPU call (default len(x_bits)), which decides the
        activation rule (act_of)."""
        xs = x_bits if rows is None else x_bits[rows]
        T = len(x_bits) if T is None else T
        act = self.act_of(T)
        return M.moe_layer(xs, self.R[layer], self.b[layer], self.cfg.k, self.weights(layer), fmt=self.cfg.fmt,
                           mode=mode, act=act)

    def admit_all(self, layer):
        self.rt.admit(layer, list(range(self.cfg.E)))
        torch.cuda.synchronize()

    def slot_row(self, layer):
        E = self.cfg.E
        return self.rt.slot_table()[layer * E:(layer + 1) * E]

    def close(self):
        self.rt.close()


def bf16_to_np(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def rel_err(got, ref, rows=None):
    if rows is not None:
        got, ref = got[rows], ref[rows]
    denom = np.abs(ref).max()
    return float(np.abs(got - ref).max() / denom) if denom > 0 else float(np.abs(got).max())


def exact_bound(setup, T, e_q, tol):
    """Bound on the error against the exact layer: the tolerance itself
    wherever the activations stay 16-bit; with quantised activations (the
    large-batch fp8 / MXFP4 kernels) the quantisation's own cost e_q (the
    mirrored oracle's distance from the exact one, fp64, same inputs) plus
    the tolerance."""
    act = setup.act_of(T)
    sixteen = act == "bf16" or (act is None and setup.cfg.fmt in (0, 3))
    return tol if sixteen else e_q + tol


def compare(setup, layer, x_bits, out_t, tol=None):
    """Checks a GPU layer output against the mirrored oracle and the exact
    oracle on tokens whose top-k margin is >= MARGIN; returns (err_mirrored,
    err_exact, n_rows)."""
    ref = setup.oracle(layer, x_bits, "mirrored")
    ex = setup.oracle(layer, x_bits, "exact")
    rows = np.nonzero(ref["margin"] >= MARGIN)[0]
    got = bf16_to_np(out_t)
    e_m = rel_err(got, ref["out"], rows)
    e_x = rel_err(got, ex["out"], rows)
    t = TOL[setup.cfg.fmt] if tol is None else tol
    assert e_m <= t, (e_m, e_x, len(rows))
    e_q = rel_err(ref["out"], ex["out"], rows)
    assert e_x <= exact_bound(setup, len(x_bits), e_q, t), (e_m, e_x, e_q, len(rows))
    return e_m, e_x, len(rows)
