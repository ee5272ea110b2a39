"""CPU tests of the C-ABI library: it loads, exports every call of
include/moe.h, sizes buffers as documented, and its host FFN path (the host
branch of the miss split) matches the oracle.  No GPU call is made."""
import ctypes
import dataclasses
import os
import re

import numpy as np
import pytest

import synth
from oracle import moe as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def B():
    from expert_ffn_execution_router_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from expert_ffn_execution_router_amd.build import build
        build()
    return binding


def _header_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\(", text, flags=re.M)
    return [n for n in names if n not in ("if", "while")]


def test_every_header_call_is_exported(B):
    names = _header_functions()
    assert len(names) >= 20
    L = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
        assert n in B.SIGNATURES, n
    assert set(B.SIGNATURES) == set(names)


def test_sizes(B):
    for c in synth.CONFIGS.values():
        cfg = B.make_config(c.L, c.E, c.k, c.H, c.I, c.fmt, min(c.n_slots, 8192), 64)
        assert B.moe_expert_bytes(ctypes.byref(cfg)) == c.expert_bytes
        assert B.moe_workspace_bytes(ctypes.byref(cfg)) > 0
    bad = B.make_config(1, 300, 2, 256, 128, 0, 8, 16)
    assert B.moe_workspace_bytes(ctypes.byref(bad)) == 0
    assert "E <= 256" in B.last_error()


def _run_host(B, cfg_s, seed, T, C, threads):
    pool = synth.pool_array(cfg_s, seed)
    x = synth.hidden(cfg_s, seed, T)
    R = synth.router_weights(cfg_s, seed, 0)
    z = M.router_logits(x, R, None)
    ids = M.select_topk(z, cfg_s.k)
    w = M.gate_weights(z, ids).astype(np.float32)
    mask = np.zeros(8, dtype=np.uint32)
    for e in C:
        mask[e >> 5] |= np.uint32(1 << (e & 31))
    out = np.zeros((T, cfg_s.H), dtype=np.float32)
    cfg = B.make_config(cfg_s.L, cfg_s.E, cfg_s.k, cfg_s.H, cfg_s.I, cfg_s.fmt, 0, T, threads)
    rc = B.moe_host_ffn(ctypes.byref(cfg), pool.ctypes.data, 0, x.ctypes.data, ids.astype(np.int32).ctypes.data,
                        w.ctypes.data, T, mask.ctypes.data, out.ctypes.data)
    assert rc == 0, B.last_error()

    def wf(e):
        return M.dequant_expert(pool[e], cfg_s.fmt, cfg_s.H, cfg_s.I)
    ref = M.host_partial(x, ids, w.astype(np.float64), C, wf)
    return out, ref


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
@pytest.mark.parametrize("threads,T", [(1, 16), (3, 16), (5, 48)])
def test_host_ffn_matches_oracle(B, fmt, threads, T):
    """T=48 gives each host expert more than 8 tokens (several row passes)."""
    c = synth.CONFIGS[1]
    if fmt:
        c = dataclasses.replace(c, fmt=fmt, H=256, I=256)
    else:
        c = dataclasses.replace(c, fmt=fmt)
    out, ref = _run_host(B, c, 7, T, [0, 2, 3, 5], threads)
    err = np.abs(out - ref).max() / np.abs(ref).max()
    assert err < 1e-5, err
    # tokens with no host expert get exactly zero
    assert np.count_nonzero(np.abs(ref).sum(1) == 0) == np.count_nonzero(np.abs(out).sum(1) == 0)


def test_host_ffn_empty_set_is_zero(B):
    c = synth.CONFIGS[1]
    out, ref = _run_host(B, c, 8, 5, [], 2)
    assert not out.any() and not ref.any()


def test_noalloc_forward_rejects_before_device_work(B):
    """The allocation-free forward's limits are checked on the host before
    any HIP call (so this runs without a GPU, and never launches a kernel):
    T above 64, a shape whose forward buffers exceed its static scratch, a
    bad shape, a missing argument."""
    buf = (ctypes.c_uint8 * 64)()
    p = ctypes.addressof(buf)
    cfg = B.make_config(1, 8, 2, 256, 128, 0, 0, 64)
    assert B.moe_layer_forward_noalloc(ctypes.byref(cfg), p, p, p, p, None, 65, None, None, p, None, None) \
        == B.MOE_E_UNSUPPORTED
    # Z alone would take 513 rows * 65536 * 2 bytes = 67 MB of the 40 MiB
    huge = B.make_config(1, 256, 8, 65536, 8192, 0, 0, 64)
    assert B.moe_layer_forward_noalloc(ctypes.byref(huge), p, p, p, p, None, 16, None, None, p, None, None) \
        == B.MOE_E_UNSUPPORTED
    assert "scratch" in B.last_error()
    bad = B.make_config(1, 8, 2, 100, 128, 0, 0, 64)
    assert B.moe_layer_forward_noalloc(ctypes.byref(bad), p, p, p, p, None, 16, None, None, p, None, None) \
        == B.MOE_E_INVAL
    assert B.moe_layer_forward_noalloc(None, p, p, p, p, None, 16, None, None, p, None, None) == B.MOE_E_INVAL
    assert B.moe_layer_forward_noalloc(ctypes.byref(cfg), p, None, p, p, None, 16, None, None, p, None, None) \
        == B.MOE_E_INVAL
    assert B.moe_layer_forward_noalloc(ctypes.byref(cfg), p, p, p, p, None, 0, None, None, p, None, None) == 0
