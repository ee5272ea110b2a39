"""The allocation-free forward (moe_layer_forward_noalloc: static device
scratch, no context) against moe_layer_forward on the same inputs: two calls
in a row, the second with fewer tokens, for every weight format; the same
kernels run on the same grid, so the outputs are bit-identical.  Also its
error flag.  (Its limits, which it checks before any device work, are tested
on the CPU.)"""
import ctypes

import numpy as np
import pytest
import torch

from expert_ffn_execution_router_amd import binding as B
from gpu_util import Setup, shape

pytestmark = pytest.mark.gpu


def _noalloc(s, layer, x, T, out, err=None, stream=None):
    cfg = B.make_config(s.cfg.L, s.cfg.E, s.cfg.k, s.cfg.H, s.cfg.I, s.cfg.fmt, 0, 64, 0)
    st = torch.cuda.current_stream() if stream is None else stream
    return B.moe_layer_forward_noalloc(ctypes.byref(cfg), s.rt.slots.data_ptr(), s.slot_row(layer).data_ptr(),
                                       x.data_ptr(), s.R_d[layer].data_ptr(),
                                       None if s.b_d[layer] is None else s.b_d[layer].data_ptr(), T, None, None,
                                       out.data_ptr(), None if err is None else err.data_ptr(), st.cuda_stream)


@pytest.mark.parametrize("fmt,base,kw", [(0, 1, {}), (1, 1, {}), (2, 1, {}), (3, 1, {}),
                                         (0, 2, dict(L=1))])
def test_noalloc_matches_forward(fmt, base, kw):
    print(f"noalloc fmt={fmt} base={base}", flush=True)
    cfg = shape(base, fmt=fmt, **kw)
    s = Setup(cfg, seed=11, max_tokens=64)
    try:
        s.admit_all(0)
        # calls in a row, each smaller (the last ones through the
        # matrix-vector kernels)
        for T in (64, 23, 8, 3, 1):
            _, x = s.hidden(T, tag=T)
            ref = torch.empty(T, cfg.H, dtype=torch.bfloat16, device="cuda")
            got = torch.full((T, cfg.H), 7.0, dtype=torch.bfloat16, device="cuda")
            s.rt.forward(0, x, s.R_d[0], s.b_d[0], s.slot_row(0), ref)
            err = torch.zeros(1, dtype=torch.int32, device="cuda")
            assert _noalloc(s, 0, x, T, got, err) == 0, B.last_error()
            torch.cuda.synchronize()
            assert err.item() == 0
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), (T, (got.float() - ref.float()).abs().max())
        assert s.rt.check_device_error() == 0
    finally:
        s.close()


@pytest.mark.parametrize("T", [16, 4])
def test_noalloc_error_flag(T):
    """A routed expert without a slot (the test's own shape, its own slot
    pool): left out, bit 0 of the caller's flag set, the output zero."""
    print(f"noalloc error flag T={T}", flush=True)
    cfg = shape(1)
    s = Setup(cfg, seed=12, max_tokens=64)
    try:
        s.admit_all(0)
        _, x = s.hidden(T)
        out = torch.full((T, cfg.H), 3.0, dtype=torch.bfloat16, device="cuda")
        row = s.slot_row(0).clone()
        row[:] = -1
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        cfgc = B.make_config(cfg.L, cfg.E, cfg.k, cfg.H, cfg.I, cfg.fmt, 0, 64, 0)
        rc = B.moe_layer_forward_noalloc(ctypes.byref(cfgc), s.rt.slots.data_ptr(), row.data_ptr(), x.data_ptr(),
                                         s.R_d[0].data_ptr(), None, T, None, None, out.data_ptr(), err.data_ptr(),
                                         torch.cuda.current_stream().cuda_stream)
        assert rc == 0
        torch.cuda.synchronize()
        assert err.item() & 1
        assert float(out.float().abs().max()) == 0.0      # nothing routed ran: the combine wrote zeros
    finally:
        s.close()
