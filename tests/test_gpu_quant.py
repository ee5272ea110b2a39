"""GPU activation quantisation (the 8-bit paths' GEMM inputs) through the
C-ABI test hook, bit-exact against the oracle's mirrored quantisers: the
dequantised values code * scale are compared for equality, and the fp8 scales
themselves."""
import ctypes

import numpy as np
import pytest
import torch

from expert_ffn_execution_router_amd import binding as B
from oracle import formats as F
from oracle import moe as M

pytestmark = pytest.mark.gpu


def _inputs(rows_src, cols, seed):
    rng = np.random.default_rng(seed)
    mag = 10.0 ** rng.uniform(-6, 6, size=(rows_src, 1))          # per-row magnitude
    v = (rng.standard_normal((rows_src, cols)) * mag).astype(np.float32)
    v[3] = 0.0                                                     # an all-zero row
    v[5, :128] = 0.0                                               # zero groups
    v[7, 32:64] = 0.0
    v[9] *= np.float32(1e30)                                       # huge and tiny groups
    v[11] *= np.float32(1e-25)
    v[13, 5] = np.float32(-3.0e38)                                 # near the fp32 limit
    return v


@pytest.mark.parametrize("wfmt", [1, 2])
@pytest.mark.parametrize("src_bf16", [True, False])
def test_quantize_matches_oracle_bit_exact(wfmt, src_bf16):
    rows_src, rows, cols = 40, 57, 768
    v = _inputs(rows_src, cols, seed=wfmt * 10 + int(src_bf16))
    if src_bf16:
        bits = F.round_to_bf16(v.astype(np.float64))
        bits = (bits.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        src_vals = F.bf16_to_f64(bits)
        src_t = torch.from_numpy(bits.view(np.int16)).cuda()
    else:
        src_vals = v.astype(np.float64)
        src_t = torch.from_numpy(v).cuda()
    rng = np.random.default_rng(99)
    row_map = rng.integers(0, rows_src, size=rows).astype(np.int32)   # repeats allowed
    row_map[:rows_src] = np.arange(rows_src)                          # every source row at least once
    rm_t = torch.from_numpy(row_map).cuda()
    q_t = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
    if wfmt == 1:
        sc_t = torch.empty(rows, cols // 128, dtype=torch.float32, device="cuda")
    else:
        sc_t = torch.empty(rows, cols // 32, dtype=torch.uint8, device="cuda")
    rc = B.moe_quantize(wfmt, int(src_bf16), src_t.data_ptr(), rows, cols, rm_t.data_ptr(), q_t.data_ptr(),
                        sc_t.data_ptr(), None)
    assert rc == 0
    torch.cuda.synchronize()
    q = q_t.cpu().numpy()
    sc = sc_t.cpu().numpy()
    x = src_vals[row_map]
    codes = F.decode_e4m3(q)
    if wfmt == 1:
        got = codes * np.repeat(sc.astype(np.float64), 128, axis=1)
        want = M.mirror_quant_fp8_groups(x, 128)
        g = x.astype(np.float32).reshape(rows, cols // 128, 128)
        amax = np.abs(g).max(axis=2)
        want_sc = np.where(amax > 0, (amax / np.float32(448.0)).astype(np.float32), np.float32(1.0))
        assert np.array_equal(sc, want_sc)
    else:
        got = codes * np.repeat(np.ldexp(1.0, sc.astype(np.int64) - 127), 32, axis=1)
        want = M.mirror_quant_mxfp8(x)
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]


def test_quantize_rejects_bad_shapes():
    assert B.moe_quantize(0, 1, None, 4, 128, None, None, None, None) != 0      # bf16 has no quantisation
    assert B.moe_quantize(1, 1, None, 4, 96, None, None, None, None) != 0       # fp8 needs cols % 128
    assert B.moe_quantize(2, 1, None, 4, 48, None, None, None, None) != 0       # mx needs cols % 32
    assert B.moe_quantize(2, 1, None, 0, 64, None, None, None, None) == 0       # nothing to do
