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


def _x6_plane(rows):
    return (rows * 112 + 1024 + 255) // 256 * 256


def _x6_codes(planes, rows, cols):
    """E2M3 codes [rows, cols] from the MXFP6 plane layout of the test hook:
    112-byte rows, group g's 24-byte code string split into its first 16
    bytes at 24g + 8*(g odd) and its last 8 at 24g + 16*(g even)."""
    q = planes.reshape(cols // 128, _x6_plane(rows))[:, :rows * 112].reshape(cols // 128, rows, 112)
    codes = np.empty((rows, cols), dtype=np.uint8)
    for c in range(cols // 128):
        for g in range(4):
            o16 = 24 * g + 8 * (g & 1)
            o8 = 24 * g + (0 if g & 1 else 16)
            b = np.concatenate([q[c, :, o16:o16 + 16], q[c, :, o8:o8 + 8]], axis=1)        # [rows, 24]
            bits = np.unpackbits(b, axis=1, bitorder="little")                            # [rows, 192]
            six = bits.reshape(rows, 32, 6).astype(np.int64)
            codes[:, 128 * c + 32 * g:128 * c + 32 * g + 32] = (six * (1 << np.arange(6))).sum(axis=2)
    return codes


@pytest.mark.parametrize("src_bf16", [True, False])
def test_quantize_mxfp6_matches_oracle_bit_exact(src_bf16):
    rows_src, rows, cols = 40, 57, 768
    v = _inputs(rows_src, cols, seed=30 + int(src_bf16))
    if src_bf16:
        bits = F.round_to_bf16(v.astype(np.float64))
        bits = (bits.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        src_vals = F.bf16_to_f64(bits)
        src_t = torch.from_numpy(bits.view(np.int16)).cuda()
    else:
        src_vals = v.astype(np.float64)
        src_t = torch.from_numpy(v).cuda()
    rng = np.random.default_rng(98)
    row_map = rng.integers(0, rows_src, size=rows).astype(np.int32)
    row_map[:rows_src] = np.arange(rows_src)
    rm_t = torch.from_numpy(row_map).cuda()
    q_t = torch.full((cols // 128 * _x6_plane(rows),), 0xAB, dtype=torch.uint8, device="cuda")
    sc_t = torch.empty(cols // 128, rows, 4, dtype=torch.uint8, device="cuda")
    rc = B.moe_quantize(B.MOE_QUANT_MXFP6, int(src_bf16), src_t.data_ptr(), rows, cols, rm_t.data_ptr(),
                        q_t.data_ptr(), sc_t.data_ptr(), None)
    assert rc == 0
    torch.cuda.synchronize()
    codes = _x6_codes(q_t.cpu().numpy(), rows, cols)
    sc = sc_t.cpu().numpy().transpose(1, 0, 2).reshape(rows, cols // 32)     # chunk-major planes
    got = F.decode_e2m3(codes) * np.repeat(np.ldexp(1.0, sc.astype(np.int64) - 127), 32, axis=1)
    want = M.mirror_quant_mxfp6(src_vals[row_map])
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]
    # the codes themselves: the sign bit only on non-zero codes
    assert not ((codes == 0x20).any())


def test_quantize_rejects_bad_shapes():
    assert B.moe_quantize(0, 1, None, 4, 128, None, None, None, None) != 0      # bf16 has no quantisation
    assert B.moe_quantize(1, 1, None, 4, 96, None, None, None, None) != 0       # fp8 needs cols % 128
    assert B.moe_quantize(2, 1, None, 4, 48, None, None, None, None) != 0       # mx needs cols % 32
    assert B.moe_quantize(2, 1, None, 0, 64, None, None, None, None) == 0       # nothing to do
    assert B.moe_quantize(B.MOE_QUANT_MXFP6, 1, None, 4, 96, None, None, None, None) != 0   # mxfp6: cols % 128
    assert B.moe_quantize(3, 1, None, 4, 128, None, None, None, None) != 0      # nvfp4 keeps bf16 activations
