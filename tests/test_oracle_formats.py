"""Pins of oracle.formats against the format definitions and torch's own
converters (an independent implementation of the same standards)."""
import math

import numpy as np
import pytest
import torch

from oracle import formats as F


def test_e4m3_table_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = F.E4M3_TABLE
    nan_ref, nan_ours = np.isnan(ref), np.isnan(ours)
    assert (nan_ref == nan_ours).all()
    assert np.array_equal(ref[~nan_ref], ours[~nan_ours])
    assert nan_ours.sum() == 2          # S.1111.111 for both signs


@pytest.mark.parametrize("code,val", [(0x7E, 448.0), (0x01, 2.0 ** -9), (0x08, 2.0 ** -6), (0x38, 1.0),
                                      (0x07, 7 * 2.0 ** -9), (0x3C, 1.5), (0xB8, -1.0), (0xFE, -448.0)])
def test_e4m3_hand_values(code, val):
    assert F.E4M3_TABLE[code] == val


def test_e4m3_negative_zero_and_nan():
    assert F.E4M3_TABLE[0x80] == 0.0 and math.copysign(1.0, F.E4M3_TABLE[0x80]) == -1.0
    assert math.isnan(F.E4M3_TABLE[0x7F]) and math.isnan(F.E4M3_TABLE[0xFF])


def test_e4m3_encoder_matches_torch_in_range():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.normal(0, 50, 20000), rng.normal(0, 0.01, 5000),
                        rng.uniform(-448, 448, 5000)]).astype(np.float32)
    # exact midpoints between neighbouring codes (ties) too
    pos = F.E4M3_TABLE[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = F.encode_e4m3(v.astype(np.float64))
    # torch keeps the sign of zero; so do we except -0 rounding from tiny negatives
    same = (ref == ours) | ((ref & 0x7F) == 0) & ((ours & 0x7F) == 0)
    assert same.all()


def test_e4m3_encoder_saturates():
    assert F.encode_e4m3(np.array([500.0, -1e9, 448.0]))[0] == 0x7E
    assert F.encode_e4m3(np.array([-1e9]))[0] == 0xFE


def test_e2m1_from_bit_fields():
    # OCP MX v1.0 E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit, no inf/nan
    for c in range(16):
        s = -1.0 if c & 8 else 1.0
        e = (c >> 1) & 3
        m = c & 1
        val = s * (m / 2.0) if e == 0 else s * 2.0 ** (e - 1) * (1 + m / 2.0)
        assert F.decode_e2m1(np.array([c]))[0] == val


def test_e2m3_values_pinned_by_e4m3():
    """E2M3 (OCP MX FP6) against what the standard fixes without retyping its
    formula: 64 finite codes (no inf/NaN), positive codes strictly increasing
    from 0 to the 7.5 maximum with 0.125 the smallest subnormal and 1.0 the
    smallest normal, negative codes the mirror image, and every value exactly
    an E4M3 value (3 mantissa bits, narrower exponent range; torch's table)."""
    t = F.E2M3_TABLE
    assert t.shape == (64,) and np.isfinite(t).all()
    pos = t[:32]
    assert (np.diff(pos) > 0).all()
    assert pos[0] == 0.0 and pos[1] == 0.125 and pos[8] == 1.0 and pos[31] == 7.5
    assert np.array_equal(t[32:], -pos)
    e4 = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.isin(pos, e4).all()
    # the step doubles with each binade: 1/8 below 2, 1/4 in [2, 4), 1/2 in [4, 7.5]
    assert set(np.diff(pos[:17])) == {0.125} and set(np.diff(pos[16:25])) == {0.25}
    assert set(np.diff(pos[24:])) == {0.5}


def test_e2m3_encoder_against_torch_grids():
    """Nearest-even rounding checked against torch: in [1, 7.5] E2M3 has E4M3's
    3-bit mantissa, so both round alike (E4M3 reaches 8 where E2M3 saturates);
    below 1 the step is 1/8, i.e. torch.round(8 v) / 8 (ties to even)."""
    rng = np.random.default_rng(3)
    hi = np.concatenate([rng.uniform(1.0, 7.75, 20000), (F.E2M3_TABLE[8:31] + F.E2M3_TABLE[9:32]) / 2])
    ref = torch.from_numpy(hi).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    ref = np.minimum(ref, 7.5)
    assert np.array_equal(F.decode_e2m3(F.encode_e2m3(hi)), ref)
    assert np.array_equal(F.decode_e2m3(F.encode_e2m3(-hi)), -ref)
    lo = np.concatenate([rng.uniform(0.0, 1.0, 20000), (np.arange(8) + 0.5) / 8])
    ref = torch.round(torch.from_numpy(lo) * 8).numpy() / 8
    assert np.array_equal(F.decode_e2m3(F.encode_e2m3(lo)), ref)
    big = np.array([7.5, 7.74, 7.76, 100.0, -1e9])
    assert list(F.encode_e2m3(big)) == [0x1F, 0x1F, 0x1F, 0x1F, 0x3F]


def test_e8m0():
    v = F.e8m0_to_f64(np.array([127, 0, 254, 128, 120, 255]))
    assert v[0] == 1.0 and v[1] == 2.0 ** -127 and v[2] == 2.0 ** 127 and v[3] == 2.0 and v[4] == 2.0 ** -7
    assert math.isnan(v[5])


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(1)
    f = rng.normal(0, 3, 50000).astype(np.float32)
    # force exact ties: low 16 bits = 0x8000
    ties = (f.view(np.uint32) & 0xFFFF0000) | 0x8000
    f = np.concatenate([f, ties.view(np.float32)])
    ref = torch.from_numpy(f).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(F.round_to_bf16(f.astype(np.float64)), ref)


def test_f16_round_matches_torch():
    rng = np.random.default_rng(4)
    v = np.concatenate([rng.normal(0, 1, 20000), rng.normal(0, 1e-5, 5000), rng.normal(0, 3e4, 5000),
                        np.array([65504.0, 65519.0, 65520.0, 1e6, -1e6, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 0.0])])
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float16).to(torch.float64).numpy()
    got = F.round_to_f16(v)
    assert np.array_equal(np.isinf(got), np.isinf(ref)) and np.array_equal(got[~np.isinf(got)], ref[~np.isinf(ref)])
    assert got[-6] == np.inf and got[-5] == -np.inf and got[-7] == np.inf and got[-8] == 65504.0
    assert got[-4] == 2.0 ** -24 and got[-3] == 0.0 and got[-2] == 2.0 ** -24     # ties to even at the bottom


def test_bf16_decode_exact():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x4049], dtype=np.uint16)
    v = F.bf16_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 0.0 and v[3] == 3.140625


def _nvfp4_blob(H, I, codes, scales, ts):
    """Blob bytes from per-matrix nibble arrays (row-major, element order),
    E4M3 scale codes [rows, cols/16] and the three tensor scales."""
    parts = []
    for c in codes:
        c = np.asarray(c, dtype=np.uint8).reshape(-1)
        parts.append((c[0::2] | (c[1::2] << 4)).astype(np.uint8))
    parts += [np.asarray(s, dtype=np.uint8).reshape(-1) for s in scales]
    parts.append(np.array(list(ts) + [0.0], dtype=np.float32).view(np.uint8))
    return np.concatenate(parts)


def test_nvfp4_layout_hand_values():
    """A hand-built NVFP4 expert (H=32, I=16): element codes, E4M3 block
    scales (1.0, 2.0, 0.5 and the subnormal 2^-9) and tensor scales with the
    values written out from the format's definition."""
    from oracle import moe as M
    H, I = 32, 16
    cg = np.zeros((I, H), np.uint8)
    cg[0, 0::2], cg[0, 1::2] = 0x2, 0xB                # 1.0, -1.5
    cg[3, :] = 0x7                                      # 6.0
    sg = np.full((I, H // 16), 0x38, np.uint8)          # 1.0
    sg[0, 1] = 0x40                                     # 2.0
    sg[3, 0] = 0x30                                     # 0.5
    cu = np.full((I, H), 0x1, np.uint8)                 # 0.5
    su = np.full((I, H // 16), 0x01, np.uint8)          # 2^-9
    cd = np.zeros((H, I), np.uint8)
    cd[5, 3] = 0xF                                      # -6.0
    sd = np.full((H, I // 16), 0x38, np.uint8)
    blob = _nvfp4_blob(H, I, [cg, cu, cd], [sg, su, sd], [0.5, 4.0, 0.25])
    assert blob.size == 3 * H * I // 2 + 3 * H * I // 16 + 16
    g, u, d = M.dequant_expert(blob, M.FMT_NVFP4, H, I)
    want0 = np.array([1.0, -1.5] * 8 + [2.0, -3.0] * 8) * 0.5
    assert np.array_equal(g[0], want0)
    assert np.array_equal(g[3], np.array([1.5] * 16 + [3.0] * 16))
    assert np.count_nonzero(g) == 2 * H
    assert np.all(u == 0.5 * 2.0 ** -9 * 4.0)
    assert d[5, 3] == -1.5 and np.count_nonzero(d) == 1


def test_nvfp4_synth_weights_track_their_draws():
    """The generator's NVFP4 blob, decoded by the oracle, stays within one
    E2M1 step (at most 1.07 x block amax / 6, the block scale rounded to E4M3)
    of the N(0, sigma) values it quantised, element by element."""
    import dataclasses
    import synth
    from oracle import moe as M
    cfg = dataclasses.replace(synth.CONFIGS[1], H=256, I=128, fmt=synth.FMT_NVFP4)
    blob = synth.expert_blob(cfg, 3, 0, 5)
    assert blob.size == cfg.expert_bytes
    g, u, d = M.dequant_expert(blob, cfg.fmt, cfg.H, cfg.I)
    k = synth.lib().synth_key(synth.pool_key(cfg, 3), 5)
    for j, (w, rows, cols) in enumerate(((g, 128, 256), (u, 128, 256), (d, 256, 128))):
        draw = synth.normal_f32(rows * cols, synth.lib().synth_key(k, j + 1), cfg.w_sigma).astype(np.float64)
        draw = draw.reshape(rows, cols)
        bmax = np.abs(draw.reshape(rows, cols // 16, 16)).max(axis=2)
        err = np.abs(w - draw).reshape(rows, cols // 16, 16).max(axis=2)
        assert np.all(err <= 1.07 * bmax / 6.0 + 1e-12)
        assert np.corrcoef(w.ravel(), draw.ravel())[0, 1] > 0.99
