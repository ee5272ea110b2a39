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


def test_bf16_decode_exact():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x4049], dtype=np.uint16)
    v = F.bf16_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 0.0 and v[3] == 3.140625
