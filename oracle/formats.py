"""Number formats of the stored expert weights, decoded exactly to float64.

TEST INFRASTRUCTURE ONLY: nothing on the product path imports this package.

The pages only name the formats the system serves (BF16, FP8, MXFP4; feature
table of "FreeToken – 边缘原生的 MoE 模型推理服务系统" and the model list in the
paper.oopus.info review, section 3).  The encodings below follow the public
format definitions, not the pages:
  * bfloat16: the upper 16 bits of an IEEE binary32;
  * OCP 8-bit floating point E4M3FN: bias 7, no infinities, S.1111.111 is NaN,
    max normal 448, subnormal step 2^-9;
  * OCP Microscaling v1.0: E2M1 elements (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 with
    a sign bit) and E8M0 scales 2^(e-127), 0xFF = NaN;
  * OCP Microscaling v1.0 FP6 E2M3 (activations of the MXFP6 variant): 1
    sign, 2 exponent bits with bias 1, 3 mantissa bits, no infinities or NaN,
    max 7.5, subnormal step 1/8;
  * NVFP4 (NVIDIA's 4-bit format, named on the same pages): the same E2M1
    elements, an E4M3 scale per 16 consecutive elements and one fp32 scale
    per tensor; value = element * block scale * tensor scale.

The encoders here serve the oracle's mirrored mode (the declared rounding
points of the GPU path): they pick the nearest representable value by
searching the decoded tables, ties to the code with an even last mantissa bit.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even), returned as float64.

    The value is first rounded to binary32 (the GPU holds it in fp32), then the
    16 low bits are rounded away with ties to even.
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    nan = np.isnan(f)
    out = r.astype(np.uint32).view(np.float32).astype(np.float64)
    out[nan] = np.nan
    return out


def round_to_f16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to IEEE binary16 (ties to even, overflow to
    infinity, subnormals kept), returned as float64.  Like round_to_bf16 the
    value passes through binary32 first (the GPU holds it in fp32)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float16).astype(np.float64)


def _e4m3_value(code: int) -> float:
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** (1 - 7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)

E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_TABLE = np.concatenate([E2M1_MAG, -E2M1_MAG])


def e8m0_to_f64(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    out = np.ldexp(1.0, c - 127).astype(np.float64)
    out[c == 255] = np.nan
    return out


# encoder for E4M3FN: candidates are the finite non-negative codes 0x00..0x7E
_E4M3_POS = E4M3_TABLE[:0x7F]


def encode_e4m3(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3FN code for each value, ties to even code, saturating at 448."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), 448.0)
    idx = np.searchsorted(_E4M3_POS, a)            # first candidate >= a
    idx = np.clip(idx, 1, 0x7E)
    lo, hi = idx - 1, idx
    dlo = a - _E4M3_POS[lo]
    dhi = _E4M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == 0.0, 0, code)
    sign = np.signbit(v) & (code != 0)
    return (code | (sign.astype(np.int64) << 7)).astype(np.uint8)


def lookup(table: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """table[codes] along the first axis (codes: uint8 array of any shape).
    Large arrays go through torch's CPU index_select, which runs the same
    gather on every core (numpy's fancy indexing is single-threaded and the
    weight blobs hold tens of millions of codes)."""
    c = np.asarray(codes, dtype=np.uint8)
    if c.size < (1 << 16):
        return table[c]
    import torch
    t = torch.from_numpy(np.ascontiguousarray(table))
    out = torch.index_select(t, 0, torch.from_numpy(c.reshape(-1)).long()).numpy()
    return out.reshape(c.shape + table.shape[1:])


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    return lookup(E4M3_TABLE, codes)


def decode_e2m1(nibbles: np.ndarray) -> np.ndarray:
    return E2M1_TABLE[np.asarray(nibbles, dtype=np.uint8) & 0xF]


def _e2m3_value(code: int) -> float:
    s = -1.0 if code & 0x20 else 1.0
    e = (code >> 3) & 0x3
    m = code & 0x7
    if e == 0:
        return s * (m / 8.0)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 1)


E2M3_TABLE = np.array([_e2m3_value(c) for c in range(64)], dtype=np.float64)
_E2M3_POS = E2M3_TABLE[:0x20]


def encode_e2m3(v: np.ndarray) -> np.ndarray:
    """Nearest E2M3 code (6 bits) for each value, ties to the even code,
    saturating at 7.5; the sign bit follows v except for a zero result."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), 7.5)
    idx = np.clip(np.searchsorted(_E2M3_POS, a), 1, 0x1F)
    lo, hi = idx - 1, idx
    dlo = a - _E2M3_POS[lo]
    dhi = _E2M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == 0.0, 0, code)
    sign = np.signbit(v) & (code != 0)
    return (code | (sign.astype(np.int64) << 5)).astype(np.uint8)


def decode_e2m3(codes: np.ndarray) -> np.ndarray:
    return E2M3_TABLE[np.asarray(codes, dtype=np.uint8) & 0x3F]
