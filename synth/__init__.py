"""Seeded synthetic inputs for the routed MoE layer.

This module only draws numbers and lays them out; it contains none of the
MoE layer's arithmetic.  Both the HIP library's callers and the oracle's
callers take their inputs from here, so the two sides read identical bytes.

The five workload shapes are the benchmark configurations of this layer
(tiny, decode-shaped, prefill-shaped, large-pool fp8, MXFP4); the value
distributions are: expert weights N(0, 0.02) stored in the pool format,
activations N(0, 1) as bf16, router weights N(0, 0.1) fp32.

Readings (the pages give no distributions; these are stated choices):
  * router bias "Zipf(s=1.1) over experts": b_e = -1.1 * ln(r_e), r_e a
    seeded per-layer permutation rank in 1..E, added to the logits;
  * "log-normal router logit scales": row e of router_w is multiplied by
    exp(0.5 * zeta_e), zeta_e ~ N(0, 1), seeded per layer;
  * "0.7 probability of reusing the previous step's expert set": per
    (layer, token slot) and step > 0, with probability 0.7 the token's hidden
    row is the previous step's row (hence the same experts), otherwise a
    fresh N(0, 1) row.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None
_table = None

FMT_BF16, FMT_FP8, FMT_MXFP4, FMT_NVFP4 = 0, 1, 2, 3
FMT_NAMES = {FMT_BF16: "bf16", FMT_FP8: "fp8_e4m3_b128", FMT_MXFP4: "mxfp4", FMT_NVFP4: "nvfp4"}

# tensor-kind tags mixed into the stream keys
_K_POOL, _K_ROUTER, _K_BIAS, _K_HIDDEN, _K_REUSE, _K_LOGNORM = 1, 2, 3, 4, 5, 6


@dataclass(frozen=True)
class MoeShape:
    name: str
    L: int
    E: int
    k: int
    H: int
    I: int
    fmt: int
    slot_fraction: float
    zipf_bias: bool = False
    lognormal_scales: bool = False
    decode_T: tuple = ()
    prefill_T: tuple = ()
    config_id: int = 0
    w_sigma: float = 0.02
    x_sigma: float = 1.0
    r_sigma: float = 0.1
    reuse_p: float = 0.7

    @property
    def expert_bytes(self) -> int:
        return expert_bytes(self.fmt, self.H, self.I)

    @property
    def n_slots(self) -> int:
        return max(self.k, int(round(self.slot_fraction * self.L * self.E)))

    def with_layers(self, L: int) -> "MoeShape":
        return replace(self, L=L)


CONFIGS = {
    1: MoeShape("tiny", L=1, E=8, k=2, H=256, I=128, fmt=FMT_BF16, slot_fraction=1.0,
                decode_T=(16,), config_id=1),
    2: MoeShape("decode_bf16", L=48, E=128, k=8, H=2048, I=768, fmt=FMT_BF16, slot_fraction=0.4,
                zipf_bias=True, decode_T=(1, 8, 32, 64), config_id=2),
    3: MoeShape("prefill_bf16", L=48, E=128, k=8, H=2048, I=768, fmt=FMT_BF16, slot_fraction=0.4,
                prefill_T=(4096, 8192, 16384), config_id=3),
    4: MoeShape("largepool_fp8", L=43, E=256, k=6, H=4096, I=2048, fmt=FMT_FP8, slot_fraction=0.3,
                lognormal_scales=True, decode_T=(1, 32), prefill_T=(4096,), config_id=4),
    5: MoeShape("mxfp4", L=16, E=256, k=8, H=6144, I=2048, fmt=FMT_MXFP4, slot_fraction=0.25,
                zipf_bias=True, decode_T=(1,), prefill_T=(16384,), config_id=5),
}


def expert_bytes(fmt: int, H: int, I: int) -> int:
    n = H * I
    if fmt == FMT_BF16:
        return 3 * n * 2
    if fmt == FMT_FP8:
        return 3 * n + 3 * (n // (128 * 128)) * 4
    if fmt == FMT_NVFP4:
        return 3 * n // 2 + 3 * n // 16 + 16
    return 3 * n // 2 + 3 * n // 32


def build(force: bool = True) -> str:
    """Compile fill.c into libsynth.so (gcc, OpenMP)."""
    src = os.path.join(_HERE, "fill.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        u64, sz, vp = ctypes.c_uint64, ctypes.c_size_t, ctypes.c_void_p
        L.synth_word.restype = u64
        L.synth_word.argtypes = [u64, u64]
        L.synth_key.restype = u64
        L.synth_key.argtypes = [u64, u64]
        L.synth_normal_bf16.argtypes = [vp, sz, u64, vp, ctypes.c_float]
        L.synth_normal_f32.argtypes = [vp, sz, u64, vp, ctypes.c_float]
        L.synth_uniform_f64.argtypes = [vp, sz, u64]
        L.synth_expert_bytes.restype = sz
        L.synth_expert_bytes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.synth_expert_blob.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, u64, vp, ctypes.c_float]
        L.synth_pool.argtypes = [vp, sz, ctypes.c_long, ctypes.c_long, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 u64, vp, ctypes.c_float]
        L.synth_keys.argtypes = [vp, sz, u64, u64]
        L.synth_rows_bf16.argtypes = [vp, vp, sz, ctypes.c_int, vp, ctypes.c_float]
        _lib = L
    return _lib


def normal_table() -> np.ndarray:
    """65536 quantiles of N(0,1) at probabilities (i+0.5)/65536, fp32."""
    global _table
    if _table is None:
        from scipy.special import ndtri
        p = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
        _table = np.ascontiguousarray(ndtri(p).astype(np.float32))
    return _table


def key(*parts: int) -> int:
    k = 0x5EED
    for p in parts:
        k = lib().synth_key(k, int(p) & 0xFFFFFFFFFFFFFFFF)
    return k


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def normal_bf16(n: int, k: int, sigma: float) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    t = normal_table()
    lib().synth_normal_bf16(_ptr(out), n, k, _ptr(t), sigma)
    return out


def normal_f32(n: int, k: int, sigma: float) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    t = normal_table()
    lib().synth_normal_f32(_ptr(out), n, k, _ptr(t), sigma)
    return out


def uniform_f64(n: int, k: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    lib().synth_uniform_f64(_ptr(out), n, k)
    return out


def pool_key(cfg: MoeShape, seed: int) -> int:
    return key(seed, cfg.config_id, _K_POOL)


def expert_blob(cfg: MoeShape, seed: int, layer: int, expert: int) -> np.ndarray:
    """Bytes of expert (layer, expert): identical to row layer*E+expert of the pool."""
    S = cfg.expert_bytes
    out = np.empty(S, dtype=np.uint8)
    g = layer * cfg.E + expert
    k = lib().synth_key(pool_key(cfg, seed), g)
    lib().synth_expert_blob(_ptr(out), cfg.fmt, cfg.H, cfg.I, k, _ptr(normal_table()), cfg.w_sigma)
    return out


def fill_pool(ptr: int, cfg: MoeShape, seed: int, first: int = 0, count: int | None = None) -> None:
    """Write experts [first, first+count) of the [L*E][S] pool at host address ptr."""
    if count is None:
        count = cfg.L * cfg.E - first
    lib().synth_pool(ptr, cfg.expert_bytes, first, count, cfg.fmt, cfg.H, cfg.I, pool_key(cfg, seed),
                     _ptr(normal_table()), cfg.w_sigma)


def pool_array(cfg: MoeShape, seed: int) -> np.ndarray:
    """Whole pool as a host numpy array [L*E, S] (small configurations only)."""
    S = cfg.expert_bytes
    out = np.empty((cfg.L * cfg.E, S), dtype=np.uint8)
    fill_pool(_ptr(out), cfg, seed)
    return out


def router_weights(cfg: MoeShape, seed: int, layer: int) -> np.ndarray:
    """router_w [E, H] fp32 (row e optionally scaled log-normally)."""
    w = normal_f32(cfg.E * cfg.H, key(seed, cfg.config_id, _K_ROUTER, layer), cfg.r_sigma).reshape(cfg.E, cfg.H)
    if cfg.lognormal_scales:
        z = normal_f32(cfg.E, key(seed, cfg.config_id, _K_LOGNORM, layer), 1.0).astype(np.float64)
        s = np.exp(0.5 * z).astype(np.float32)
        w = (w * s[:, None]).astype(np.float32)
    return np.ascontiguousarray(w)


def router_bias(cfg: MoeShape, seed: int, layer: int) -> np.ndarray | None:
    """Additive logit bias [E] fp32 (Zipf log-prior) or None."""
    if not cfg.zipf_bias:
        return None
    u = uniform_f64(cfg.E, key(seed, cfg.config_id, _K_BIAS, layer))
    rank = np.empty(cfg.E, dtype=np.int64)
    rank[np.argsort(u, kind="stable")] = np.arange(1, cfg.E + 1)
    return (-1.1 * np.log(rank.astype(np.float64))).astype(np.float32)


def hidden_rows(cfg: MoeShape, row_keys: np.ndarray) -> np.ndarray:
    """bf16 bit patterns [len(row_keys), H], one N(0,1) row per key."""
    keys = np.ascontiguousarray(row_keys, dtype=np.uint64).reshape(-1)
    out = np.empty((len(keys), cfg.H), dtype=np.uint16)
    lib().synth_rows_bf16(_ptr(out), _ptr(keys), len(keys), cfg.H, _ptr(normal_table()), cfg.x_sigma)
    return out


def keys_range(base: int, first: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    lib().synth_keys(_ptr(out), n, base, first)
    return out


def hidden(cfg: MoeShape, seed: int, T: int, tag: int = 0) -> np.ndarray:
    """Fresh activations [T, H] as bf16 bit patterns."""
    return hidden_rows(cfg, keys_range(key(seed, cfg.config_id, _K_HIDDEN, tag), 0, T))


def decode_row_keys(cfg: MoeShape, seed: int, steps: int, T: int, layers: int | None = None) -> np.ndarray:
    """Row keys [steps, layers, T] of the decode locality model.

    Step 0 is fresh; for step > 0, each (layer, slot) keeps its previous row
    with probability reuse_p, else draws a fresh row.
    """
    L = cfg.L if layers is None else layers
    keys = np.empty((steps, L, T), dtype=np.uint64)
    base = key(seed, cfg.config_id, _K_HIDDEN, 0xDEC0DE, T)
    reuse_base = key(seed, cfg.config_id, _K_REUSE, T)
    for s in range(steps):
        fresh = keys_range(base, s * L * 65536, L * 65536).reshape(L, 65536)[:, :T]
        if s == 0:
            keys[s] = fresh
        else:
            u = uniform_f64(L * T, lib().synth_key(reuse_base, s)).reshape(L, T)
            keys[s] = np.where(u < cfg.reuse_p, keys[s - 1], fresh)
    return keys

