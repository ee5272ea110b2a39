"""Plain, slow float64 oracle of one routed MoE layer.

TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the bench's
CPU-baseline leg; nothing on the product path imports it.

What the layer computes (source: the paper.oopus.info review of FreeToken,
section 2 and 2.5; the gpts24 analysis "FreeToken 重写本地 MoE 推理", where a
gate network picks a few experts per token):
  * every token is routed to k of E experts by a gate (softmax router, top-k,
    weights renormalised over the chosen k);
  * each expert is an independent feed-forward network (SwiGLU, no biases);
  * the layer output is the gate-weighted sum of the chosen experts' outputs.
Section 2.5 of the review states the split of the miss set between the GPU
and the host changes only where a partial sum is computed; the partials are
added exactly.  Section 2 states the cache contents never change the result.
So the oracle is the plain definition of the layer, independent of caching,
slots and transport.

Readings where the pages are silent (also listed in the design notes):
  * gate = softmax over E logits z = x R^T + b; selection on logits, larger
    first, equal values -> lower expert index; weights = softmax over the k
    selected logits (identical to the full softmax renormalised over them);
  * expert e: W_gate, W_up [I,H], W_down [H,I]; FFN(x) = W_down (silu(W_gate x)
    * (W_up x)), silu(g) = g / (1 + exp(-g));
  * expert blob: gate, up, down row-major [out,in], then scale arrays in the
    same order (fp8: fp32 per 128x128 block; mxfp4: E8M0 per 32 inputs, two
    E2M1 codes per byte, even element in the low nibble; nvfp4: codes as
    mxfp4, E4M3 per 16 inputs, then the three fp32 tensor scales).

Two modes: "exact" (float64 throughout, weights dequantised exactly) and
"mirrored" (float64 arithmetic with the GPU path's declared rounding and
quantisation points applied; see `mirror_*` below).

Parity pins: the tests check this module against a dense brute force, the
single-FFN special cases (E = 1; identical experts), linearity of the split,
worked examples with hand-computed values, and the format definitions.
"""
from __future__ import annotations

import numpy as np

from .formats import (bf16_to_f64, decode_e2m1, decode_e2m3, decode_e4m3, e8m0_to_f64, encode_e2m3,
                      encode_e4m3, lookup, round_to_bf16, round_to_f16)

FMT_BF16, FMT_FP8, FMT_MXFP4, FMT_NVFP4 = 0, 1, 2, 3

# the two E2M1 values packed in each byte value: [low nibble, high nibble]
E2M1_PAIRS = np.stack([decode_e2m1(np.arange(256) & 0xF), decode_e2m1(np.arange(256) >> 4)], axis=1)


# ----------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------

def router_logits(x_bits: np.ndarray, router_w: np.ndarray, bias: np.ndarray | None) -> np.ndarray:
    """z[t,e] = sum_h x[t,h] * R[e,h] + b[e], float64 (x bf16, R fp32 exact in f64)."""
    x = bf16_to_f64(x_bits)
    R = np.asarray(router_w, dtype=np.float32).astype(np.float64)
    z = x @ R.T
    if bias is not None:
        z = z + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    return z


def select_topk(z: np.ndarray, k: int) -> np.ndarray:
    """Per row, the k indices of the largest values, ordered by value descending,
    ties broken by lower index.  Values are compared as given (fp32 logits are
    passed as float64 exactly)."""
    z = np.asarray(z, dtype=np.float64)
    T, E = z.shape
    ids = np.empty((T, k), dtype=np.int32)
    idx = np.arange(E)
    for t in range(T):
        # lexsort: last key is primary -> sort by -z, then by index
        order = np.lexsort((idx, -z[t]))
        ids[t] = order[:k]
    return ids


def topk_margin(z: np.ndarray, k: int) -> np.ndarray:
    """z_(k) - z_(k+1) per row (inf when k == E): how far a token is from a tie."""
    z = np.asarray(z, dtype=np.float64)
    if k >= z.shape[1]:
        return np.full(z.shape[0], np.inf)
    s = -np.sort(-z, axis=1)
    return s[:, k - 1] - s[:, k]


def gate_weights(z: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """w[t,j] = exp(z[t,ids[t,j]]) / sum_i exp(z[t,ids[t,i]]) (softmax over the chosen)."""
    sel = np.take_along_axis(np.asarray(z, dtype=np.float64), ids.astype(np.int64), axis=1)
    m = sel.max(axis=1, keepdims=True)
    e = np.exp(sel - m)
    return e / e.sum(axis=1, keepdims=True)


def route_index(ids: np.ndarray, E: int):
    """Group the (token, choice) assignments by expert.

    Returns counts [E], offsets [E+1] (exclusive scan), perm_tok [T*k] (token of
    each grouped row, experts ascending, tokens ascending within an expert),
    perm_j [T*k] (which choice j of that token), pos [T,k] (grouped row of each
    assignment).
    """
    T, k = ids.shape
    counts = np.zeros(E, dtype=np.int64)
    for e in ids.reshape(-1):
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    fill = offsets[:-1].copy()
    perm_tok = np.empty(T * k, dtype=np.int32)
    perm_j = np.empty(T * k, dtype=np.int32)
    pos = np.empty((T, k), dtype=np.int32)
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if ids[t, j] == e:
                    r = fill[e]
                    fill[e] += 1
                    perm_tok[r] = t
                    perm_j[r] = j
                    pos[t, j] = r
    return counts.astype(np.int32), offsets.astype(np.int32), perm_tok, perm_j, pos


# ----------------------------------------------------------------------------
# expert weights
# ----------------------------------------------------------------------------

def dequant_expert(blob: np.ndarray, fmt: int, H: int, I: int):
    """Exact float64 (W_gate [I,H], W_up [I,H], W_down [H,I]) from one expert blob."""
    b = np.asarray(blob, dtype=np.uint8)
    n = H * I
    if fmt == FMT_BF16:
        w = b[: 6 * n].view(np.uint16)
        g = bf16_to_f64(w[:n]).reshape(I, H)
        u = bf16_to_f64(w[n:2 * n]).reshape(I, H)
        d = bf16_to_f64(w[2 * n:3 * n]).reshape(H, I)
        return g, u, d
    if fmt == FMT_FP8:
        ns = n // (128 * 128)
        sc = b[3 * n: 3 * n + 3 * ns * 4].view(np.float32).astype(np.float64)

        def mat(q, s, rows, cols):
            # element (r, c) times the scale of block (r // 128, c // 128)
            v = decode_e4m3(q).reshape(rows // 128, 128, cols // 128, 128)
            v *= s.reshape(rows // 128, 1, cols // 128, 1)
            return v.reshape(rows, cols)

        g = mat(b[:n], sc[:ns], I, H)
        u = mat(b[n:2 * n], sc[ns:2 * ns], I, H)
        d = mat(b[2 * n:3 * n], sc[2 * ns:], H, I)
        return g, u, d
    if fmt == FMT_MXFP4:
        npk, ns = n // 2, n // 32
        sc = b[3 * npk: 3 * npk + 3 * ns]

        def mat(p, s, rows, cols):
            # byte -> (even element = low nibble, odd element = high nibble)
            v = lookup(E2M1_PAIRS, p).reshape(rows, cols // 32, 32)
            v *= e8m0_to_f64(s).reshape(rows, cols // 32, 1)
            return v.reshape(rows, cols)

        g = mat(b[:npk], sc[:ns], I, H)
        u = mat(b[npk:2 * npk], sc[ns:2 * ns], I, H)
        d = mat(b[2 * npk:3 * npk], sc[2 * ns:], H, I)
        return g, u, d
    if fmt == FMT_NVFP4:
        npk, ns = n // 2, n // 16
        sc = b[3 * npk: 3 * npk + 3 * ns]
        ts = b[3 * npk + 3 * ns: 3 * npk + 3 * ns + 12].view(np.float32).astype(np.float64)

        def mat(p, s, t, rows, cols):
            v = lookup(E2M1_PAIRS, p).reshape(rows, cols // 16, 16)
            v *= decode_e4m3(s).reshape(rows, cols // 16, 1)
            v = v.reshape(rows, cols)
            v *= t
            return v

        g = mat(b[:npk], sc[:ns], ts[0], I, H)
        u = mat(b[npk:2 * npk], sc[ns:2 * ns], ts[1], I, H)
        d = mat(b[2 * npk:3 * npk], sc[2 * ns:], ts[2], H, I)
        return g, u, d
    raise ValueError(f"unknown weight format {fmt}")


def silu(g: np.ndarray) -> np.ndarray:
    return g / (1.0 + np.exp(-g))


def expert_ffn(x: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    """SwiGLU expert on rows of x (float64): (silu(x Wg^T) * (x Wu^T)) Wd^T."""
    g = x @ Wg.T
    u = x @ Wu.T
    return (silu(g) * u) @ Wd.T


# ----------------------------------------------------------------------------
# mirrored rounding / quantisation points of the GPU path
# ----------------------------------------------------------------------------

def mirror_quant_fp8_groups(v: np.ndarray, group: int = 128) -> np.ndarray:
    """Per (row, group of `group` columns): amax, inv = fp32(448/amax),
    code = E4M3(fp32(v*inv)), value = code * fp32(amax/448).  Decisions in fp32."""
    v32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    rows, cols = v32.shape
    g = v32.reshape(rows, cols // group, group)
    amax = np.abs(g).max(axis=2, keepdims=True)
    safe = np.where(amax > 0, amax, np.float32(1.0)).astype(np.float32)
    inv = np.where(amax > 0, np.float32(448.0) / safe, np.float32(1.0)).astype(np.float32)
    scale = np.where(amax > 0, safe / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    scaled = (g * inv).astype(np.float32)
    codes = encode_e4m3(scaled.astype(np.float64))
    return (decode_e4m3(codes) * scale.astype(np.float64)).reshape(rows, cols)


def mirror_quant_mxfp8(v: np.ndarray) -> np.ndarray:
    """OCP MX rule with E4M3 elements per 32 columns: x = floor(log2 amax) - 8
    (clamped to [-127,127], amax = 0 -> x = 0), code = E4M3(v * 2^-x), value =
    code * 2^x."""
    v32 = np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)
    rows, cols = v32.shape
    g = v32.reshape(rows, cols // 32, 32)
    amax = np.abs(g).max(axis=2, keepdims=True)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    x = np.where(amax > 0, np.clip(ex - 1 - 8, -127, 127), 0)
    codes = encode_e4m3(np.ldexp(g, -x))
    return np.ldexp(decode_e4m3(codes), x).reshape(rows, cols)


def mirror_quant_mxfp6(v: np.ndarray) -> np.ndarray:
    """OCP MX rule with FP6 E2M3 elements per 32 columns: x = floor(log2 amax)
    - 2 (2 = exponent of E2M3's largest normal; clamped to [-127,127], amax
    = 0 -> x = 0), code = E2M3(v * 2^-x) saturating at 7.5, value = code *
    2^x."""
    v32 = np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)
    rows, cols = v32.shape
    g = v32.reshape(rows, cols // 32, 32)
    amax = np.abs(g).max(axis=2, keepdims=True)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    x = np.where(amax > 0, np.clip(ex - 1 - 2, -127, 127), 0)
    codes = encode_e2m3(np.ldexp(g, -x))
    return np.ldexp(decode_e2m3(codes), x).reshape(rows, cols)


def mirror_activation(v: np.ndarray, fmt: int, act: str | None = None) -> np.ndarray:
    """The GPU path's rounding of a GEMM input activation (x before GEMM 1,
    A before GEMM 2).  act="bf16": rounded to bf16 whatever the weight
    format (fp8 and mxfp4 weights dequantised exactly to bf16 meet bf16
    activations: the small-batch kernels).  Otherwise by format: bf16 ->
    bf16, nvfp4 -> fp16 (its dequantised weights and the activations meet in
    the fp16 MFMA), fp8 -> per-128 E4M3, mxfp4 -> MXFP8, or MXFP6 with
    act="mxfp6" (the large-batch kernels' 8-bit and 6-bit activations)."""
    if fmt == FMT_BF16 or act == "bf16":
        return round_to_bf16(v)
    if fmt == FMT_NVFP4:
        return round_to_f16(v)
    if fmt == FMT_FP8:
        return mirror_quant_fp8_groups(v, 128)
    if act == "mxfp6":
        return mirror_quant_mxfp6(v)
    return mirror_quant_mxfp8(v)


def expert_ffn_mirrored(x: np.ndarray, Wg, Wu, Wd, fmt: int, act: str | None = None) -> np.ndarray:
    """Expert output Z with the GPU path's rounding points: x quantised (fp8,
    mxfp4) or rounded to fp16 (nvfp4), A = silu(g)*u rounded to bf16 or fp16
    or quantised, Z rounded to bf16.  nvfp4 weights enter the fp16 MFMA as
    element * block scale (exact in fp16) and the tensor scale multiplies
    the fp32 sums, so the weights are not rounded here; fp8 and mxfp4
    weights meeting bf16 activations are exact in bf16 as well (E4M3 codes,
    and E2M1 codes times a power-of-two block scale; the fp8 block scale
    multiplies fp32 partial sums).  act: "bf16" (16-bit activations for any
    format), None (the format's rule above) or "mxfp6" (mxfp4 weights)."""
    xq = x if fmt == FMT_BF16 else mirror_activation(x, fmt, act)
    g = xq @ Wg.T
    u = xq @ Wu.T
    a = silu(g) * u
    aq = mirror_activation(a, fmt, act)
    return round_to_bf16(aq @ Wd.T)


# ----------------------------------------------------------------------------
# the layer
# ----------------------------------------------------------------------------

def moe_layer(x_bits, router_w, bias, k, expert_weights, fmt=FMT_BF16, mode="exact",
              host_set=None, logits=None, act=None):
    """One routed MoE layer.

    x_bits: bf16 bit patterns [T,H]; router_w [E,H] fp32; bias [E] or None;
    expert_weights(e) -> (Wg, Wu, Wd) float64; mode "exact", "mirrored" or
    "both" (one pass over the experts, each dequantised once: out = the
    mirrored output, out_exact = the exact one);
    host_set: experts whose contribution is computed by the host branch.  In
    "mirrored" mode those are evaluated exactly (the host branch keeps fp32,
    without the GPU's intermediate rounding) and added before the final bf16
    rounding.  logits: optional precomputed [T,E] logits.  act: activation
    rule in "mirrored" mode ("bf16", None: the format's own, "mxfp6").
    Returns dict(out [T,H] float64, ids, w, z, margin).
    """
    x = bf16_to_f64(x_bits)
    z = router_logits(x_bits, router_w, bias) if logits is None else np.asarray(logits, np.float64)
    T, E = z.shape
    ids = select_topk(z, k)
    w = gate_weights(z, ids)
    host_set = set() if host_set is None else set(int(e) for e in host_set)
    out = np.zeros_like(x)
    out_x = np.zeros_like(x) if mode == "both" else None
    for e in sorted(set(ids.reshape(-1).tolist())):
        rows, js = np.nonzero(ids == e)
        Wg, Wu, Wd = expert_weights(e)
        xe = x[rows]
        ye_x = expert_ffn(xe, Wg, Wu, Wd) if mode != "mirrored" or e in host_set else None
        if mode == "exact" or e in host_set:
            ye = ye_x
        else:
            ye = expert_ffn_mirrored(xe, Wg, Wu, Wd, fmt, act)
        out[rows] += w[rows, js][:, None] * ye
        if out_x is not None:
            out_x[rows] += w[rows, js][:, None] * ye_x
    if mode in ("mirrored", "both"):
        out = round_to_bf16(out)
    res = dict(out=out, ids=ids, w=w, z=z, margin=topk_margin(z, k))
    if out_x is not None:
        res["out_exact"] = out_x
    return res


def host_partial(x_bits, ids, w, host_set, expert_weights) -> np.ndarray:
    """sum over j with ids[t,j] in host_set of w[t,j] * FFN_e(x_t), float64 [T,H]."""
    x = bf16_to_f64(x_bits)
    out = np.zeros_like(x)
    for e in sorted(set(int(v) for v in host_set)):
        rows, js = np.nonzero(ids == e)
        if len(rows) == 0:
            continue
        out[rows] += w[rows, js][:, None] * expert_ffn(x[rows], *expert_weights(e))
    return out
