"""Pins of the oracle's expert FFN, dequantisation and layer: hand-computed
worked examples, a dense brute force, special cases and invariants."""
import dataclasses
import math

import numpy as np
import pytest
import torch
from scipy.special import expit, softmax

import synth
from oracle import formats as F
from oracle import moe as M


def _bf16_bits(vals):
    return torch.tensor(np.asarray(vals, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_blob(Wg, Wu, Wd):
    return np.concatenate([_bf16_bits(Wg).ravel(), _bf16_bits(Wu).ravel(), _bf16_bits(Wd).ravel()]).view(np.uint8)


def test_ffn_worked_example_bf16():
    # H=4, I=2.  g = Wg x = [1, 2], u = Wu x = [2, 3]
    # a = [silu(1)*2, silu(2)*3] with silu(g) = g*sigmoid(g); out = Wd a = [a0, a1, 2 a0, -a1]
    Wg = [[1, 0, 0, 0], [0, 0, 1, 0]]
    Wu = [[0, 2, 0, 0], [0, 0, 0, 1]]
    Wd = [[1, 0], [0, 1], [2, 0], [0, -1]]
    blob = _bf16_blob(Wg, Wu, Wd)
    g, u, d = M.dequant_expert(blob, M.FMT_BF16, 4, 2)
    x = np.array([[1.0, 1.0, 2.0, 3.0]])
    a0 = 2.0 / (1.0 + math.exp(-1.0))
    a1 = 3.0 * 2.0 / (1.0 + math.exp(-2.0))
    want = np.array([a0, a1, 2 * a0, -a1])
    np.testing.assert_allclose(M.expert_ffn(x, g, u, d)[0], want, rtol=1e-15)


def test_silu_textbook():
    g = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(M.silu(g), g * expit(g), rtol=1e-13, atol=1e-300)
    assert M.silu(np.array([0.0]))[0] == 0.0


def test_fp8_blob_worked_example():
    H = I = 128
    n = H * I
    q = np.zeros(3 * n, dtype=np.uint8)
    q[0 * n + 0 * H + 0] = 0x38            # gate[0,0] code 1.0
    q[1 * n + 0 * H + 1] = 0x40            # up[0,1] code 2.0
    q[2 * n + 5 * I + 0] = 0xB8            # down[5,0] code -1.0
    scales = np.array([0.5, 0.25, 2.0], dtype=np.float32)   # one 128x128 block per matrix
    blob = np.concatenate([q, scales.view(np.uint8)])
    g, u, d = M.dequant_expert(blob, M.FMT_FP8, H, I)
    assert g[0, 0] == 0.5 and u[0, 1] == 0.5 and d[5, 0] == -2.0
    assert np.count_nonzero(g) == 1 and np.count_nonzero(u) == 1 and np.count_nonzero(d) == 1
    x = np.zeros((1, H)); x[0, 0] = 2.0; x[0, 1] = 4.0
    # g0 = 0.5*2 = 1, u0 = 0.5*4 = 2, a0 = silu(1)*2, out[5] = -2 a0
    out = M.expert_ffn(x, g, u, d)[0]
    assert out[5] == pytest.approx(-2.0 * 2.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert np.count_nonzero(out) == 1


def test_mxfp4_blob_worked_example():
    H, I = 64, 32
    n = H * I
    packed = np.zeros(3 * n // 2, dtype=np.uint8)
    scales = np.full(3 * n // 32, 127, dtype=np.uint8)       # 2^0
    packed[0] = 0x2 | (0xB << 4)            # gate[0,0] = 1.0 (low nibble), gate[0,1] = -1.5
    scales[0] = 128                         # gate row 0, inputs 0..31: x2
    # up[3, 40] = 6.0 (code 7), in byte (3*64+40)/2, even -> low nibble; block (3, 1) scale 2^-1
    packed[n // 2 + (3 * H + 40) // 2] = 0x7
    scales[n // 32 + 3 * (H // 32) + 1] = 126
    # down[10, 31] = -0.5 (code 0x9), odd element -> high nibble; block (10, 0) scale 2^3
    packed[n + (10 * I + 31) // 2] = 0x9 << 4
    scales[2 * n // 32 + 10 * (I // 32) + 0] = 130
    blob = np.concatenate([packed, scales])
    g, u, d = M.dequant_expert(blob, M.FMT_MXFP4, H, I)
    assert g[0, 0] == 2.0 and g[0, 1] == -3.0 and np.count_nonzero(g) == 2
    assert u[3, 40] == 3.0 and np.count_nonzero(u) == 1
    assert d[10, 31] == -4.0 and np.count_nonzero(d) == 1


def _tiny(fmt=M.FMT_BF16, **kw):
    c = dataclasses.replace(synth.CONFIGS[1], fmt=fmt, **kw)
    if fmt != M.FMT_BF16:
        c = dataclasses.replace(c, H=256, I=128)
    return c


def _weights_fn(cfg, seed, layer=0):
    cache = {}

    def get(e):
        if e not in cache:
            cache[e] = M.dequant_expert(synth.expert_blob(cfg, seed, layer, e), cfg.fmt, cfg.H, cfg.I)
        return cache[e]
    return get


def _brute_layer(x_bits, R, b, k, weights, E):
    """Dense: every token through every expert, weighted by the renormalised
    softmax restricted to the token's k largest logits (selection by sort)."""
    x = F.bf16_to_f64(x_bits)
    z = x @ R.astype(np.float64).T + (0 if b is None else b.astype(np.float64))
    p = softmax(z, axis=1)
    T = x.shape[0]
    out = np.zeros_like(x)
    for e in range(E):
        Wg, Wu, Wd = weights(e)
        g = x @ Wg.T
        y = (g * expit(g) * (x @ Wu.T)) @ Wd.T
        for t in range(T):
            order = sorted(range(E), key=lambda i: (-z[t, i], i))[:k]
            if e in order:
                out[t] += p[t, e] / p[t, order].sum() * y[t]
    return out


@pytest.mark.parametrize("fmt", [M.FMT_BF16, M.FMT_FP8, M.FMT_MXFP4])
def test_layer_matches_dense_brute_force(fmt):
    cfg = _tiny(fmt)
    x = synth.hidden(cfg, 0, 16)
    R = synth.router_weights(cfg, 0, 0)
    wf = _weights_fn(cfg, 0)
    r = M.moe_layer(x, R, None, cfg.k, wf, fmt=fmt, mode="exact")
    ref = _brute_layer(x, R, None, cfg.k, wf, cfg.E)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-11, atol=1e-13)


def test_single_expert_is_plain_ffn():
    cfg = dataclasses.replace(_tiny(), E=1, k=1)
    x = synth.hidden(cfg, 1, 5)
    R = synth.router_weights(cfg, 1, 0)
    wf = _weights_fn(cfg, 1)
    r = M.moe_layer(x, R, None, 1, wf)
    assert np.array_equal(r["w"], np.ones((5, 1)))
    np.testing.assert_array_equal(r["out"], M.expert_ffn(F.bf16_to_f64(x), *wf(0)))


def test_identical_experts_give_single_ffn():
    cfg = _tiny()
    x = synth.hidden(cfg, 2, 16)
    R = synth.router_weights(cfg, 2, 0)
    same = M.dequant_expert(synth.expert_blob(cfg, 2, 0, 0), cfg.fmt, cfg.H, cfg.I)
    r = M.moe_layer(x, R, synth.router_bias(synth.CONFIGS[2], 0, 0)[:8], cfg.k, lambda e: same)
    np.testing.assert_allclose(r["out"], M.expert_ffn(F.bf16_to_f64(x), *same), rtol=1e-12, atol=1e-14)


def test_split_is_exact_sum_of_partials():
    cfg = _tiny()
    x = synth.hidden(cfg, 3, 16)
    R = synth.router_weights(cfg, 3, 0)
    wf = _weights_fn(cfg, 3)
    full = M.moe_layer(x, R, None, cfg.k, wf)
    C = {1, 4, 6}
    zero = tuple(np.zeros_like(w) for w in wf(0))
    gpu_only = M.moe_layer(x, R, None, cfg.k, lambda e: zero if e in C else wf(e))
    hp = M.host_partial(x, full["ids"], full["w"], C, wf)
    np.testing.assert_allclose(gpu_only["out"] + hp, full["out"], rtol=1e-13, atol=1e-15)


# Sanity bound only: the mirrored mode adds the GPU path's activation rounding
# (bf16: 2^-9 relative; E4M3: 2^-4 relative per element), so it sits a
# quantisation step away from the exact layer.
@pytest.mark.parametrize("fmt,tol,act", [(M.FMT_BF16, 1e-2, None), (M.FMT_FP8, 0.1, None),
                                         (M.FMT_MXFP4, 0.1, None), (M.FMT_MXFP4, 0.1, "mxfp6"),
                                         (M.FMT_NVFP4, 1e-2, None)])
def test_mirrored_mode_close_to_exact(fmt, tol, act):
    cfg = _tiny(fmt)
    x = synth.hidden(cfg, 4, 16)
    R = synth.router_weights(cfg, 4, 0)
    wf = _weights_fn(cfg, 4)
    ex = M.moe_layer(x, R, None, cfg.k, wf, fmt=fmt, mode="exact")["out"]
    mi = M.moe_layer(x, R, None, cfg.k, wf, fmt=fmt, mode="mirrored", act=act)["out"]
    err = np.abs(mi - ex).max() / np.abs(ex).max()
    assert 0 < err <= tol


def test_fp8_activation_quant_codes_match_torch():
    rng = np.random.default_rng(5)
    v = rng.normal(0, 1, size=(7, 256)).astype(np.float32)
    got = M.mirror_quant_fp8_groups(v.astype(np.float64))
    g = v.reshape(7, 2, 128)
    amax = np.abs(g).max(axis=2, keepdims=True)
    inv = (np.float32(448.0) / amax).astype(np.float32)
    codes = torch.from_numpy((g * inv).astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    want = codes * (amax / np.float32(448.0)).astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(got, want.reshape(7, 256))


def test_mxfp8_scale_rule():
    # one block whose amax is 1.0 -> shared exponent floor(log2 1) - 8 = -8; 1.0 -> 256 is exact
    v = np.zeros((1, 32)); v[0, 0] = 1.0; v[0, 1] = 0.1; v[0, 2] = -0.75
    q = M.mirror_quant_mxfp8(v)
    assert q[0, 0] == 1.0 and q[0, 2] == -0.75
    # 0.1 * 256 = 25.6 -> nearest E4M3 is 26 (step 2 in [16,32)) -> 26/256
    assert q[0, 1] == 26.0 / 256.0
    # amax 1.9 -> exponent still -8; 1.9*256 = 486.4 saturates to 448
    v[0, 0] = 1.9
    assert M.mirror_quant_mxfp8(v)[0, 0] == 448.0 / 256.0


def test_mxfp6_scale_rule():
    # amax 1.0 -> shared exponent floor(log2 1) - 2 = -2 (E2M3's largest normal
    # is 1.875 * 2^2): elements are scaled by 4 onto the E2M3 grid
    v = np.zeros((2, 64)); v[0, 0] = 1.0; v[0, 1] = 0.1; v[0, 2] = -0.75
    q = M.mirror_quant_mxfp6(v)
    assert q[0, 0] == 1.0 and q[0, 2] == -0.75
    # 0.1 * 4 = 0.4 -> nearest E2M3 subnormal 3/8 -> 3/32
    assert q[0, 1] == 3.0 / 32.0
    # amax 1.9 -> exponent -2; 1.9 * 4 = 7.6 saturates to 7.5 -> 1.875
    v[0, 0] = 1.9
    assert M.mirror_quant_mxfp6(v)[0, 0] == 1.875
    # an all-zero block stays zero, blocks are independent
    v[1, 32:] = 1000.0
    q = M.mirror_quant_mxfp6(v)
    assert (q[1, :32] == 0).all() and (q[1, 32:] == 1024.0 * 7.5 / 8.0).all()


def test_mxfp6_relative_error_bound():
    """Elements within a binade of their block's amax keep E2M3's 3-bit
    mantissa: relative error <= 2^-4."""
    rng = np.random.default_rng(8)
    v = rng.normal(0, 1, size=(64, 256))
    q = M.mirror_quant_mxfp6(v)
    g = np.abs(v).reshape(64, 8, 32)
    amax = g.max(axis=2, keepdims=True)
    _, ex = np.frexp(amax)
    near = (g >= np.ldexp(1.0, ex - 1)).reshape(64, 256)   # same binade as amax
    rel = np.abs(q - v)[near] / np.abs(v)[near]
    assert rel.max() <= 2.0 ** -4 + 1e-12
    assert np.abs(q - v).max() <= np.abs(v).max() * 2.0 ** -3


@pytest.mark.parametrize("fmt,act", [(M.FMT_BF16, None), (M.FMT_FP8, None), (M.FMT_FP8, "bf16"),
                                     (M.FMT_MXFP4, "mxfp6"), (M.FMT_NVFP4, None)])
def test_both_modes_in_one_pass_equal_the_single_modes(fmt, act):
    cfg = _tiny(fmt)
    x = synth.hidden(cfg, 7, 16)
    R = synth.router_weights(cfg, 7, 0)
    wf = _weights_fn(cfg, 7)
    both = M.moe_layer(x, R, None, cfg.k, wf, fmt=fmt, mode="both", act=act, host_set={2})
    mi = M.moe_layer(x, R, None, cfg.k, wf, fmt=fmt, mode="mirrored", act=act, host_set={2})
    ex = M.moe_layer(x, R, None, cfg.k, wf, fmt=fmt, mode="exact", act=act)
    np.testing.assert_array_equal(both["out"], mi["out"])
    np.testing.assert_array_equal(both["out_exact"], ex["out"])


def test_bf16_activation_rule_applies_to_quantised_weights():
    """act="bf16": fp8 / MXFP4 weights (dequantised exactly) meet bf16-rounded
    activations, so the mirrored layer equals the bf16 rule applied to the
    same float64 weights."""
    cfg = _tiny(M.FMT_FP8)
    x = synth.hidden(cfg, 8, 16)
    R = synth.router_weights(cfg, 8, 0)
    wf = _weights_fn(cfg, 8)
    a = M.moe_layer(x, R, None, cfg.k, wf, fmt=M.FMT_FP8, mode="mirrored", act="bf16")["out"]
    b = M.moe_layer(x, R, None, cfg.k, wf, fmt=M.FMT_BF16, mode="mirrored")["out"]
    np.testing.assert_array_equal(a, b)
