"""Worked examples that pin the mirrored oracle's rounding points.

`expert_ffn_mirrored` applies the GPU path's declared rounding and
quantisation points in float64 arithmetic.  Each example below is built by
hand so that every one of those points changes the result: the expected
values are derived step by step in the comments (exact binary arithmetic, no
call into the oracle), and each lists which plausible mistake the example
catches.  A gate value g >= 40 gives silu(g) = g / (1 + e^-g) == g in
float64 (e^-40 < 2^-53), which keeps the examples free of transcendental
values except where silu itself is pinned.
"""
import math

import numpy as np

from oracle import moe as M


def _zeros(*shape):
    return np.zeros(shape, dtype=np.float64)


def test_bf16_rounds_A_and_Z_to_nearest_even():
    # one token, H = 2, I = 3
    x = np.array([[1.0, 0.0]])
    Wg, Wu, Wd = _zeros(3, 2), _zeros(3, 2), _zeros(2, 3)
    Wg[:, 0] = 128.0                        # g = 128 for every feature: silu(g) = 128
    Wu[0, 0] = 2.0 ** -7 + 2.0 ** -15       # A0 = 1 + 2^-8: a bf16 tie (ulp 2^-7 at 1) -> 1.0 (even)
    Wu[1, 0] = 2.0 ** -7                    # A1 = 1.0 exactly
    Wu[2, 0] = 1.0 / 128.0                  # A2 = 1.0 (g = 128, u = 2^-7)
    Wd[0, 0] = 3.0                          # Z0 = 3 * bf16(A0) = 3.0
    #   (A0 unrounded: 3 + 3*2^-8 = 3.01171875 -> bf16 (ulp 2^-6 in [2,4)) 3.015625)
    Wd[1, 1] = 1.0 + 2.0 ** -8 + 2.0 ** -10  # Z1 = 1.0048828125 -> bf16 1.0078125 (above the tie 1 + 2^-8)
    #   (Z unrounded: 1.0048828125)
    z = M.expert_ffn_mirrored(x, Wg, Wu, Wd, M.FMT_BF16)
    np.testing.assert_array_equal(z, [[3.0, 1.0078125]])
    # a rounding of A away from zero on ties would give Z0 = 3 * 1.0078125 = 3.0234375 -> 3.03125
    # a truncation of Z would give Z1 = 1.0


def test_bf16_silu_and_A_rounding():
    # g = 1: silu(1) = 1 / (1 + e^-1) = 0.7310585786300049; u = 1 -> A = 0.73105857...
    # bf16 in [0.5, 1) has ulp 2^-8: 0.7310585786 * 256 = 187.151 -> 187 / 256 = 0.73046875
    x = np.array([[1.0]])
    Wg = np.array([[1.0]])
    Wu = np.array([[1.0]])
    Wd = np.array([[1.0], [-2.0]])
    z = M.expert_ffn_mirrored(x, Wg, Wu, Wd, M.FMT_BF16)
    np.testing.assert_array_equal(z, [[0.73046875, -1.4609375]])
    assert abs(1.0 / (1.0 + math.exp(-1.0)) - 0.7310585786300049) < 1e-15


def _fp8_example():
    """One token, H = 256 (two activation groups of 128), I = 128 (one group)."""
    x = _zeros(1, 256)
    x[0, 0] = 448.0            # group 0 amax: scale = 448/448 = 1, inv = 1
    x[0, 1] = 1.0625           # on the E4M3 grid at scale 1: a tie of 1.0 (mantissa 000) and 1.125 -> 1.0
    x[0, 128] = 3.5            # group 1 amax: scale = 3.5/448 = 2^-7, inv = 128
    x[0, 129] = 0.005          # fp32(0.005) * 128 = 0.64 -> E4M3 step 1/16 in [0.5, 1): 0.625 -> 0.625/128
    #                            = 0.0048828125 (one group of 256, scale 1: 0.005 / 2^-9 = 2.56 -> 3 * 2^-9
    #                            = 0.005859375; unquantised 0.005)
    Wg, Wu, Wd = _zeros(128, 256), _zeros(128, 256), _zeros(256, 128)
    Wg[:, 0] = 0.25            # g = 0.25 * 448 = 112 for every feature: silu(112) = 112
    Wu[0, 1] = 1.0             # u0 = 1.0      -> A0 = 112
    Wu[1, 129] = 1024.0        # u1 = 5.0      -> A1 = 560   (one group of 256: 6.0 -> 672; unquantised 5.12)
    Wu[2, 128] = 0.25          # u2 = 0.875    -> A2 = 98
    # A row [112, 560, 98, 0...]: amax 560, scale fp32(560/448) = 1.25, inv = fp32(448/560) = fp32(0.8)
    #   112 * 0.8 = 89.6  -> E4M3 step 8 in [64, 128): 88  -> 88 * 1.25  = 110
    #   560 * 0.8 = 448   -> 448                          -> 448 * 1.25 = 560
    #    98 * 0.8 = 78.4  -> 80                           -> 80 * 1.25  = 100
    # (A unquantised, or quantised per feature over the tokens, stays 112, 560, 98)
    Wd[0, 0] = 1.0             # Z0 = 110
    Wd[1, 1] = 1.0             # Z1 = 560
    Wd[2, 2] = 1.0             # Z2 = 100
    Wd[3, 2] = 1.0 + 2.0 ** -8  # Z3 = 100.390625 -> bf16 (ulp 0.5 in [64, 128)) 100.5
    return x, Wg, Wu, Wd


def test_fp8_groups_quantise_x_and_A_per_row_and_128_columns():
    x, Wg, Wu, Wd = _fp8_example()
    z = M.expert_ffn_mirrored(x, Wg, Wu, Wd, M.FMT_FP8)
    want = np.zeros((1, 256))
    want[0, :4] = [110.0, 560.0, 100.0, 100.5]
    np.testing.assert_array_equal(z, want)


def test_fp8_example_detects_misplaced_rounding():
    """The example's value moves under each plausible mistake (computed with
    the same function on mutated inputs that reproduce the mistake)."""
    x, Wg, Wu, Wd = _fp8_example()
    good = M.expert_ffn_mirrored(x, Wg, Wu, Wd, M.FMT_FP8)
    # x left unquantised: as if x1 = 1.0625 and x129 = 0.005 had passed through
    # unrounded; the bf16 path (no x quantisation) on the same weights differs
    assert not np.array_equal(good, M.expert_ffn_mirrored(x, Wg, Wu, Wd, M.FMT_BF16))
    # x quantised as one group of 256 (group 1 shares group 0's amax 448)
    xg = x.copy()
    xg[0, 129] = 0.005859375
    xg[0, 1] = 1.0
    zg = M.round_to_bf16(M.mirror_quant_fp8_groups(M.silu(xg @ Wg.T) * (xg @ Wu.T), 128) @ Wd.T)
    assert not np.array_equal(good, zg)


def test_mxfp8_quantises_per_32_columns_with_power_of_two_scales():
    """MXFP4 weights' activations: E4M3 per 32 columns, E8M0 scale
    2^(floor(log2 amax) - 8).  H = 64 (two blocks), I = 32 (one block)."""
    x = _zeros(1, 64)
    x[0, 0] = 1.5              # block 0 amax: floor(log2 1.5) = 0 -> scale 2^-8; 1.5 * 256 = 384 (on the grid)
    x[0, 1] = 0.03125 + 2.0 ** -9   # * 256 = 8.5 -> E4M3 step 1 in [8, 16): tie of 8 and 9 -> 8 (even) -> 1/32
    x[0, 32] = 7.0             # block 1 amax: floor(log2 7) = 2 -> scale 2^-6; 7 * 64 = 448
    x[0, 33] = 0.5 + 2.0 ** -6 + 2.0 ** -7  # * 64 = 33.5 -> E4M3 step 4 in [32, 64): 32 -> 0.5
    Wg, Wu, Wd = _zeros(32, 64), _zeros(32, 64), _zeros(64, 32)
    Wg[:, 32] = 8.0            # g = 56 for every feature: silu(56) = 56
    Wu[0, 1] = 64.0            # u0 = 2.0  -> A0 = 112   (ties away from zero: 9/256 * 64 = 2.25 -> 126)
    Wu[1, 33] = 3.0            # u1 = 1.5  -> A1 = 84
    Wu[2, 0] = 1.0             # u2 = 1.5  -> A2 = 84
    # A row [112, 84, 84, 0...]: amax 112, floor(log2 112) = 6 -> scale 2^-2
    #   112 * 4 = 448 -> 448 -> 112;  84 * 4 = 336 -> E4M3 step 32 in [256, 448]: 320 or 352, 336 is a
    #   tie -> 320 (mantissa 010, even) -> 80
    Wd[0, 0] = 1.0             # Z0 = 112
    Wd[1, 1] = 1.0             # Z1 = 80
    Wd[2, 2] = 0.5             # Z2 = 40
    z = M.expert_ffn_mirrored(x, Wg, Wu, Wd, M.FMT_MXFP4)
    want = np.zeros((1, 64))
    want[0, :3] = [112.0, 80.0, 40.0]
    np.testing.assert_array_equal(z, want)


def test_nvfp4_rounds_x_and_A_to_binary16():
    """NVFP4's 16-bit path: x and A rounded to IEEE binary16 (ties to even),
    Z to bf16."""
    # fp16: 1 + 2^-11 is a tie -> 1.0 (ulp 2^-10); 2^-25 is half the smallest subnormal 2^-24, a tie -> 0
    x = np.array([[1.0 + 2.0 ** -11, 2.0 ** -25]])
    Wg = np.array([[64.0, 0.0], [64.0, 0.0]])      # g = 64 (x0 rounded) -> silu = 64
    Wu = np.array([[2.0 ** -6, 0.0], [0.0, 2.0 ** 30]])
    # u0 = 2^-6 -> A0 = 1.0;  u1 = 2^30 * fp16(2^-25) = 0 -> A1 = 0 (with x1 unrounded: 32 -> A1 = 2048)
    Wd = np.array([[1.0 + 2.0 ** -11, 0.0], [0.0, 1.0]])
    # Z0 = 1 + 2^-11 -> bf16 1.0;  Z1 = 0
    z = M.expert_ffn_mirrored(x, Wg, Wu, Wd, M.FMT_NVFP4)
    np.testing.assert_array_equal(z, [[1.0, 0.0]])
    # x0 unrounded would make g = 64 + 2^-5 and A0 = (64 + 2^-5) * 2^-6 = 1 + 2^-11 -> fp16 tie -> 1.0;
    # the pin on x therefore rests on x1 (rounded to zero)
