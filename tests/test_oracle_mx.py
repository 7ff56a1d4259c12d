"""Pins of the oracle's block-wise FP8 (power-of-two block scales).

The block exponent against brute force and its edge values, the codes against
the half-step quantization bound, the reduction to per-channel / per-token
quantization when every block of a row has the row's absmax and that absmax is
448 times a power of two, and the block product against exact rationals.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from oracle import formats as F
from w8a8_gemm_rl_amd import inputs as I


def test_block_exponent_is_the_smallest_without_saturation():
    rng = np.random.default_rng(0)
    a = np.concatenate([
        np.abs(rng.standard_normal(2000) * 10.0 ** rng.uniform(-30, 30, 2000)),
        448.0 * 2.0 ** np.arange(-120, 120),                       # exact boundaries
        np.nextafter(448.0 * 2.0 ** np.arange(-20, 20), np.inf),   # just above
        np.nextafter(448.0 * 2.0 ** np.arange(-20, 20), 0),        # just below
    ]).astype(np.float32).astype(np.float64)
    X = O.mx_exponent(a).astype(np.int64)
    inside = (X > -127) & (X < 127)
    for ai, xi in zip(a[inside], X[inside]):
        assert Fraction(ai) <= 448 * Fraction(2) ** int(xi)
        assert Fraction(ai) > 448 * Fraction(2) ** int(xi - 1)
    assert O.mx_exponent(0.0) == -127
    assert O.mx_exponent(448.0) == 0 and O.mx_exponent(448.00003) == 1 and O.mx_exponent(224.0) == -1


def test_codes_within_half_a_step_and_block_layout():
    A = I.activations(6, 256, seed=1, kind="heavy")
    Af = F.bf16_bits_to_f32(A)
    codes, X = O.mx_quantize_rows(Af)
    assert codes.shape == (6, 256) and X.shape == (6, 8)
    dec = F.e4m3fn_decode(codes) * np.repeat(2.0 ** X.astype(np.float64), 32, axis=1)
    # E4M3FN spacing at |v| 2^-X is at most 2^(e-3); half of it bounds the error
    v = Af.astype(np.float64)
    scaled = np.abs(v) * np.repeat(2.0 ** -X.astype(np.float64), 32, axis=1)
    step = np.where(scaled < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(scaled, 1e-300))) - 3))
    assert np.all(np.abs(dec - v) <= 0.5 * step * np.repeat(2.0 ** X.astype(np.float64), 32, axis=1) + 1e-300)
    # every block's absmax reaches at least half the E4M3 range (no wasted exponent)
    bmax = np.abs(Af).reshape(6, 8, 32).max(axis=2)
    assert np.all((bmax == 0) | (bmax * 2.0 ** -X.astype(np.float64) > 224.0))


def test_reduces_to_per_channel_when_blocks_share_a_power_of_two_absmax():
    """Rows whose every block has absmax 448 * 2^X_row: the block scales are all
    2^X_row, the per-channel fp32 scale is exactly 2^X_row, and the codes agree."""
    rng = np.random.default_rng(2)
    R, K = 8, 128
    Xr = rng.integers(-20, 20, size=R)
    A = rng.uniform(-1, 1, size=(R, K)) * 448.0
    A[:, ::32] = 448.0  # each block's absmax
    A = (A * 2.0 ** Xr[:, None]).astype(np.float32)
    codes, X = O.mx_quantize_rows(A)
    assert np.all(X == Xr[:, None])
    pc_codes, pc_scale = O.quantize_rows(A, "fp8")
    assert np.array_equal(pc_scale, (2.0 ** Xr).astype(np.float32))
    assert np.array_equal(codes, pc_codes.view(np.uint8))


def test_block_product_against_exact_rationals():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((3, 64)) * 5).astype(np.float32)
    w = (rng.standard_normal((4, 64)) * 0.02).astype(np.float32)
    xc, xe = O.mx_quantize_rows(x)
    wc, we = O.mx_quantize_rows(w)
    acc, y = O.mx_linear(xc, xe, wc, we)
    xd, wd = F.e4m3fn_decode(xc), F.e4m3fn_decode(wc)
    for m in range(3):
        for n in range(4):
            ex = sum(Fraction(float(xd[m, k])) * Fraction(float(wd[n, k]))
                     * Fraction(2) ** int(xe[m, k // 32] + we[n, k // 32]) for k in range(64))
            assert Fraction(acc[m, n]) == ex
    # and the product approximates the float product within the two quantizations
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.allclose(acc, ref, rtol=0.15, atol=0.05 * np.abs(ref).max())


def test_zero_blocks_and_bad_width():
    A = np.zeros((2, 64), np.float32)
    A[1, 32:] = 3.0
    codes, X = O.mx_quantize_rows(A)
    assert np.all(X[0] == -127) and X[1, 0] == -127 and not codes[0].any()
    with pytest.raises(ValueError):
        O.mx_quantize_rows(np.zeros((1, 48), np.float32))
