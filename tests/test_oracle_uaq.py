"""Pins for the oracle's UAQ reparameterization and the update-masking experiment.

What the pages fix (QuRL paper notes, "Key designs > UAQ"): the linear is
invariant under W X = (W/s)(s X); the quantization step shrinks by s; the update
on the stored parameter grows by s, an s^2 gain; with updates ~1e-7 INT8
quantization hides nearly every update. Checked here with exact rational
arithmetic, closed forms and brute-force code-flip counts.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from oracle import formats as F
from w8a8_gemm_rl_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _pages():
    with open(os.path.join(GOLDEN, "pages_constants.json")) as f:
        return json.load(f)


def _frac_matrix(g, shape, den=97):
    return np.array([[Fraction(int(v), den) for v in row]
                     for row in g.integers(-500, 500, shape)], dtype=object)


def test_invariance_exact_rational_norm_fed():
    """RMSNorm-fed linear: (x * gamma') @ W'^T == (x * gamma) @ W^T exactly, s = 3/2."""
    g = np.random.default_rng(20)
    W = _frac_matrix(g, (6, 8))
    x = _frac_matrix(g, (3, 8))
    gamma = _frac_matrix(g, (1, 8))[0]
    beta = _frac_matrix(g, (1, 8))[0]
    s = Fraction(3, 2)
    assert s == Fraction(_pages()["uaq_s"]["value"])
    Wp, gp, bp = O.uaq_reparameterize(W, s, gamma, beta)
    ref = (x * gamma[None, :]) @ W.T
    got = (x * gp[None, :]) @ Wp.T
    assert np.all(ref == got)
    # LayerNorm with a bias: (x*gamma + beta) feeds W
    ref_b = (x * gamma[None, :] + beta[None, :]) @ W.T
    got_b = (x * gp[None, :] + bp[None, :]) @ Wp.T
    assert np.all(ref_b == got_b)
    # a fold in the other direction (gamma / s) would not be invariant
    wrong = (x * (gamma / s)[None, :]) @ Wp.T
    assert not np.all(wrong == ref)


def test_invariance_exact_rational_activation_side():
    """Linear without a norm: (W/s)(s x) == W x, the activation side carried by s."""
    g = np.random.default_rng(21)
    W = _frac_matrix(g, (5, 7))
    x = _frac_matrix(g, (4, 7))
    s = Fraction(3, 2)
    Wp, _, _ = O.uaq_reparameterize(W, s)
    assert np.all((x * s) @ Wp.T == x @ W.T)


def test_step_shrinks_by_s_exact_and_fp32():
    """scale(W/s) == scale(W)/s exactly in rationals; within 2 ulp in fp32."""
    s = 1.5
    W = I.weights(64, 512, 0.02, seed=22)
    # rational: absmax is homogeneous
    Wr = np.array([[Fraction(float(v)) for v in row] for row in W[:4]], dtype=object)
    Wpr, _, _ = O.uaq_reparameterize(Wr, Fraction(s))
    for r in range(4):
        a = max(abs(v) for v in Wr[r])
        ap = max(abs(v) for v in Wpr[r])
        assert ap / 127 == (a / 127) / Fraction(s)
    # fp32: the oracle's scales
    sw = O.quantize_weights_uaq(W, 1.0, "int8")["scale_w"]
    sws = O.quantize_weights_uaq(W, s, "int8")["scale_w"]
    ratio = sws.astype(np.float64) * s / sw.astype(np.float64)
    assert np.all(np.abs(ratio - 1) <= 2 * 2.0 ** -23 * 2)


@pytest.mark.parametrize("qt", ["int8", "fp8"])
def test_codes_invariant_under_uaq_except_fp32_ties(qt):
    """In real arithmetic codes(W/s) == codes(W); fp32 rounding moves only rare near-ties."""
    W = I.weights(512, 512, 0.02, seed=23)
    c1 = O.quantize_weights_uaq(W, 1.0, qt)["Wq"]
    c2 = O.quantize_weights_uaq(W, 1.5, qt)["Wq"]
    assert np.count_nonzero(c1 != c2) <= 5


def test_quantized_linear_invariant_under_uaq():
    """The quantized forward pass is (nearly) unchanged by UAQ: near-zero overhead."""
    cfg = I.SINGLE
    X = I.activations(cfg["M"], cfg["K"], seed=0)
    W = I.weights(cfg["N"], cfg["K"], cfg["w_sigma"], seed=1)
    a = O.quantize_weights_uaq(W, 1.0, "int8")
    b = O.quantize_weights_uaq(W, 1.5, "int8")
    ya = F.bf16_bits_to_f32(O.w8a8_linear(X, a["Wq"], a["scale_w"], 1.0, "int8")["y"])
    yb = F.bf16_bits_to_f32(O.w8a8_linear(X, b["Wq"], b["scale_w"], 1.5, "int8")["y"])
    rel = np.abs(ya - yb) / np.maximum(np.abs(ya), 1e-3)
    assert np.percentile(rel, 99) <= 2 ** -7
    assert np.linalg.norm(ya - yb) <= 4e-3 * np.linalg.norm(ya)


def test_update_size_from_pages():
    p = _pages()
    lr = p["rl_learning_rate"]["value"]
    g_lo, g_hi = p["rl_gradient_range"]["value"]
    assert lr * g_lo == pytest.approx(p["weight_update_size"]["value"])
    assert I.DW_SIGMA == p["weight_update_size"]["value"] and lr * g_hi <= 1e-6


def _flip_totals(qt, shape, seeds, s=1.5, sigma=I.DW_SIGMA):
    tot = {"base": 0, "uaq_same": 0, "uaq_pages": 0, "control": 0, "n": 0}
    exp = {"base": 0.0, "uaq_same": 0.0, "uaq_pages": 0.0, "control": 0.0}
    for sd in seeds:
        W = I.weights(shape[0], shape[1], 0.02, seed=sd)
        dW = I.normal_f32(shape, sigma, seed=10_000 + sd)
        c = O.flip_counts(W, dW, s, qt)
        for k in tot:
            tot[k] += c[k]
        Ws = (W / np.float32(s)).astype(np.float32)
        exp["base"] += O.flip_expectation(W, sigma, qt)
        exp["uaq_same"] += O.flip_expectation(Ws, sigma, qt)
        exp["uaq_pages"] += O.flip_expectation(Ws, sigma * s, qt)
        exp["control"] += O.flip_expectation(Ws, sigma / s, qt)
    return tot, exp


def test_flip_count_brute_force_tiny_int8_more_flips_with_uaq():
    """Brute-force count on tiny matrices: more INT8 codes flip under a 1e-7 update with s=1.5."""
    tot, exp = _flip_totals("int8", (64, 512), seeds=range(32))
    # masking: almost every update is invisible to INT8 codes
    assert tot["base"] / tot["n"] < 1e-3
    assert tot["uaq_same"] > tot["base"] and tot["uaq_pages"] > tot["base"]
    for k in ("base", "uaq_same", "uaq_pages", "control"):
        e = exp[k]
        assert abs(tot[k] - e) <= 5 * np.sqrt(e) + 0.05 * e, (k, tot[k], e)


@pytest.mark.slow
@pytest.mark.parametrize("qt", ["int8", "fp8"])
def test_flip_ratios_follow_s_and_s_squared(qt):
    """Aggregated counts: same-size update ~ s x base, s*dW update ~ s^2 x base, control ~ 1 x."""
    tot, exp = _flip_totals(qt, (512, 512), seeds=range(8))
    s = 1.5
    b = tot["base"]
    assert b > 200
    assert tot["uaq_same"] / b == pytest.approx(s, rel=0.15)
    assert tot["uaq_pages"] / b == pytest.approx(s * s, rel=0.15)
    assert tot["control"] / b == pytest.approx(1.0, rel=0.15)
    for k in ("base", "uaq_same", "uaq_pages", "control"):
        e = exp[k]
        assert abs(tot[k] - e) <= 5 * np.sqrt(e) + 0.05 * e, (k, tot[k], e)


def test_flip_expectation_closed_form_special_case():
    """One row, all |w| equal except the absmax: INT8 step = a/127, p = sqrt(2/pi) sigma sqrt(127^2+v^2)/a."""
    a = 0.05
    W = np.full((1, 4), 0.01, np.float64)
    W[0, 0] = a
    sigma = 1e-7
    v = 0.01 / (a / 127)
    p = np.sqrt(2 / np.pi) * sigma * np.sqrt((127 / a) ** 2 + (v / a) ** 2)
    assert O.flip_expectation(W, sigma, "int8") == pytest.approx(3 * p, rel=1e-12)


# ------------------------------------------------- per-step refresh and flip counting

def test_count_flips_special_cases():
    rng = np.random.default_rng(3)
    a = rng.integers(-127, 128, size=1000, dtype=np.int64).astype(np.int8)
    assert O.count_flips(a, a, "int8") == 0
    b = a.copy()
    b[[5, 17, 999]] += 1
    b[[5, 17, 999]] = np.where(b[[5, 17, 999]] == a[[5, 17, 999]], b[[5, 17, 999]] - 2, b[[5, 17, 999]])
    assert O.count_flips(a, b, "int8") == 3
    # INT8: byte 0x80 (-128) is a different value from 0 (it is never produced, but if present it counts)
    assert O.count_flips(np.array([0], np.int8), np.array([-128], np.int8), "int8") == 1
    # FP8: +0 and -0 are one value; every other byte change is a change of value
    assert O.count_flips(np.array([0x00, 0x80, 0x01], np.uint8),
                         np.array([0x80, 0x00, 0x81], np.uint8), "fp8") == 1


def test_count_flips_fp8_matches_decoded_values_for_every_pair():
    """Exhaustive over all pairs of finite E4M3FN bytes: a flip is a change of decoded value."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)  # drop the NaNs
    a = np.repeat(codes, codes.size)
    b = np.tile(codes, codes.size)
    expect = int(np.count_nonzero(F.e4m3fn_decode(a) != F.e4m3fn_decode(b)))
    assert O.count_flips(a, b, "fp8") == expect
    # brute force on a random sample against a plain Python loop over values
    rng = np.random.default_rng(4)
    x = rng.choice(codes, 4000)
    y = rng.choice(codes, 4000)
    loop = sum(1 for u, v in zip(x.tolist(), y.tolist())
               if float(F.e4m3fn_decode(np.array([u], np.uint8))[0])
               != float(F.e4m3fn_decode(np.array([v], np.uint8))[0]))
    assert O.count_flips(x, y, "fp8") == loop


@pytest.mark.parametrize("qt", ["int8", "fp8"])
def test_requantize_weights_is_quantize_rows_plus_count(qt):
    Wp = I.weights(48, 256, 0.02, seed=7)
    c0, s0, f0 = O.requantize_weights(Wp, qt)
    assert f0 is None
    rc, rs = O.quantize_rows(Wp, qt)
    assert np.array_equal(c0.view(np.uint8), rc.view(np.uint8)) and np.array_equal(s0, rs)
    # an update far below one step changes few codes; the refresh counts exactly those
    Wn = (Wp + I.normal_f32(Wp.shape, 1e-4, seed=8)).astype(np.float32)
    c1, s1, f1 = O.requantize_weights(Wn, qt, c0)
    assert f1.shape == (48,) and f1.sum() == O.count_flips(c0, c1, qt) and 0 < f1.sum() < c0.size // 4
    assert all(f1[r] == O.count_flips(c0[r], c1[r], qt) for r in range(48))
    assert all(f1[r] == sum(int(x) != int(y) for x, y in zip(c0[r], c1[r])) for r in range(0, 48, 7))
    # s = 1 requantization of W' equals the UAQ quantizer's codes of W with W' = fl32(W / s)
    W = I.weights(16, 128, 0.02, seed=9)
    ref = O.quantize_weights_uaq(W, 1.5, qt)
    c2, s2, _ = O.requantize_weights(ref["W_scaled"], qt)
    assert np.array_equal(c2.view(np.uint8), ref["Wq"].view(np.uint8))
    assert np.array_equal(s2, ref["scale_w"])
