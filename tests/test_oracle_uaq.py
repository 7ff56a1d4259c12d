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
