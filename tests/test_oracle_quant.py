"""Pins for the oracle's quantizers, accumulators and epilogue.

Each check is independent of the code it pins: brute-force search over every
code, special cases whose answer is known in closed form, a pure-Python triple
loop, torch's CPU integer / FP8 matrix products, and an a-priori error bound
against the unquantized float64 product (which a dropped term, a wrong sign,
a swapped scale or a transposed operand would break).
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from oracle import formats as F
from w8a8_gemm_rl_amd import inputs as I


# ---------------------------------------------------------------- quantizers

def _all_codes(qt):
    if qt == "int8":
        c = np.arange(-127, 128)
        return c.astype(np.int8), c.astype(np.float64)
    c = np.arange(256, dtype=np.uint8)
    v = F.e4m3fn_decode(c)
    keep = ~np.isnan(v)
    return c[keep], v[keep]


@pytest.mark.parametrize("qt", ["int8", "fp8"])
def test_quantize_rows_picks_nearest_code_by_search(qt):
    A = I.normal_f32((24, 96), 0.05, seed=11)
    A[3] = 0.0
    codes, scale = O.quantize_rows(A, qt)
    Q = O.QMAX[qt]
    cands, cvals = _all_codes(qt)
    for r in range(A.shape[0]):
        if scale[r] == 0:
            assert np.all(codes[r].view(np.uint8) == 0)
            continue
        # scale is the fp32 quotient absmax / Q
        assert scale[r] == np.float32(np.float32(np.abs(A[r]).max()) / np.float32(Q))
        v = (A[r] / scale[r]).astype(np.float32).astype(np.float64)
        v = np.clip(v, -Q, Q)
        dist = np.abs(v[:, None] - cvals[None, :])
        best = dist.min(axis=1)
        got = cvals[np.searchsorted(cands, codes[r])] if qt == "int8" else \
            F.e4m3fn_decode(codes[r])
        assert np.array_equal(np.abs(got - v), best)


@pytest.mark.parametrize("qt", ["int8", "fp8"])
def test_quantize_rows_special_cases(qt):
    Q = O.QMAX[qt]
    A = np.zeros((5, 64), np.float32)
    A[0] = 0.37                       # constant row -> all +Q
    A[1, 7] = -2.5                    # one-hot -> a single -Q, rest 0
    A[2] = np.linspace(-1, 1, 64, dtype=np.float32)
    A[4, :] = -1e-3
    A[4, 10] = 4e-3                   # absmax element positive
    codes, scale = O.quantize_rows(A, qt)
    dec = (codes.astype(np.float64) if qt == "int8" else F.e4m3fn_decode(codes))
    assert np.all(dec[0] == Q)
    assert dec[1, 7] == -Q and np.count_nonzero(dec[1]) == 1
    assert dec[2, 0] == -Q and dec[2, -1] == Q
    assert scale[3] == 0 and np.all(codes[3].view(np.uint8) == 0)
    assert dec[4, 10] == Q
    if qt == "int8":
        assert np.all(dec[4, np.arange(64) != 10] == np.rint(-Q / 4))  # -31.75 -> -32
        assert codes.min() >= -127  # -128 never produced


@pytest.mark.parametrize("qt", ["int8", "fp8"])
def test_dequantized_error_bound(qt):
    A = I.normal_f32((32, 256), 0.02, seed=12)
    codes, scale = O.quantize_rows(A, qt)
    dec = codes.astype(np.float64) if qt == "int8" else F.e4m3fn_decode(codes)
    err = np.abs(dec * scale[:, None].astype(np.float64) - A)
    if qt == "int8":
        bound = 0.5 * scale[:, None] * (1 + 1e-5)
    else:
        # half a code step at the element's binade, or half the subnormal step
        bound = np.maximum(np.abs(A) * 2.0 ** -4, 2.0 ** -10 * scale[:, None]) * (1 + 1e-5)
    assert np.all(err <= bound)


def test_act_quant_scale_carries_act_mult_only():
    X = I.activations(8, 128, seed=13)
    c1, s1 = O.quantize_act_per_token(X, 1.0, "int8")
    c2, s2 = O.quantize_act_per_token(X, 1.5, "int8")
    assert np.array_equal(c1, c2)
    assert np.array_equal(s2, (s1 * np.float32(1.5)).astype(np.float32))


# ---------------------------------------------------------------- accumulators

def test_acc_int8_matches_triple_loop():
    g = np.random.default_rng(14)
    Xq = g.integers(-127, 128, (3, 40)).astype(np.int8)
    Wq = g.integers(-127, 128, (5, 40)).astype(np.int8)
    acc = O.acc_int8(Xq, Wq)
    for m in range(3):
        for n in range(5):
            s = 0
            for k in range(40):
                s += int(Xq[m, k]) * int(Wq[n, k])
            assert acc[m, n] == s


def test_acc_int8_matches_torch_int_mm():
    g = np.random.default_rng(15)
    Xq = g.integers(-127, 128, (48, 512)).astype(np.int8)
    Wq = g.integers(-127, 128, (80, 512)).astype(np.int8)
    ref = torch._int_mm(torch.from_numpy(Xq), torch.from_numpy(Wq).t().contiguous()).numpy()
    assert np.array_equal(O.acc_int8(Xq, Wq), ref)


def test_acc_int8_extremes_no_overflow():
    K = 27648
    Xq = np.full((2, K), 127, np.int8)
    Xq[1] = -127
    Wq = np.full((3, K), 127, np.int8)
    Wq[2] = -127
    acc = O.acc_int8(Xq, Wq)
    assert acc[0, 0] == K * 127 * 127 and acc[1, 0] == -K * 127 * 127
    assert acc[1, 2] == K * 127 * 127
    assert acc.dtype == np.int32


def test_acc_fp8_exact_by_fractions_and_torch():
    g = np.random.default_rng(16)
    x = g.standard_normal((4, 64)).astype(np.float32) * 20
    w = g.standard_normal((6, 64)).astype(np.float32) * 20
    Xq = F.e4m3fn_encode(np.clip(x, -448, 448))
    Wq = F.e4m3fn_encode(np.clip(w, -448, 448))
    acc = O.acc_fp8(Xq, Wq)
    dx, dw = F.e4m3fn_decode(Xq), F.e4m3fn_decode(Wq)
    for m in range(4):
        for n in range(6):
            exact = sum(Fraction(float(dx[m, k])) * Fraction(float(dw[n, k])) for k in range(64))
            assert Fraction(float(acc[m, n])) == exact
    # torch's CPU FP8 product (fp32 accumulation) agrees within the fp32 bound
    tx = torch.from_numpy(Xq).view(torch.float8_e4m3fn)
    tw = torch.from_numpy(Wq).view(torch.float8_e4m3fn)
    one = torch.tensor(1.0)
    ref = torch._scaled_mm(tx, tw.t(), scale_a=one, scale_b=one, out_dtype=torch.float32).double().numpy()
    bound = 63 * 2.0 ** -24 * (np.abs(dx) @ np.abs(dw).T)
    assert np.all(np.abs(ref - acc) <= bound)


def test_acc_fp8_all_max_codes():
    K = 5120
    Xq = np.full((1, K), 0x7E, np.uint8)
    Wq = np.full((2, K), 0x7E, np.uint8)
    Wq[1] = 0xFE
    acc = O.acc_fp8(Xq, Wq)
    assert acc[0, 0] == K * 448.0 * 448.0 and acc[0, 1] == -K * 448.0 * 448.0


# ---------------------------------------------------------------- epilogue

def test_epilogue_identity_and_torch_crosscheck():
    acc = np.array([[0, 1, -3, 200]], np.int32)
    y, b = O.dequant_epilogue(acc, np.float32([1.0]), np.float32([1, 1, 1, 1]))
    assert np.array_equal(y, acc.astype(np.float32))
    g = np.random.default_rng(17)
    acc = g.integers(-2 ** 30, 2 ** 30, (16, 64)).astype(np.int32)
    sx = (g.random(16) * 1e-2).astype(np.float32)
    sw = (g.random(64) * 1e-3).astype(np.float32)
    y, b = O.dequant_epilogue(acc, sx, sw)
    ta = torch.from_numpy(acc).double().float()
    ty = (ta * torch.from_numpy(sx)[:, None]) * torch.from_numpy(sw)[None, :]
    assert np.array_equal(y, ty.numpy())
    assert np.array_equal(b, ty.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


# ---------------------------------------------------------------- whole linear

@pytest.mark.parametrize("qt", ["int8", "fp8"])
def test_linear_error_bound_vs_float_product(qt):
    """End-to-end bound against the unquantized product of X and the effective weight.

    With x_k = dx_k + ex_k and w_k = dw_k + ew_k (decoded value plus error):
    |sum x w - sum dx dw| <= sum |ex||dw| + sum |dx||ew| + sum |ex||ew|, with
    the per-element error bounds of test_dequantized_error_bound; the bf16
    rounding adds 2^-8 relative. Square weights make a transposed operand fail.
    """
    cfg = I.SINGLE
    M, N, K, s = cfg["M"], cfg["N"], cfg["K"], cfg["s"]
    X = I.activations(M, K, seed=0)
    W = I.weights(N, K, cfg["w_sigma"], seed=1)
    wq = O.quantize_weights_uaq(W, s, qt)
    r = O.w8a8_linear(X, wq["Wq"], wq["scale_w"], s, qt)
    x = F.bf16_bits_to_f32(X).astype(np.float64)
    weff = wq["W_scaled"].astype(np.float64) * s  # (W/s) * s
    exact = x @ weff.T
    if qt == "int8":
        dx = r["Xq"].astype(np.float64) * (r["scale_x"][:, None] / s)
        dw = wq["Wq"].astype(np.float64) * wq["scale_w"][:, None] * s
        ex = 0.5 * (r["scale_x"] / s)[:, None] * np.ones_like(x)
        ew = 0.5 * (wq["scale_w"] * s)[:, None] * np.ones_like(weff)
    else:
        dx = F.e4m3fn_decode(r["Xq"]) * (r["scale_x"][:, None] / s)
        dw = F.e4m3fn_decode(wq["Wq"]) * wq["scale_w"][:, None] * s
        ex = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * (r["scale_x"] / s)[:, None])
        ew = np.maximum(np.abs(weff) * 2.0 ** -4, 2.0 ** -10 * (wq["scale_w"] * s)[:, None])
    bound = ex @ np.abs(dw).T + np.abs(dx) @ ew.T + ex @ ew.T
    bound = bound * (1 + 1e-4) + np.abs(exact) * 2.0 ** -8 + 1e-6
    y = F.bf16_bits_to_f32(r["y"]).astype(np.float64)
    assert np.all(np.abs(y - exact) <= bound + np.abs(exact) * 2e-6)
    # and the bound is not vacuous: errors are a small fraction of the outputs
    assert np.linalg.norm(y - exact) < 0.05 * np.linalg.norm(exact)


def test_linear_matches_torch_pipeline_int8():
    """Quantize -> int matmul -> scales -> bf16 with torch CPU ops instead of numpy."""
    X = I.activations(16, 512, seed=0)
    W = I.weights(512, 512, 0.02, seed=1)
    wq = O.quantize_weights_uaq(W, 1.5, "int8")
    r = O.w8a8_linear(X, wq["Wq"], wq["scale_w"], 1.5, "int8")
    tx = torch.from_numpy(X.view(np.int16)).view(torch.bfloat16).float()
    a = tx.abs().amax(dim=1)
    sc = a / 127.0
    q = torch.round(tx / sc[:, None]).clamp(-127, 127).to(torch.int8)
    assert np.array_equal(q.numpy(), r["Xq"])
    acc = torch._int_mm(q, torch.from_numpy(wq["Wq"]).t().contiguous())
    assert np.array_equal(acc.numpy(), r["acc"])
    sx = sc * 1.5
    y = (acc.double().float() * sx[:, None]) * torch.from_numpy(wq["scale_w"])[None, :]
    assert np.array_equal(y.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16), r["y"])


def _torch_linear_int8(x_bits, Wq, scale_w, act_mult):
    """Per-token INT8 linear with torch CPU ops (as above); bf16 bits out."""
    tx = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).float()
    sc = tx.abs().amax(dim=1) / 127.0
    q = torch.round(tx / sc[:, None]).clamp(-127, 127).to(torch.int8)
    acc = torch._int_mm(q, torch.from_numpy(Wq).t().contiguous())
    y = (acc.double().float() * (sc * act_mult)[:, None]) * torch.from_numpy(scale_w)[None, :]
    return y.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_decode_chain_wiring_matches_torch_pipeline():
    """A chain whose linears read the layer input, an earlier output and a
    column slice of one: every output equals the torch pipeline fed the same
    way, so a wrong source or slice fails. Token count and sizes are
    multiples of 8 (torch's int matmul needs them)."""
    M = 16
    x0 = I.activations(M, 32, seed=3, kind="outliers")
    spec = [("a", "x0", None, 48, 32), ("b", "a", (8, 32), 24, 24), ("c", "a", None, 16, 48),
            ("d", "b", None, 40, 24)]
    layers, ref = [], {}
    for i, (name, src, cols, N, K) in enumerate(spec):
        wq = O.quantize_weights_uaq(I.weights(N, K, 0.05, seed=10 + i), 1.5, "int8")
        layers.append(dict(name=name, src=src, cols=cols, Wq=wq["Wq"], scale_w=wq["scale_w"],
                           act_mult=1.5))
        inp = x0 if src == "x0" else ref[src]
        if cols is not None:
            inp = inp[:, cols[0]:cols[1]]
        ref[name] = _torch_linear_int8(inp, wq["Wq"], wq["scale_w"], 1.5)
    got = O.decode_chain(x0, layers, "int8")
    for name in ref:
        assert np.array_equal(got[name]["y"], ref[name]), name
    # the slice matters: feeding b the whole of a's first 24 columns differs
    alt = _torch_linear_int8(ref["a"][:, :24], layers[1]["Wq"], layers[1]["scale_w"], 1.5)
    assert not np.array_equal(alt, ref["b"])
