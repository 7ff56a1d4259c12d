"""Parity at the workloads' full sizes, in the launch plans the benchmark uses.

The device always runs the full-size shapes. The oracle computes what it can
in seconds:
* 7B-shaped decode layer, INT8, M = 256 (outlier activations): the whole
  device chain against the whole oracle chain, every element, bit for bit.
* The same 7B linears in FP8 at M in {1, 32, 256}, and the seven 32B linears
  in FP8 at M = 512: 512 sampled output channels per matrix. A channel's codes
  and scale depend only on its own weight row, and its outputs only on those
  and the activations, so the oracle quantizes just the sampled rows.
* 32B-shaped batched decode layer (seven linears, or five with q, k and v
  stacked into one projection; the stacked one also in FP8 on sampled
  channels), INT8, M = 512, and 32B
  prefill, INT8, M = 4096 (heavy-tailed channels): the device chain runs at
  full size; sampled tokens are computed by the oracle chain from the same
  input rows (quantization is per token, so a token's outputs depend only on
  its own row) and compared bit for bit. INT8 weight codes and scales are
  compared in full.
* Per-RL-step weight refresh of the 7B-shaped O, stacked gate+up and down
  matrices, and of the 32B-shaped O and down (both row lengths of each
  stack), after one update of the pages' size: codes, scales and the flip
  count against the oracle in full, and the count against the closed-form
  first-order expectation.
* The update-masking experiment on the five 7B matrices, INT8 and FP8:
  codes changed by one update without UAQ and under the three readings of
  where it lands with UAQ, counted by the refresh kernel, equal to the
  oracle's counts and within the closed form's band.
"""

import numpy as np
import pytest
import torch

import oracle as O
from w8a8_gemm_rl_amd import binding as B
from w8a8_gemm_rl_amd import inputs as I

from gpu_helpers import assert_bf16_close, bf16_np, codes_np, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu

_NAMES = ["qkv", "q", "k", "v", "o", "gate", "up", "down"]
_wcache = {}


def _weights(tag, name, N, K, sigma, idx):
    """Seeded fp32 master weights, cached across tests of one workload family."""
    key = (tag, name, idx)
    if key not in _wcache:
        _wcache[key] = I.weights(N, K, sigma, seed=I.matrix_seed(idx, _NAMES.index(name)))
    return _wcache[key]


def _sample(n_total, n, seed):
    r = np.sort(np.random.default_rng(seed).choice(n_total, min(n, n_total), replace=False))
    r[0], r[-1] = 0, n_total - 1
    return np.unique(r)


def _quant_full_int8(W, s=I.UAQ_S):
    ref = O.quantize_weights_uaq(W, s, "int8")
    Wq, sw = B.quantize_weights_uaq(to_dev_f32(W), s, "int8")
    torch.cuda.synchronize()
    assert np.array_equal(codes_np(Wq), ref["Wq"].view(np.uint8))
    assert np.array_equal(sw.cpu().numpy(), ref["scale_w"])
    return ref, (Wq, sw)


def _device_chain(chain, x0_bits, Wdev, qt, s=I.UAQ_S):
    outs = {}
    X0 = to_dev_bf16(x0_bits)
    for L in chain:
        src = X0 if L["src"] == "x0" else outs[L["src"]]
        if L["cols"] is not None:
            src = src[:, L["cols"][0]:L["cols"][1]]
        outs[L["name"]] = B.linear_fused(src, s, *Wdev[L["name"]], qt)
    torch.cuda.synchronize()
    return {k: bf16_np(v) for k, v in outs.items()}


def _int8_chain(tag, idx, chain, shapes, sigma, M, kind, n_tokens):
    qt = "int8"
    K0 = shapes[chain[0]["name"]][1]
    x0 = I.activations(M, K0, seed=I.matrix_seed(idx, 0), kind=kind)
    Wdev, layers = {}, []
    for L in chain:
        N, K = shapes[L["name"]]
        ref, dev = _quant_full_int8(_weights(tag, L["name"], N, K, sigma, idx))
        Wdev[L["name"]] = dev
        layers.append(dict(L, Wq=ref["Wq"], scale_w=ref["scale_w"], act_mult=I.UAQ_S))
    got = _device_chain(chain, x0, Wdev, qt)
    rows = np.arange(M) if n_tokens >= M else _sample(M, n_tokens, seed=idx)
    oref = O.decode_chain(x0[rows], layers, qt)
    for L in chain:
        assert np.array_equal(got[L["name"]][rows], oref[L["name"]]["y"]), L["name"]


def test_7b_decode_chain_int8_full():
    _int8_chain("7b", 2, I.CHAIN_7B, I.LINEARS_7B, I.W_SIGMA_7B, 256, "outliers", 256)


def test_7b_decode_chain_int8_gate_up_stacked():
    # gate and up as one GEMM over [W_gate; W_up] (N = 37888): the device
    # chain with the stacked linear equals the oracle chain with separate
    # gate and up, bit for bit, on sampled tokens.
    idx, M = 2, 256
    x0 = I.activations(M, 3584, seed=I.matrix_seed(idx, 0), kind="outliers")
    Wdev, layers = {}, []
    for L in I.CHAIN_7B:
        N, K = I.LINEARS_7B[L["name"]]
        ref, dev = _quant_full_int8(_weights("7b", L["name"], N, K, I.W_SIGMA_7B, idx))
        Wdev[L["name"]] = dev
        layers.append(dict(L, Wq=ref["Wq"], scale_w=ref["scale_w"], act_mult=I.UAQ_S))
    Wdev["gateup"] = (torch.cat([Wdev["gate"][0], Wdev["up"][0]]),
                      torch.cat([Wdev["gate"][1], Wdev["up"][1]]))
    got = _device_chain(I.CHAIN_7B_GATEUP, x0, Wdev, "int8")
    rows = _sample(M, 48, seed=7)
    oref = O.decode_chain(x0[rows], layers, "int8")
    n = I.LINEARS_7B["gate"][0]
    assert np.array_equal(got["gateup"][rows, :n], oref["gate"]["y"])
    assert np.array_equal(got["gateup"][rows, n:], oref["up"]["y"])
    for name in ("qkv", "o", "down"):
        assert np.array_equal(got[name][rows], oref[name]["y"]), name


def test_32b_decode_chain_int8_m512_sampled_tokens():
    _int8_chain("32b", 5, I.CHAIN_32B, I.LINEARS_32B, I.W_SIGMA_32B, 512, "normal", 128)


def test_32b_decode_chain_int8_m512_stacked_qkv_sampled_tokens():
    # q, k and v stacked into one 7168x5120 projection over the shared
    # quantized input (the stacked-QKV decode workload), 512 tokens.
    _int8_chain("32b", 5, I.CHAIN_32B_PREFILL, I.LINEARS_32B, I.W_SIGMA_32B, 512, "normal", 64)


def test_32b_prefill_int8_m4096_sampled_tokens():
    _int8_chain("32b", 5, I.CHAIN_32B_PREFILL, I.LINEARS_32B, I.W_SIGMA_32B, 4096, "heavy", 96)


_fp8_dev = {}


def _fp8_linear_sampled(tag, idx, name, N, K, sigma, M, kind):
    qt = "fp8"
    W = _weights(tag, name, N, K, sigma, idx)
    key = (tag, name)
    if key not in _fp8_dev:
        _fp8_dev.clear()
        _fp8_dev[key] = B.quantize_weights_uaq(to_dev_f32(W), I.UAQ_S, qt)
    Wq, sw = _fp8_dev[key]
    rows = _sample(N, 512, seed=N + K)
    ref = O.quantize_weights_uaq(W[rows], I.UAQ_S, qt)
    torch.cuda.synchronize()
    assert np.array_equal(codes_np(Wq)[rows], ref["Wq"].view(np.uint8)), name
    assert np.array_equal(sw.cpu().numpy()[rows], ref["scale_w"]), name
    X = I.activations(M, K, seed=I.matrix_seed(idx, 100 + _NAMES.index(name)), kind=kind)
    r = O.w8a8_linear(X, ref["Wq"], ref["scale_w"], I.UAQ_S, qt)
    Xq, sx = B.quantize_act_per_token(to_dev_bf16(X), I.UAQ_S, qt)
    y = B.w8a8_gemm(Xq, sx, Wq, sw, qt)
    torch.cuda.synchronize()
    assert np.array_equal(codes_np(Xq), r["Xq"].view(np.uint8)), name
    assert np.array_equal(sx.cpu().numpy(), r["scale_x"]), name
    assert_bf16_close(bf16_np(y)[:, rows], r["y"], what=f"fp8 {tag} {name} M={M}")


@pytest.mark.parametrize("name", ["qkv", "o", "gate", "up", "down"])
def test_7b_linears_fp8_sampled_channels(name):
    N, K = I.LINEARS_7B[name]
    for M in (1, 32, 256):
        _fp8_linear_sampled("7b", 3, name, N, K, I.W_SIGMA_7B, M, "outliers")


@pytest.mark.parametrize("name", ["qkv", "q", "k", "v", "o", "gate", "up", "down"])
def test_32b_linears_fp8_m512_sampled_channels(name):
    N, K = I.LINEARS_32B[name]
    _fp8_linear_sampled("32b", 5, name, N, K, I.W_SIGMA_32B, 512, "normal")


def _refresh_full_size(qt, name, linears, sigma, idx):
    """Refresh after W' += s * dW, dW ~ N(0, 1e-7^2), at one of the stack's
    matrix sizes, in the launch the refresh benchmark uses (the kernel is
    chosen by row length). The closed-form check is made on O and down (the
    two row lengths of each stack; skipped on gate+up to keep the test within
    seconds)."""
    N, K = linears[name]
    s32 = np.float32(I.UAQ_S)
    seed = I.matrix_seed(idx, _NAMES.index("gate" if name == "gateup" else name))
    Wp0 = (I.weights(N, K, sigma, seed=seed) / s32).astype(np.float32)
    Wp1 = I.normal_f32((N, K), I.DW_SIGMA, seed=seed + 1)
    Wp1 *= s32
    Wp1 += Wp0
    Wd = to_dev_f32(Wp0)
    Wq, _ = B.requantize_weights(Wd, qt, torch.empty((N, K), dtype=B.code_dtype(qt), device=Wd.device))
    Wd.copy_(torch.from_numpy(Wp1))
    rf = torch.empty(N, dtype=torch.int32, device=Wd.device)
    _, sw = B.requantize_weights(Wd, qt, Wq, row_flips=rf)
    c0, _, _ = O.requantize_weights(Wp0, qt)
    c1, s1, f1 = O.requantize_weights(Wp1, qt, codes_old=c0)
    del c0
    torch.cuda.synchronize()
    assert np.array_equal(codes_np(Wq), c1.view(np.uint8))
    assert np.array_equal(sw.cpu().numpy(), s1)
    assert np.array_equal(rf.cpu().numpy().astype(np.int64), f1)
    del Wq, Wd, c1, Wp1
    if name != "gateup":
        total = int(f1.sum())
        e = O.flip_expectation(Wp0, I.DW_SIGMA * I.UAQ_S, qt)
        assert abs(total - e) <= 5 * np.sqrt(e) + 0.02 * e, (total, e)


@pytest.mark.parametrize("qt", ["int8", "fp8"])
@pytest.mark.parametrize("name", ["o", "gateup", "down"])
def test_7b_refresh_full_size(qt, name):
    _refresh_full_size(qt, name, I.LINEARS_7B, I.W_SIGMA_7B, 7)


@pytest.mark.parametrize("qt,name", [("int8", "o"), ("int8", "down"), ("fp8", "o")])
def test_32b_refresh_full_size(qt, name):
    # Row lengths 5120 (q/k/v, O, gate, up) and 27648 (down): the two
    # launches of the 32B-shaped stack's refresh.
    _refresh_full_size(qt, name, I.LINEARS_32B, I.W_SIGMA_32B, 8)


@pytest.mark.parametrize("qt", ["int8", "fp8"])
@pytest.mark.parametrize("name", ["qkv", "o", "gate", "up", "down"])
def test_7b_uaq_flip_readings(qt, name):
    """The update-masking experiment at the 7B matrix sizes, counted by the
    library's refresh kernel: codes changed by one update dW ~ N(0, 1e-7^2)
    without UAQ (base) and with it under the three readings of where the
    update lands (same size on W/s, the pages' s dW, and the control dW/s).
    Every count equals the oracle's, and each lies within 5 sqrt(E) + 2% E of
    the closed-form expectation E (first order in the update)."""
    N, K = I.LINEARS_7B[name]
    s32 = np.float32(I.UAQ_S)
    seed = I.matrix_seed(11, _NAMES.index(name))
    W = I.weights(N, K, I.W_SIGMA_7B, seed=seed)
    dW = I.normal_f32((N, K), I.DW_SIGMA, seed=seed + 1)
    Ws = (W / s32).astype(np.float32)
    cases = {
        "base": (W, (W + dW).astype(np.float32), I.DW_SIGMA),
        "uaq_same": (Ws, (Ws + dW).astype(np.float32), I.DW_SIGMA),
        "uaq_pages": (Ws, (Ws + (dW * s32).astype(np.float32)).astype(np.float32),
                      I.DW_SIGMA * I.UAQ_S),
        "control": (Ws, (Ws + (dW / s32).astype(np.float32)).astype(np.float32),
                    I.DW_SIGMA / I.UAQ_S),
    }
    rf = torch.empty(N, dtype=torch.int32, device="cuda:0")
    ref_codes = {}
    got = {}
    for k, (A0, A1, _) in cases.items():
        key = "W" if A0 is W else "Ws"
        if key not in ref_codes:
            ref_codes[key], _ = B.requantize_weights(
                to_dev_f32(A0), qt, torch.empty((N, K), dtype=B.code_dtype(qt), device="cuda:0"))
        Wq = ref_codes[key].clone()
        B.requantize_weights(to_dev_f32(A1), qt, Wq, row_flips=rf)
        got[k] = int(rf.sum().item())
        del Wq
    del ref_codes
    torch.cuda.synchronize()
    ref = O.flip_counts(W, dW, I.UAQ_S, qt)
    for k, (A0, _, sigma) in cases.items():
        assert got[k] == ref[k], (k, got[k], ref[k])
        e = O.flip_expectation(A0, sigma, qt)
        assert abs(got[k] - e) <= 5 * np.sqrt(e) + 0.02 * e, (k, got[k], e)
    assert got["base"] < got["uaq_same"] < got["uaq_pages"]
    print(f"{qt} {name} {N}x{K}: " + ", ".join(f"{k} {v}" for k, v in got.items()))
