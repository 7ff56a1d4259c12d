"""qr_linear_fused at 1-4 tokens (one launch, input quantized in the kernel) against the oracle.

qr_linear_fused is one rollout linear (paper notes, "Loss / training
strategy": token-wise activation and channel-wise weight scales, INT8 or
FP8): the per-token quantization of the bf16 input, the quantized product
and the bf16 epilogue. At 1-4 tokens (when the token rows' codes fit the
limit M K <= 8192, or up to M K <= 20480 when forced) it runs as one launch whose blocks quantize the input
themselves and split K among their waves.

* INT8: every output equals the oracle's w8a8_linear bit for bit: every
  block height (16 to 80 output channels), ragged N and K, strided X and Y,
  all-zero rows, graph replays, and the 7B-shaped layer chain at one token.
* FP8: against the oracle's exact accumulators. The device accumulator lies
  within the MFMA accumulation bound of the exact sum (fp8_acc_bound), and
  the two fp32 scale products and the bf16 rounding move the result by at
  most 2^-8 of its value more, so
  |y - acc_exact sx sw| <= bound |sx sw| (1 + 2^-7) + 2^-8 |acc_exact sx sw|,
  and the outputs meet the 1e-2 bar against the oracle's bf16 outputs.
* The path is the one-launch one: it never touches the workspace (filled
  with a pattern that must survive), while the two-launch path (the
  override -1) writes the codes there. qr_linear_fused takes it by itself
  up to M K = 8192 ("auto") and wherever the kernel can run (M <= 4,
  M K <= 20480) when forced.
"""

import functools

import numpy as np
import pytest
import torch

import oracle as O
from oracle import formats as F
from w8a8_gemm_rl_amd import binding as B
from w8a8_gemm_rl_amd import inputs as I

from gpu_helpers import DEV, assert_bf16_close, bf16_np, fp8_acc_bound, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu

QTS = ["int8", "fp8"]
def can_run(M, K):
    """The kernel's own limits (qr_set_small_m_override 1..5)."""
    return 1 <= M <= 4 and K >= 16 and M * K <= 20480


def auto(M, K):
    """Where qr_linear_fused takes the path by itself (the faster path)."""
    return can_run(M, K) and M * K <= 8192


def rf_for(N):
    """The library's block height: the fewest 16-row fragments (1-5) with at
    most 256 blocks."""
    for rf in range(1, 5):
        if -(-N // (16 * rf)) <= 256:
            return rf
    return 5


@pytest.fixture(autouse=True)
def _reset():
    B.set_small_m_override(0)
    B.set_plan_override(-1)
    yield
    B.set_small_m_override(0)
    B.set_plan_override(-1)
    torch.cuda.synchronize()


@functools.lru_cache(maxsize=8)
def _weights(N, K, qt, seed):
    W = I.weights(N, K, I.W_SIGMA_7B, seed=seed)
    r = O.quantize_weights_uaq(W, I.UAQ_S, qt)
    dev = B.quantize_weights_uaq(to_dev_f32(W), I.UAQ_S, qt)
    return r["Wq"], r["scale_w"], dev


def _run(X_bits, N, K, qt, seed, ws_fill=0xAB, Y=None):
    """Device linear_fused on X_bits; returns (y bits, workspace untouched?)."""
    Wq, sw, (dWq, dsw) = _weights(N, K, qt, seed)
    X = to_dev_bf16(X_bits) if not torch.is_tensor(X_bits) else X_bits
    M = X.shape[0]
    need = B.workspace_size("qr_linear_fused", M, N, K, qt)
    ws = torch.full((max(need, 256),), ws_fill, dtype=torch.uint8, device=DEV)
    Y = B.linear_fused(X, I.UAQ_S, dWq, dsw, qt, Y=Y, ws=ws)
    torch.cuda.synchronize()
    untouched = bool((ws == ws_fill).all())
    return Y, untouched, Wq, sw


def _check_fp8(y_bits, X_bits, Wq, sw, what):
    Xq, sx = O.quantize_act_per_token(X_bits, I.UAQ_S, "fp8")
    acc = O.acc_fp8(Xq, Wq)
    bound = fp8_acc_bound(Xq, Wq)
    s = np.abs(sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :])
    yx = acc * sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :]
    y = F.bf16_bits_to_f32(y_bits).astype(np.float64)
    lim = bound * s * (1 + 2.0 ** -7) + 2.0 ** -8 * np.abs(yx) + 1e-30
    bad = np.abs(y - yx) > lim
    assert not bad.any(), (what, int(bad.sum()), float(np.abs(y - yx).max()))
    ref = O.dequant_epilogue(acc, sx, sw)[1]
    assert_bf16_close(y_bits, ref, 1e-2, what)


SHAPES = [(3584, 3584), (4608, 3584), (18944, 3584), (3584, 18944), (200, 1040), (37, 16)]


# forced cases only where the kernel can run (the others are the auto cases'
# fallback to the general path)
CASES = [(mode, qt, N, K, M) for mode in ("auto", "forced") for qt in QTS for N, K in SHAPES
         for M in (1, 2, 3, 4) if mode == "auto" or can_run(M, K)]


@pytest.mark.parametrize("mode,qt,N,K,M", CASES)
def test_linear_fused_small_m_vs_oracle(mode, qt, N, K, M):
    if mode == "forced":
        B.set_small_m_override(rf_for(N))
    X_bits = I.activations(M, K, seed=I.matrix_seed(6, M * 7 + K % 97), kind="outliers")
    y, untouched, Wq, sw = _run(X_bits, N, K, qt, seed=N + K)
    expect = auto(M, K) if mode == "auto" else True
    assert untouched == expect, (mode, M, N, K, untouched)
    what = (qt, M, N, K)
    if qt == "int8":
        ref = O.w8a8_linear(X_bits, Wq, sw, I.UAQ_S, qt)["y"]
        assert np.array_equal(bf16_np(y), ref), what
    else:
        _check_fp8(bf16_np(y), X_bits, Wq, sw, what)


@pytest.mark.parametrize("qt", QTS)
@pytest.mark.parametrize("rf", [1, 2, 3, 4, 5])
def test_every_block_height_ragged(qt, rf):
    # N not a multiple of any block height, K with a 16-byte last chunk,
    # one all-zero token row (scale 0, codes 0, outputs 0)
    M, N, K = 3, 200, 1040
    X_bits = I.activations(M, K, seed=I.matrix_seed(6, 40 + rf), kind="outliers")
    X_bits[1] = 0
    B.set_small_m_override(rf)
    y, untouched, Wq, sw = _run(X_bits, N, K, qt, seed=7)
    assert untouched
    if qt == "int8":
        ref = O.w8a8_linear(X_bits, Wq, sw, I.UAQ_S, qt)["y"]
        assert np.array_equal(bf16_np(y), ref), rf
    else:
        _check_fp8(bf16_np(y), X_bits, Wq, sw, (qt, rf))
    assert not F.bf16_bits_to_f32(bf16_np(y)[1]).any()


@pytest.mark.parametrize("qt", QTS)
def test_equals_two_launch_path(qt):
    """The same call with the path switched off (quantizer + GEMM launches):
    INT8 outputs are the same bits; FP8 outputs meet the 1e-2 bar."""
    M, N, K = 1, 3584, 18944
    X_bits = I.activations(M, K, seed=I.matrix_seed(6, 90), kind="outliers")
    B.set_small_m_override(1)
    y1, u1, _, _ = _run(X_bits, N, K, qt, seed=11)
    B.set_small_m_override(-1)
    y2, u2, _, _ = _run(X_bits, N, K, qt, seed=11)
    assert u1 and not u2
    if qt == "int8":
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    else:
        assert_bf16_close(bf16_np(y1), bf16_np(y2), 1e-2, "fp8 paths")


@pytest.mark.parametrize("qt", QTS)
def test_strided_input_and_output(qt):
    """X a column slice of a wider bf16 matrix (row stride > K), Y a column
    slice of a wider output (columns outside it keep their values)."""
    M, N, K, W = 4, 1024, 2048, 3072
    big = I.activations(M, W, seed=I.matrix_seed(6, 91), kind="outliers")
    X = to_dev_bf16(big)[:, 512:512 + K]
    Yb = torch.full((M, N + 40), 3.0, dtype=torch.bfloat16, device=DEV)
    Y = Yb[:, 8:8 + N]
    y, untouched, Wq, sw = _run(X, N, K, qt, seed=13, Y=Y)
    assert untouched
    X_bits = np.ascontiguousarray(big[:, 512:512 + K])
    if qt == "int8":
        ref = O.w8a8_linear(X_bits, Wq, sw, I.UAQ_S, qt)["y"]
        assert np.array_equal(bf16_np(Y), ref)
    else:
        _check_fp8(bf16_np(Y), X_bits, Wq, sw, "strided")
    pad = torch.cat([Yb[:, :8], Yb[:, 8 + N:]], dim=1)
    assert bool((pad == 3.0).all())


def test_size_limit():
    """At the largest token rows (M K = 20480) the path runs; 16 elements
    more fall back to the two launches."""
    qt = "int8"
    B.set_small_m_override(1)
    for K, expect in [(5120, True), (5136, False)]:
        X_bits = I.activations(4, K, seed=I.matrix_seed(6, 92), kind="outliers")
        y, untouched, Wq, sw = _run(X_bits, 512, K, qt, seed=17)
        assert untouched == expect, K
        ref = O.w8a8_linear(X_bits, Wq, sw, I.UAQ_S, qt)["y"]
        assert np.array_equal(bf16_np(y), ref), K


def test_plan_override_disables_path():
    X_bits = I.activations(1, 3584, seed=I.matrix_seed(6, 93), kind="outliers")
    B.set_plan_override(0)
    y, untouched, Wq, sw = _run(X_bits, 3584, 3584, "int8", seed=19)
    assert not untouched
    ref = O.w8a8_linear(X_bits, Wq, sw, I.UAQ_S, "int8")["y"]
    assert np.array_equal(bf16_np(y), ref)


@pytest.mark.parametrize("qt", QTS)
def test_graph_replays(qt):
    """The one-launch linears of a short chain captured in a HIP graph: every
    replay equals the eager result."""
    K0, shapes = 3584, [(4608, 3584), (3584, 3584)]
    X = to_dev_bf16(I.activations(1, K0, seed=I.matrix_seed(6, 94), kind="outliers"))
    Ws = [_weights(N, K, qt, 23 + i)[2] for i, (N, K) in enumerate(shapes)]
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device=DEV)
    ys = [torch.empty((1, N), dtype=torch.bfloat16, device=DEV) for N, _ in shapes]

    def chain():
        B.linear_fused(X, I.UAQ_S, *Ws[0], qt, Y=ys[0], ws=ws)
        B.linear_fused(ys[0][:, :3584], I.UAQ_S, *Ws[1], qt, Y=ys[1], ws=ws)

    chain()
    torch.cuda.synchronize()
    ref = [t.clone() for t in ys]
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            chain()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in ys:
            t.zero_()
        junk = torch.randn(1000, device=DEV).sum()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(ys, ref):
            assert torch.equal(t.view(torch.int16), r.view(torch.int16)), f"replay {rep}"
        chain()
        torch.cuda.synchronize()
        assert float(junk) == float(junk)


def test_7b_chain_one_token_equals_oracle():
    """The 7B-shaped layer at one token with one linear_fused call per linear
    (QKV, O, gate and up on the one-launch path, gate and up each quantizing
    the O output themselves; down, K = 18944, on the quantizer and GEMM
    launches): every output of every linear equals the oracle chain bit for
    bit."""
    qt, M = "int8", 1
    x0 = I.activations(M, 3584, seed=I.matrix_seed(2, 80), kind="outliers")
    layers, dev = [], {}
    for i, L in enumerate(I.CHAIN_7B):
        N, K = I.LINEARS_7B[L["name"]]
        W = I.weights(N, K, I.W_SIGMA_7B, seed=I.matrix_seed(2, 20 + i))
        r = O.quantize_weights_uaq(W, I.UAQ_S, qt)
        dev[L["name"]] = B.quantize_weights_uaq(to_dev_f32(W), I.UAQ_S, qt)
        layers.append(dict(L, Wq=r["Wq"], scale_w=r["scale_w"], act_mult=I.UAQ_S))
    oref = O.decode_chain(x0, layers, qt)
    ys = {"x0": to_dev_bf16(x0)}
    for L in I.CHAIN_7B:
        src = ys[L["src"]]
        if L["cols"] is not None:
            src = src[:, L["cols"][0]:L["cols"][1]]
        ys[L["name"]] = B.linear_fused(src, I.UAQ_S, *dev[L["name"]], qt)
    torch.cuda.synchronize()
    for L in I.CHAIN_7B:
        assert np.array_equal(bf16_np(ys[L["name"]]), oref[L["name"]]["y"]), L["name"]
