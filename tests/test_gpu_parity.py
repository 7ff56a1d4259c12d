"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bar: bit-exact quantized codes, scales, W/s and int32 accumulators (and, since
the accumulators and the epilogue order agree, bit-exact INT8 bf16 outputs);
FP8 accumulators within the bound of the MFMA accumulation (gpu_helpers.fp8_acc_bound)
and FP8 bf16 outputs within
the relative tolerance 1e-2 (tests/gpu_helpers.assert_bf16_close).
Inputs come from the seeded generators in w8a8_gemm_rl_amd.inputs.
"""

import re

import numpy as np
import pytest
import torch

import oracle as O
from w8a8_gemm_rl_amd import binding as B
from w8a8_gemm_rl_amd import inputs as I

from gpu_helpers import (DEV, assert_bf16_close, bf16_np, codes_np, fp8_acc_bound, to_dev_bf16,
                         to_dev_codes, to_dev_f32)

pytestmark = pytest.mark.gpu

QTS = ["int8", "fp8"]


@pytest.fixture(autouse=True)
def _reset_plan():
    B.set_plan_override(-1)
    yield
    B.set_plan_override(-1)
    torch.cuda.synchronize()


# ------------------------------------------------------------ weight quantizer

@pytest.mark.parametrize("qt", QTS)
@pytest.mark.parametrize("N,K,s", [(512, 512, 1.5), (37, 48, 1.5), (5, 16, 2.0), (64, 3584, 1.5),
                                   (3, 40960, 1.5), (300, 1024, 1.0), (33, 5120, 1.5),
                                   (17, 18944, 1.5), (9, 27648, 1.5)])
def test_weight_quant_bit_exact(qt, N, K, s):
    W = I.weights(N, K, 0.02, seed=N * 7 + K)
    W[min(2, N - 1)] = 0.0  # an all-zero channel
    ref = O.quantize_weights_uaq(W, s, qt)
    Wd = to_dev_f32(W)
    Wsc = torch.empty_like(Wd)
    Wq, sw = B.quantize_weights_uaq(Wd, s, qt, W_scaled=Wsc)
    torch.cuda.synchronize()
    assert np.array_equal(codes_np(Wq), ref["Wq"].view(np.uint8))
    assert np.array_equal(sw.cpu().numpy(), ref["scale_w"])
    assert np.array_equal(Wsc.cpu().numpy(), ref["W_scaled"])


@pytest.mark.parametrize("qt", QTS)
def test_weight_quant_in_place_strided_and_norm_fold(qt):
    N, K, ld = 96, 512, 640
    W = I.weights(N, ld, 0.02, seed=31)
    g = I.normal_f32((K,), 1.0, seed=32)
    b = I.normal_f32((K,), 0.1, seed=33)
    ref = O.quantize_weights_uaq(W[:, :K], 1.5, qt, gamma=g, beta=b)
    Wd = to_dev_f32(W)
    view = Wd[:, :K]
    gd, bd = to_dev_f32(g), to_dev_f32(b)
    Wq, sw = B.quantize_weights_uaq(view, 1.5, qt, W_scaled=view, gamma=gd, beta=bd)
    torch.cuda.synchronize()
    assert np.array_equal(codes_np(Wq), ref["Wq"].view(np.uint8))
    assert np.array_equal(sw.cpu().numpy(), ref["scale_w"])
    Wout = Wd.cpu().numpy()
    assert np.array_equal(Wout[:, :K], ref["W_scaled"])
    assert np.array_equal(Wout[:, K:], W[:, K:])  # padding untouched
    assert np.array_equal(gd.cpu().numpy(), ref["gamma"])
    assert np.array_equal(bd.cpu().numpy(), ref["beta"])


_CAP = 1 << 21  # blocks per quantizer launch; more rows take several launches


def _loop_rows(N, rpb):
    """Rows at the start, around each multiple of one launch's row span, and at the end."""
    span = _CAP * rpb
    r = [0, 1, 2, N - 3, N - 2, N - 1]
    for m in range(span, N, span):
        r += [m - 2, m - 1, m, m + 1]
    return np.unique(np.array(r, np.int64))


@pytest.mark.parametrize("qt", QTS)
@pytest.mark.parametrize("N,K,rpb", [(4 * _CAP + 37, 16, 4), (_CAP + 5, 1040, 1)])
def test_weight_quantizers_past_the_launch_cap(qt, N, K, rpb):
    """More rows than one launch's blocks cover: every row is still quantized,
    by the UAQ quantizer and by the refresh (with per-row change counts)."""
    gen = torch.Generator(device=DEV)
    gen.manual_seed(N + K)
    W = torch.randn((N, K), generator=gen, device=DEV).mul_(0.02)
    rows = _loop_rows(N, rpb)
    Wh = W[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    ref = O.quantize_weights_uaq(Wh, 1.5, qt)
    Wq, sw = B.quantize_weights_uaq(W, 1.5, qt)
    torch.cuda.synchronize()
    idx = torch.from_numpy(rows).to(DEV)
    assert np.array_equal(codes_np(Wq[idx]), ref["Wq"].view(np.uint8))
    assert np.array_equal(sw[idx].cpu().numpy(), ref["scale_w"])
    # refresh of W itself over zeroed codes: counts = nonzero-valued codes per row
    Wq.zero_()
    rf = torch.full((N,), -1, dtype=torch.int32, device=DEV)
    B.requantize_weights(W, qt, Wq, sw, row_flips=rf)
    c1, s1, f1 = O.requantize_weights(Wh, qt, codes_old=np.zeros((len(rows), K), np.uint8))
    torch.cuda.synchronize()
    assert np.array_equal(codes_np(Wq[idx]), c1.view(np.uint8))
    assert np.array_equal(sw[idx].cpu().numpy(), s1)
    assert np.array_equal(rf[idx].cpu().numpy().astype(np.int64), f1)
    assert int((rf < 0).sum().item()) == 0  # every row written


@pytest.mark.parametrize("qt", QTS)
@pytest.mark.parametrize("M,K,rpb", [(4 * _CAP + 37, 16, 4), (_CAP + 5, 2064, 1)])
def test_act_quantizer_past_the_launch_cap(qt, M, K, rpb):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(M + K)
    X = torch.randn((M, K), generator=gen, device=DEV, dtype=torch.bfloat16)
    rows = _loop_rows(M, rpb)
    idx = torch.from_numpy(rows).to(DEV)
    Xh = bf16_np(X[idx])
    codes, sx = O.quantize_act_per_token(Xh, 1.5, qt)
    Xq, sxd = B.quantize_act_per_token(X, 1.5, qt)
    torch.cuda.synchronize()
    assert np.array_equal(codes_np(Xq[idx]), codes.view(np.uint8))
    assert np.array_equal(sxd[idx].cpu().numpy(), sx)


def test_norm_fold_longer_than_the_grid():
    """gamma/beta of more elements than one pass of the fold's grid covers
    (FP8: INT8 rows are limited far below this by the int32 accumulator)."""
    K = (1 << 28) + 16
    W = torch.zeros((1, K), dtype=torch.float32, device=DEV)
    W[0, 0] = 1.0
    gen = torch.Generator(device=DEV)
    gen.manual_seed(3)
    gd = torch.randn(K, generator=gen, device=DEV)
    g0 = gd.clone()
    B.quantize_weights_uaq(W, 1.5, "fp8", gamma=gd)
    torch.cuda.synchronize()
    pos = torch.tensor([0, 1, (1 << 28) - 1, 1 << 28, K - 1], device=DEV)
    ref = (g0[pos].cpu().numpy() * np.float32(1.5)).astype(np.float32)
    assert np.array_equal(gd[pos].cpu().numpy(), ref)
    assert torch.equal(gd, g0 * 1.5)


# ------------------------------------------------------------ activation quantizer

@pytest.mark.parametrize("qt", QTS)
@pytest.mark.parametrize("M,K,kind", [(16, 512, "normal"), (1, 3584, "outliers"), (3, 16, "normal"),
                                      (257, 3584, "outliers"), (33, 18944, "outliers"),
                                      (8, 5120, "heavy"), (2, 40960, "normal"), (5, 2048, "heavy"),
                                      (4, 8192, "heavy"), (3, 8208, "normal")])
def test_act_quant_bit_exact(qt, M, K, kind):
    X = I.activations(M, K, seed=M + K, kind=kind)
    if M > 2:
        X[1] = 0  # an all-zero token
    codes, sx = O.quantize_act_per_token(X, 1.5, qt)
    Xq, sxd = B.quantize_act_per_token(to_dev_bf16(X), 1.5, qt)
    torch.cuda.synchronize()
    assert np.array_equal(codes_np(Xq), codes.view(np.uint8))
    assert np.array_equal(sxd.cpu().numpy(), sx)


@pytest.mark.parametrize("qt", QTS)
def test_act_quant_strided_rows(qt):
    X = I.activations(40, 4608, seed=5, kind="outliers")
    codes, sx = O.quantize_act_per_token(X[:, :3584], 1.0, qt)
    Xd = to_dev_bf16(X)[:, :3584]
    Xq, sxd = B.quantize_act_per_token(Xd, 1.0, qt)
    torch.cuda.synchronize()
    assert np.array_equal(codes_np(Xq), codes.view(np.uint8))
    assert np.array_equal(sxd.cpu().numpy(), sx)


def test_fp8_encoder_boundaries_on_device():
    """Every E4M3FN midpoint, its fp32 neighbours and signed zeros, through the act quantizer.

    A row whose absmax is 448 has step t = 1, so x / t = x and the codes are
    the encoder applied to x itself (inputs are bf16, so midpoints that bf16
    cannot hold are covered by their nearest bf16 values).
    """
    vals = O.formats.e4m3fn_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    xs = np.concatenate([vals, mids, -vals, -mids, [0.0, -0.0, 2 ** -10, -2 ** -10, 3 * 2 ** -11]])
    xs = xs.astype(np.float32)
    bits = I.bf16_bits(xs)
    n = len(bits)
    K = ((n + 1 + 15) // 16) * 16
    row = np.zeros(K, np.uint16)
    row[:n] = bits
    row[n] = I.bf16_bits(np.float32([448.0]))[0]
    X = row[None, :]
    codes, sx = O.quantize_act_per_token(X, 1.0, "fp8")
    assert sx[0] == 1.0
    Xq, sxd = B.quantize_act_per_token(to_dev_bf16(X), 1.0, "fp8")
    torch.cuda.synchronize()
    assert np.array_equal(codes_np(Xq), codes.view(np.uint8))


# ------------------------------------------------------------ GEMM

def _codes_pair(M, N, K, qt, seed):
    X = I.activations(M, K, seed=seed, kind="outliers")
    W = I.weights(N, K, 0.02, seed=seed + 1)
    wq = O.quantize_weights_uaq(W, 1.5, qt)
    xq, sx = O.quantize_act_per_token(X, 1.5, qt)
    return xq, sx, wq["Wq"], wq["scale_w"]


def _run_gemm(xq, sx, wq, sw, qt, out):
    return B.w8a8_gemm(to_dev_codes(xq, qt), to_dev_f32(sx), to_dev_codes(wq, qt), to_dev_f32(sw),
                       qt, out=out)


def _check_gemm(xq, sx, wq, sw, qt, what):
    acc = O.acc_int8(xq, wq) if qt == "int8" else O.acc_fp8(xq, wq)
    _, yref = O.dequant_epilogue(acc, sx, sw)
    raw = _run_gemm(xq, sx, wq, sw, qt, "raw")
    y = _run_gemm(xq, sx, wq, sw, qt, "bf16")
    torch.cuda.synchronize()
    raw = raw.cpu().numpy()
    yb = bf16_np(y)
    if qt == "int8":
        assert np.array_equal(raw, acc), what
        assert np.array_equal(yb, yref), what
    else:
        err = np.abs(raw.astype(np.float64) - acc)
        assert np.all(err <= fp8_acc_bound(xq, wq)), (what, err.max())
        assert_bf16_close(yb, yref, what=what)


@pytest.mark.parametrize("qt", QTS)
@pytest.mark.parametrize("M,N,K", [(16, 512, 512), (1, 64, 16), (37, 200, 528), (130, 264, 1040),
                                   (257, 96, 256), (300, 520, 384)])
def test_gemm_auto_plan(qt, M, N, K):
    xq, sx, wq, sw = _codes_pair(M, N, K, qt, seed=M * 3 + N)
    _check_gemm(xq, sx, wq, sw, qt, f"{qt} M={M} N={N} K={K} plan={B.gemm_plan(M, N, K, qt)}")


NUM_TILES = 11  # entries of the library's tile table


def _tile_height(tile):
    return int(re.search(r"_n(\d+)_", B.tile_name(tile)).group(1))


@pytest.mark.parametrize("qt", QTS)
@pytest.mark.parametrize("tile", range(NUM_TILES))
@pytest.mark.parametrize("splitk", [1, 3, 9])
@pytest.mark.parametrize("M,N,K", [(70, 300, 1152), (45, 136, 1040), (40, 72, 96)])
def test_gemm_every_tile_and_split(qt, tile, splitk, M, N, K):
    # Ragged in M and N for every tile; 9 K steps of 128, the second shape
    # with a 16-byte last step, the third a single step shorter than 128
    # bytes. Split 9 leaves one or two K steps per block, fewer than the LDS
    # ring holds.
    assert B.num_tiles() == NUM_TILES
    xq, sx, wq, sw = _codes_pair(M, N, K, qt, seed=tile * 10 + splitk + M)
    B.set_plan_override(tile, splitk)
    _check_gemm(xq, sx, wq, sw, qt, f"{qt} tile={tile} splitk={splitk} M={M} N={N} K={K}")


@pytest.mark.parametrize("qt", QTS)
@pytest.mark.parametrize("tile", range(NUM_TILES))
@pytest.mark.parametrize("splitk", [1, 3])
@pytest.mark.parametrize("shrink", ["min", "one_block_less", "half"])
def test_gemm_partial_row_tiles(qt, tile, splitk, shrink):
    # Tiles that own fewer weight rows than their height (rows past the owned
    # ones read as zero and are not stored), with split K: 8 rows per tile;
    # one 8-row block less than the height; about half the height. N = 300
    # ends the last tile inside a row block; M and K are ragged too (a
    # 16-byte last K step).
    M, N, K = 70, 300, 1040
    bn = _tile_height(tile)
    rows = {"min": 8, "one_block_less": max(8, bn - 8), "half": max(8, (bn // 2 + 4) // 8 * 8)}[shrink]
    xq, sx, wq, sw = _codes_pair(M, N, K, qt, seed=tile * 7 + splitk + rows)
    B.set_plan_override(tile, splitk, rows)
    _check_gemm(xq, sx, wq, sw, qt, f"{qt} tile={tile} splitk={splitk} rows={rows} M={M} N={N} K={K}")


@pytest.mark.parametrize("qt", QTS)
@pytest.mark.parametrize("tile", range(NUM_TILES))
@pytest.mark.parametrize("pad", [4, 3])
def test_gemm_strided_output(qt, tile, pad):
    # Y with a row stride of N + pad elements (N + 4 = 304: bf16 rows staged
    # through LDS and stored 16 bytes at a time; N + 3: stored from the MFMA
    # layout), ragged M and N, tiles owning fewer rows than their height:
    # the same bytes as a packed Y, and the padding columns untouched.
    M, N, K = 70, 300, 1040
    rows = max(8, (_tile_height(tile) // 2 + 4) // 8 * 8)
    xq, sx, wq, sw = _codes_pair(M, N, K, qt, seed=tile * 5 + pad)
    B.set_plan_override(tile, 1, rows)
    args = (to_dev_codes(xq, qt), to_dev_f32(sx), to_dev_codes(wq, qt), to_dev_f32(sw), qt)
    big = torch.full((M, N + pad), -3.0, dtype=torch.bfloat16, device=DEV)
    B.w8a8_gemm(*args, Y=big[:, :N])
    packed = B.w8a8_gemm(*args)
    torch.cuda.synchronize()
    assert torch.equal(big[:, :N].view(torch.int16), packed.view(torch.int16)), (qt, tile, pad)
    assert bool((big[:, N:] == -3.0).all()), (qt, tile, pad)
    acc = O.acc_int8(xq, wq) if qt == "int8" else O.acc_fp8(xq, wq)
    _, yref = O.dequant_epilogue(acc, sx, sw)
    if qt == "int8":
        assert np.array_equal(bf16_np(packed), yref)
    else:
        assert_bf16_close(bf16_np(packed), yref, what=f"fp8 tile={tile}")


@pytest.mark.parametrize("qt", QTS)
@pytest.mark.parametrize("tile", range(NUM_TILES))
@pytest.mark.parametrize("splitk", [1, 3])
def test_gemm_partial_tile_rows(qt, tile, splitk):
    # Tiles that own fewer weight rows than their height: 8 rows, and the
    # largest multiple of 8 below 5/8 of the height.
    M, N, K = 45, 136, 1040
    bn = _tile_height(tile)
    for rows in sorted({8, max(8, (5 * bn // 8) // 8 * 8)}):
        xq, sx, wq, sw = _codes_pair(M, N, K, qt, seed=tile * 7 + splitk + rows)
        B.set_plan_override(tile, splitk, rows)
        assert B.gemm_plan(M, N, K, qt) == (tile, splitk, rows)
        _check_gemm(xq, sx, wq, sw, qt, f"{qt} tile={tile} splitk={splitk} rows={rows}")


@pytest.mark.parametrize("qt", QTS)
def test_gemm_split_deterministic_and_reusable(qt):
    M, N, K = 32, 1024, 4096
    xq, sx, wq, sw = _codes_pair(M, N, K, qt, seed=77)
    t, s, _ = B.gemm_plan(M, N, K, qt)
    assert s > 1
    a = [_run_gemm(xq, sx, wq, sw, qt, "raw") for _ in range(3)]
    torch.cuda.synchronize()
    for r in a[1:]:
        assert torch.equal(r.view(torch.int32), a[0].view(torch.int32))


@pytest.mark.parametrize("qt", QTS)
def test_gemm_edge_sizes(qt):
    # M = 0 and N = 0 are no-ops; K = 0 gives zeros.
    e = torch.empty((0, 64), dtype=B.code_dtype(qt), device=DEV)
    w = torch.zeros((8, 64), dtype=torch.int8, device=DEV).view(B.code_dtype(qt))
    y = B.w8a8_gemm(e, torch.empty(0, device=DEV), w, torch.ones(8, device=DEV), qt)
    assert y.shape == (0, 8)
    x0 = torch.zeros((4, 0), dtype=torch.int8, device=DEV).view(B.code_dtype(qt))
    w0 = torch.zeros((8, 0), dtype=torch.int8, device=DEV).view(B.code_dtype(qt))
    y = B.w8a8_gemm(x0, torch.ones(4, device=DEV), w0, torch.ones(8, device=DEV), qt)
    y2 = B.w8a8_gemm(x0, torch.ones(4, device=DEV), w0[:0], torch.ones(0, device=DEV), qt)
    torch.cuda.synchronize()
    assert y2.shape == (4, 0)
    assert torch.count_nonzero(y.float()) == 0


def test_gemm_int8_extreme_codes_no_overflow():
    M, N, K = 4, 32, 27648
    xq = np.full((M, K), 127, np.int8)
    xq[1] = -127
    wq = np.full((N, K), 127, np.int8)
    wq[3] = -127
    sx = np.ones(M, np.float32)
    sw = np.ones(N, np.float32)
    raw = _run_gemm(xq, sx, wq, sw, "int8", "raw").cpu().numpy()
    assert np.array_equal(raw, O.acc_int8(xq, wq))
    assert raw[0, 0] == K * 127 * 127


# ------------------------------------------------------------ fused linear, single-linear workload

@pytest.mark.parametrize("qt", QTS)
def test_single_linear_workload_end_to_end(qt):
    """X[16,512] bf16 ~ N(0,1), W[512,512] ~ N(0,0.02), UAQ s = 1.5, seed 0."""
    c = I.SINGLE
    X = I.activations(c["M"], c["K"], seed=c["seed"])
    W = I.weights(c["N"], c["K"], c["w_sigma"], seed=c["seed"] + 1)
    wref = O.quantize_weights_uaq(W, c["s"], qt)
    ref = O.w8a8_linear(X, wref["Wq"], wref["scale_w"], c["s"], qt)
    Wq, sw = B.quantize_weights_uaq(to_dev_f32(W), c["s"], qt)
    Xd = to_dev_bf16(X)
    y = B.linear_fused(Xd, c["s"], Wq, sw, qt)
    Xq, sx = B.quantize_act_per_token(Xd, c["s"], qt)
    raw = B.w8a8_gemm(Xq, sx, Wq, sw, qt, out="raw")
    torch.cuda.synchronize()
    assert np.array_equal(codes_np(Wq), wref["Wq"].view(np.uint8))
    assert np.array_equal(codes_np(Xq), ref["Xq"].view(np.uint8))
    assert np.array_equal(sx.cpu().numpy(), ref["scale_x"])
    if qt == "int8":
        assert np.array_equal(raw.cpu().numpy(), ref["acc"])
        assert np.array_equal(bf16_np(y), ref["y"])
    else:
        assert_bf16_close(bf16_np(y), ref["y"], what="single linear fp8")


# ------------------------------------------------------------ update masking on device codes

@pytest.mark.parametrize("qt", QTS)
def test_flip_counts_from_device_codes(qt):
    """The UAQ flip experiment with the device quantizer gives the oracle's counts exactly."""
    N, K, s = 512, 512, 1.5
    W = I.weights(N, K, 0.02, seed=3)
    dW = I.normal_f32((N, K), I.DW_SIGMA, seed=10_003)
    ref = O.flip_counts(W, dW, s, qt)
    s32 = np.float32(s)
    Ws = (W / s32).astype(np.float32)

    def dev_codes(A):
        return codes_np(B.quantize_weights_uaq(to_dev_f32(A), 1.0, qt)[0])

    c0, cs = dev_codes(W), dev_codes(Ws)
    def flips(A, c):
        return O.count_flips(c, dev_codes(A.astype(np.float32)), qt)

    got = {
        "base": flips(W + dW, c0),
        "uaq_same": flips(Ws + dW, cs),
        "uaq_pages": flips(Ws + (dW * s32).astype(np.float32), cs),
        "control": flips(Ws + (dW / s32).astype(np.float32), cs),
    }
    for k in got:
        assert got[k] == ref[k], (k, got[k], ref[k])
    # UAQ's effect as quantized on the device: same-size W/s quantization == the device's s path
    cq = codes_np(B.quantize_weights_uaq(to_dev_f32(W), s, qt)[0])
    assert np.array_equal(cq, cs)


# ------------------------------------------------------------ per-step weight refresh

def _refresh_case(N, K, qt, seed, ld=None):
    """Stored parameters W' = W / s before and after one update s * dW (fp32)."""
    s32 = np.float32(I.UAQ_S)
    W = I.weights(N, ld or K, 0.02, seed=seed)
    W[min(1, N - 1)] = 0.0  # an all-zero channel stays all zero
    Wp0 = (W / s32).astype(np.float32)
    dW = I.normal_f32(Wp0.shape, I.DW_SIGMA * 30, seed=seed + 1)
    Wp1 = (Wp0 + (dW * s32).astype(np.float32)).astype(np.float32)
    Wp1[min(1, N - 1)] = 0.0
    return Wp0, Wp1


def _row_flips(N):
    return torch.full((N,), -1, dtype=torch.int32, device=DEV)


@pytest.mark.parametrize("qt", QTS)
@pytest.mark.parametrize("N,K", [(512, 512), (37, 48), (300, 1024), (64, 3584), (3, 40960),
                                 (129, 1040), (33, 5120), (17, 18944), (9, 27648)])
def test_requantize_codes_scales_and_flips(qt, N, K):
    """Refresh after an update: codes, scales and per-row flip counts bit-exact."""
    Wp0, Wp1 = _refresh_case(N, K, qt, seed=N * 13 + K)
    c0, _, _ = O.requantize_weights(Wp0, qt)
    c1, s1, f1 = O.requantize_weights(Wp1, qt, codes_old=c0)
    assert f1.sum() > 0
    Wq = to_dev_codes(c0, qt)
    rf = _row_flips(N)
    _, sw = B.requantize_weights(to_dev_f32(Wp1), qt, Wq, row_flips=rf)
    torch.cuda.synchronize()
    assert np.array_equal(codes_np(Wq), c1.view(np.uint8))
    assert np.array_equal(sw.cpu().numpy(), s1)
    assert np.array_equal(rf.cpu().numpy().astype(np.int64), f1)
    # without counts: the same codes
    Wq2 = to_dev_codes(c0, qt)
    _, sw2 = B.requantize_weights(to_dev_f32(Wp1), qt, Wq2)
    torch.cuda.synchronize()
    assert np.array_equal(codes_np(Wq2), c1.view(np.uint8))
    assert np.array_equal(sw2.cpu().numpy(), s1)


@pytest.mark.parametrize("qt", QTS)
def test_requantize_strided_params_and_repeat(qt):
    """Row stride > K; counts are written, so a second refresh of unchanged
    parameters reports zero changes per row."""
    N, K, ld = 96, 512, 640
    Wp0, Wp1 = _refresh_case(N, K, qt, seed=77, ld=ld)
    c0, _, _ = O.requantize_weights(Wp0[:, :K], qt)
    c1, s1, f1 = O.requantize_weights(Wp1[:, :K], qt, codes_old=c0)
    Wq = to_dev_codes(c0, qt)
    Wd = to_dev_f32(Wp1)[:, :K]
    rf = _row_flips(N)
    B.requantize_weights(Wd, qt, Wq, row_flips=rf)
    torch.cuda.synchronize()
    assert np.array_equal(rf.cpu().numpy().astype(np.int64), f1)
    B.requantize_weights(Wd, qt, Wq, row_flips=rf)
    torch.cuda.synchronize()
    assert not rf.cpu().numpy().any()
    assert np.array_equal(codes_np(Wq), c1.view(np.uint8))


def test_requantize_fp8_signed_zero_is_no_flip():
    """E4M3FN +0 and -0 are one value: previous codes planted with the other
    zero, or with random other codes, give exactly the oracle's counts."""
    N, K = 64, 256
    rng = np.random.default_rng(5)
    Wp = np.zeros((N, K), np.float32)
    Wp[:, 0] = 1.0  # absmax 1 per row: v = 448 w
    tiny = rng.choice(np.array([-1e-9, 1e-9, 0.0, -0.0], np.float32), size=(N, K - 1))
    Wp[:, 1:] = tiny
    Wp[::3, 1:] += rng.normal(0, 0.05, size=(len(range(0, N, 3)), K - 1)).astype(np.float32)
    c1, s1, _ = O.requantize_weights(Wp, "fp8")
    zeros = (c1 & 0x7F) == 0
    assert zeros.sum() > 1000 and ((c1 == 0x80).sum() > 100) and ((c1 == 0x00).sum() > 100)
    prev = c1.copy()
    prev[zeros] ^= 0x80  # the other zero everywhere: no flips
    other = rng.random(prev.shape) < 0.02
    prev[other] = rng.integers(0, 0x7F, size=int(other.sum()), dtype=np.uint8)  # some real changes
    expect = O.count_flips_rows(prev, c1, "fp8")
    assert 0 < expect.sum() <= other.sum()
    Wq = to_dev_codes(prev, "fp8")
    rf = _row_flips(N)
    _, sw = B.requantize_weights(to_dev_f32(Wp), "fp8", Wq, row_flips=rf)
    torch.cuda.synchronize()
    assert np.array_equal(codes_np(Wq), c1)
    assert np.array_equal(sw.cpu().numpy(), s1)
    assert np.array_equal(rf.cpu().numpy().astype(np.int64), expect)


def test_requantize_rejects_bad_arguments():
    Wp = torch.zeros((4, 64), dtype=torch.float32, device=DEV)
    Wq = torch.zeros((4, 64), dtype=torch.int8, device=DEV)
    with pytest.raises(ValueError):
        B.requantize_weights(Wp, "int8", Wq.view(torch.float8_e4m3fn))
    with pytest.raises(ValueError):
        B.requantize_weights(Wp, "int8", Wq, row_flips=torch.zeros(4, dtype=torch.int64, device=DEV))
    with pytest.raises(ValueError):
        B.requantize_weights(Wp, "int8", Wq, row_flips=torch.zeros(3, dtype=torch.int32, device=DEV))
    with pytest.raises(B.QRError):
        B.requantize_weights(torch.zeros((4, 66), dtype=torch.float32, device=DEV)[:, :64], "int8",
                             Wq)
