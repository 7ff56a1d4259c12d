"""GPU parity of block-wise FP8 (power-of-two block scales) against the oracle.

Codes and E8M0 scales must be bit-identical. The product is compared as fp32
accumulators against the exact block sums within the FP8 MFMA's accumulation
bound (products of a group added at reduced precision, groups in fp32), with
every product scaled by its two block scales; bf16 outputs must be the
rounding of the device's own accumulators and within the benchmark spec's tolerance
of the oracle's.
"""

import numpy as np
import pytest
import torch

import oracle as O
from oracle import formats as F
from w8a8_gemm_rl_amd import binding as B
from w8a8_gemm_rl_amd import inputs as I

from gpu_helpers import DEV, assert_bf16_close, bf16_np, codes_np, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu


def _rowmajor(ds, R, K):
    # device scale panels [ceil(K/128), R, 4] -> [R, K/32]
    s = ds.cpu().numpy()
    return s.transpose(1, 0, 2).reshape(R, -1)[:, : K // 32]


def _scaled(codes, X):
    return F.e4m3fn_decode(codes) * np.repeat(2.0 ** X.astype(np.float64), 32, axis=1)


@pytest.mark.parametrize("R,K", [(64, 512), (37, 96), (3, 32), (300, 3584), (5, 18944)])
def test_mx_quantize_weights_and_activations_bit_exact(R, K):
    W = I.weights(R, K, 0.02, seed=R + K)
    W[min(1, R - 1), :32] = 0.0  # an all-zero block
    W[0, :4] = [3e38, -1e-38, 1e-45, -0.0]  # huge, subnormal-range and signed zero elements
    codes, X = O.mx_quantize_rows(W)
    dc, ds = B.mx_quantize(to_dev_f32(W))
    torch.cuda.synchronize()
    assert np.array_equal(codes_np(dc), codes)
    assert np.array_equal(_rowmajor(ds, R, K), (X + 127).astype(np.uint8))
    Xb = I.activations(R, K, seed=R * 3 + K, kind="outliers" if K >= 100 else "normal")
    codes, X = O.mx_quantize_rows(F.bf16_bits_to_f32(Xb))
    dc, ds = B.mx_quantize(to_dev_bf16(Xb))
    torch.cuda.synchronize()
    assert np.array_equal(codes_np(dc), codes)
    assert np.array_equal(_rowmajor(ds, R, K), (X + 127).astype(np.uint8))


def _mx_operands(M, N, K, seed, rows=None):
    Xb = I.activations(M, K, seed=seed, kind="outliers")
    W = I.weights(N, K, 0.02, seed=seed + 1)
    xc, xe = O.mx_quantize_rows(F.bf16_bits_to_f32(Xb))
    dxc, dxs = B.mx_quantize(to_dev_bf16(Xb))
    dwc, dws = B.mx_quantize(to_dev_f32(W))
    Wh = W if rows is None else W[rows]
    wc, we = O.mx_quantize_rows(Wh)
    return (xc, xe, wc, we), (dxc, dxs, dwc, dws)


@pytest.mark.parametrize("M,N,K", [(16, 512, 512), (32, 200, 384), (45, 136, 1024), (1, 64, 128),
                                   (256, 384, 3584), (100, 4608, 3584), (33, 130, 256), (7, 203, 128)])
def test_mx_gemm_against_exact_block_sums(M, N, K):
    (xc, xe, wc, we), (dxc, dxs, dwc, dws) = _mx_operands(M, N, K, seed=M * 7 + N + K)
    acc, y = O.mx_linear(xc, xe, wc, we)
    raw = B.mx_gemm(dxc, dxs, dwc, dws, out="raw")
    yd = B.mx_gemm(dxc, dxs, dwc, dws, out="bf16")
    torch.cuda.synchronize()
    a = raw.cpu().numpy().astype(np.float64)
    bound = (2.0 ** -12 + (K - 1) * 2.0 ** -24) * (np.abs(_scaled(xc, xe)) @ np.abs(_scaled(wc, we)).T)
    assert np.all(np.abs(a - acc) <= bound + 1e-30)
    assert np.array_equal(bf16_np(yd), F.f32_to_bf16_bits(raw.cpu().numpy()))
    assert_bf16_close(bf16_np(yd), y, what=f"mx {M}x{N}x{K}")


@pytest.mark.parametrize("M", [256, 32, 7])
def test_mx_gemm_7b_gate_sampled_channels(M):
    """The 7B gate at M = 256 (8-wave 192 x 128 tiles), 32 and 7 (128 x 32 tiles owning
    80 of their 128 rows, so the grid fills the CUs), full size on the device; 512 sampled
    output channels (a channel's codes, scales and outputs depend only on its own weight
    row)."""
    N, K = 18944, 3584
    rows = np.unique(np.r_[0, np.random.default_rng(4).choice(N, 510, replace=False), N - 1])
    (xc, xe, wc, we), (dxc, dxs, dwc, dws) = _mx_operands(M, N, K, seed=99, rows=rows)
    assert np.array_equal(codes_np(dwc)[rows], wc)
    acc, y = O.mx_linear(xc, xe, wc, we)
    raw = B.mx_gemm(dxc, dxs, dwc, dws, out="raw")
    torch.cuda.synchronize()
    a = raw.cpu().numpy()[:, rows].astype(np.float64)
    bound = (2.0 ** -12 + (K - 1) * 2.0 ** -24) * (np.abs(_scaled(xc, xe)) @ np.abs(_scaled(wc, we)).T)
    assert np.all(np.abs(a - acc) <= bound + 1e-30)


@pytest.mark.parametrize("M,N,K,pad", [(40, 130, 256, 6), (9, 130, 384, 6), (9, 64, 384, 1)])
def test_mx_gemm_strided_output(M, N, K, pad):
    """Y with padded rows and ragged N, on both tile shapes (up to 32 tokens and above): a
    stride that is a multiple of 8 elements (bf16 staged through LDS into 16-byte stores,
    the last piece of a row partial) or one that is not a multiple of 4 (outputs stored one
    by one). The same values as into a packed Y of stride N = 130 or 64 (the other store
    path), and the padding left untouched."""
    (xc, xe, wc, we), (dxc, dxs, dwc, dws) = _mx_operands(M, N, K, seed=M + N + pad)
    for out, dt in (("bf16", torch.bfloat16), ("raw", torch.float32)):
        big = torch.full((M, N + pad), -7.0, dtype=dt, device=DEV)
        B.mx_gemm(dxc, dxs, dwc, dws, out=out, Y=big[:, :N])
        packed = B.mx_gemm(dxc, dxs, dwc, dws, out=out)
        torch.cuda.synchronize()
        assert torch.equal(big[:, :N], packed), out
        assert bool((big[:, N:] == -7.0).all()), out


def test_mx_rejects_bad_shapes():
    W = torch.zeros((4, 48), dtype=torch.float32, device=DEV)
    with pytest.raises(B.QRError):
        B.mx_quantize(W)  # K not a multiple of 32
    c, s = B.mx_quantize(torch.zeros((4, 96), dtype=torch.float32, device=DEV))
    with pytest.raises(B.QRError):
        B.mx_gemm(c, s, c, s)  # K not a multiple of 128
    c, s = B.mx_quantize(torch.zeros((4, 128), dtype=torch.float32, device=DEV))
    Y = torch.empty(4 * 4 + 1, dtype=torch.bfloat16, device=DEV)[1:].view(4, 4)
    with pytest.raises(B.QRError):
        B.mx_gemm(c, s, c, s, Y=Y)  # output not on a 16-byte boundary
    z, zs = B.mx_quantize(torch.zeros((0, 128), dtype=torch.float32, device=DEV))
    assert z.shape == (0, 128)
