"""Shared helpers of the GPU parity tests (host-side marshalling only)."""

import numpy as np
import torch

from oracle import formats as F

DEV = "cuda:0"


def to_dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def to_dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)


def to_dev_codes(codes, qt):
    t = torch.from_numpy(np.ascontiguousarray(codes).view(np.int8)).to(DEV)
    return t if qt == "int8" else t.view(torch.float8_e4m3fn)


def codes_np(t):
    return t.view(torch.uint8).cpu().numpy()


def bf16_np(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def f32_of_bits(bits):
    return F.bf16_bits_to_f32(bits).astype(np.float64)


def assert_bf16_close(y_bits, ref_bits, rel=1e-2, what=""):
    """Spec tolerance on bf16 outputs, read as: elementwise
    |y - ref| <= rel*|ref| + rel*rms(ref), and ||y - ref||_F <= rel*||ref||_F."""
    y = f32_of_bits(y_bits)
    r = f32_of_bits(ref_bits)
    rms = np.sqrt(np.mean(r * r)) if r.size else 0.0
    err = np.abs(y - r)
    bad = err > rel * np.abs(r) + rel * rms
    assert not bad.any(), f"{what}: {bad.sum()} elements outside tolerance, max err {err.max()}"
    assert np.linalg.norm(y - r) <= rel * np.linalg.norm(r) + 1e-30, what
    return int(np.count_nonzero(y_bits != ref_bits))


def fp8_acc_bound(Xq, Wq):
    """Bound on the device's FP8 accumulators against the exact sums.

    The gfx950 FP8 MFMA (every form: 16x16x32 fp8, 16x16x128 / 32x32x64
    f8f6f4) adds the products of a group of k at reduced precision: bits far
    below the group's largest product are dropped (measured: 448 plus seven
    2^-9 terms in one group returns 448; on random data the error stayed below
    2^-16.5 of sum_k |x_k w_k|). Allowed here: 2^-12 of sum |x w| for that, plus
    the worst-case fp32 summation error of any order, (K-1) 2^-24 sum |x w|.
    """
    dx = np.abs(F.e4m3fn_decode(Xq))
    dw = np.abs(F.e4m3fn_decode(Wq))
    K = Xq.shape[1]
    return (2.0 ** -12 + max(K - 1, 1) * 2.0 ** -24) * (dx @ dw.T)


def assert_bf16_close_fro(y_bits, ref_bits, rel, what=""):
    """End-to-end form of the tolerance, for chains whose inputs already differ
    upstream: ||y - ref||_F <= rel ||ref||_F only. Returns the relative
    Frobenius error and the number of elements outside the elementwise
    1e-2 bound, for the report."""
    y = f32_of_bits(y_bits)
    r = f32_of_bits(ref_bits)
    nr = max(float(np.linalg.norm(r)), 1e-30)
    e = float(np.linalg.norm(y - r)) / nr
    assert e <= rel, (what, e)
    rms = np.sqrt(np.mean(r * r)) if r.size else 0.0
    return e, int(np.count_nonzero(np.abs(y - r) > 1e-2 * np.abs(r) + 1e-2 * rms))
