"""Pins for the oracle's number formats (bf16 and FP8 E4M3FN codecs).

The codecs are checked against the format definition's tabulated reference
points (OCP OFP8 spec, tests/golden/e4m3fn_reference_points.json), by
exhaustive round trips, by brute-force nearest-value search and against
torch's independent CPU casts.
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_e4m3_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_e4m3fn_reference_points():
    with open(os.path.join(GOLDEN, "e4m3fn_reference_points.json")) as f:
        ref = json.load(f)
    for p in ref["points"]:
        got = F.e4m3fn_decode(np.array([p["code"]], np.uint8))[0]
        if p["value"] == "nan":
            assert np.isnan(got), p
        else:
            assert got == p["value"], p
            assert np.signbit(got) == np.signbit(p["value"]), p
    assert F.E4M3FN_MAX == 448.0


def test_e4m3fn_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e4m3fn_decode(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(theirs)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], theirs[~nan])
    assert nan.sum() == 2  # only S.1111.111: no infinities in the fn encoding


def test_e4m3fn_roundtrip_every_finite_code():
    codes = np.arange(256, dtype=np.uint8)
    vals = F.e4m3fn_decode(codes)
    fin = ~np.isnan(vals)
    back = F.e4m3fn_encode(vals[fin].astype(np.float32))
    assert np.array_equal(back, codes[fin])


def test_e4m3fn_encode_is_nearest_by_brute_force():
    g = np.random.default_rng(1)
    x = np.concatenate([
        g.uniform(-448, 448, 20000),
        g.uniform(-1, 1, 20000),
        g.uniform(-0.02, 0.02, 20000),
    ]).astype(np.float32)
    enc = F.e4m3fn_encode(x)
    dec = F.e4m3fn_decode(enc)
    allv = F.e4m3fn_decode(np.arange(256, dtype=np.uint8))
    allv = allv[~np.isnan(allv)]
    best = np.abs(x.astype(np.float64)[:, None] - allv[None, :]).min(axis=1)
    assert np.array_equal(np.abs(dec - x.astype(np.float64)), best)


def test_e4m3fn_ties_to_even_at_every_midpoint():
    vals = F.e4m3fn_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2  # exact in float64 and float32 here
    assert np.all(mids.astype(np.float32).astype(np.float64) == mids)
    enc = F.e4m3fn_encode(mids.astype(np.float32))
    lo = np.arange(0x7E, dtype=np.uint8)
    expect = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)
    assert np.array_equal(enc, expect)
    assert np.array_equal(F.e4m3fn_encode(-mids.astype(np.float32)), expect | 0x80)


def test_e4m3fn_encode_matches_torch_cast():
    g = np.random.default_rng(2)
    x = np.concatenate([
        g.uniform(-448, 448, 400000),
        (g.standard_normal(400000) * 3).clip(-448, 448),
        g.uniform(-2 ** -6, 2 ** -6, 200000),
    ]).astype(np.float32)
    vals = F.e4m3fn_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1000)])
    x = x[np.abs(x) <= 448]
    assert np.array_equal(F.e4m3fn_encode(x), _torch_e4m3_bits(x))


def test_e4m3fn_encode_boundaries():
    # 2^-10 is the midpoint between 0 and the smallest subnormal: ties to 0.
    assert F.e4m3fn_encode(np.float32([2.0 ** -10]))[0] == 0x00
    assert F.e4m3fn_encode(np.float32([np.nextafter(np.float32(2 ** -10), 1)]))[0] == 0x01
    assert F.e4m3fn_encode(np.float32([-2.0 ** -10]))[0] == 0x80
    assert F.e4m3fn_encode(np.float32([448.0]))[0] == 0x7E
    with pytest.raises(ValueError):
        F.e4m3fn_encode(np.float32([448.5]))


def test_bf16_widen_is_exact_top_half():
    bits = np.array([0x3F80, 0xBF80, 0x0001, 0x7F7F, 0x8000], np.uint16)
    f = F.bf16_bits_to_f32(bits)
    assert f[0] == 1.0 and f[1] == -1.0 and f[3] == np.float32(3.3895314e38)
    assert np.signbit(f[4]) and f[4] == 0
    assert f[2] == np.float32(2.0 ** -133)


def test_bf16_round_matches_torch_and_ties():
    g = np.random.default_rng(3)
    x = np.concatenate([
        g.standard_normal(500000).astype(np.float32),
        (g.standard_normal(100000) * 1e30).astype(np.float32),
        (g.standard_normal(100000) * 1e-30).astype(np.float32),
    ])
    # exact ties: low 16 bits 0x8000, with even and odd kept parts
    tb = (g.integers(0x0080, 0x7F00, 4000).astype(np.uint32) << 16) | 0x8000
    x = np.concatenate([x, tb.view(np.float32), -tb.view(np.float32)])
    ours = F.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    # direct tie cases: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1.0)
    assert F.f32_to_bf16_bits(np.float32([1 + 2 ** -8]))[0] == 0x3F80
    # 1 + 3*2^-8 is halfway between 1+2^-7 (odd) and 1+2^-6 (even) -> up
    assert F.f32_to_bf16_bits(np.float32([1 + 3 * 2 ** -8]))[0] == 0x3F82


def test_bf16_round_is_nearest_by_brute_force():
    g = np.random.default_rng(4)
    x = g.standard_normal(5000).astype(np.float32)
    b = F.f32_to_bf16_bits(x)
    y = F.bf16_bits_to_f32(b).astype(np.float64)
    # neighbours one bf16 step either side must not be nearer
    up = F.bf16_bits_to_f32((b.astype(np.int32) + 1).astype(np.uint16)).astype(np.float64)
    dn = F.bf16_bits_to_f32((b.astype(np.int32) - 1).astype(np.uint16)).astype(np.float64)
    d = np.abs(y - x)
    assert np.all(d <= np.abs(up - x)) and np.all(d <= np.abs(dn - x))
