"""Number formats used by the W8A8 path, written from their definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* bfloat16: the top 16 bits of an IEEE binary32 (1 sign, 8 exponent, 7
  fraction bits). Widening bf16 -> fp32 is exact; narrowing fp32 -> bf16 is
  round-to-nearest, ties to the value whose last fraction bit is 0.
* FP8 E4M3FN (OCP 8-bit floating point, "E4M3"): 1 sign, 4 exponent bits with
  bias 7, 3 mantissa bits. Exponent field 0 encodes subnormals m/8 * 2^-6; the
  pattern S.1111.111 is NaN; there is no infinity, so the largest finite value
  is 1.75 * 2^8 = 448. The paper-notes page ("Loss / training strategy") says
  only "FP8"; E4M3 with the OCP "fn" encoding is the reading taken, being the
  FP8 format the rollout linear is specified in and the native one of the
  target GPU.

The encoders here are deliberately naive: they enumerate the candidate values
of the target format and pick the nearest one, so a reader can check them
against the definitions above without following any bit tricks.
"""

import numpy as np

E4M3FN_MAX = 448.0


# ----------------------------------------------------------------------------
# bfloat16
# ----------------------------------------------------------------------------

def bf16_bits_to_f32(bits):
    """Widen bf16 bit patterns (uint16) to float32: place them in the top half."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def f32_to_bf16_bits(x):
    """Round float32 values to bf16, nearest with ties to even; return uint16 bits.

    For each x the two bf16 neighbours are found: ``lo`` (x with its low 16
    bits cleared, i.e. truncated toward zero) and ``hi`` (the next bf16 value
    away from zero). The nearer one wins; on an exact tie the one with an even
    last fraction bit wins. Inputs must be finite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("f32_to_bf16_bits: non-finite input")
    bits = x.view(np.uint32)
    lo = bits & np.uint32(0xFFFF0000)
    hi = lo + np.uint32(0x10000)            # next magnitude up, same sign
    ax = np.abs(x.astype(np.float64))
    vlo = np.abs(lo.view(np.float32).astype(np.float64))
    vhi = np.abs(hi.view(np.float32).astype(np.float64))
    # hi may be the infinity pattern; its "value" for the distance is 2^128.
    vhi = np.where(np.isinf(vhi), 2.0 ** 128, vhi)
    d_lo = ax - vlo
    d_hi = vhi - ax
    lo_odd = ((lo >> np.uint32(16)) & np.uint32(1)) == 1
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & lo_odd)
    out = np.where(take_hi, hi, lo) >> np.uint32(16)
    return out.astype(np.uint16)


# ----------------------------------------------------------------------------
# FP8 E4M3FN
# ----------------------------------------------------------------------------

def e4m3fn_decode(codes):
    """Decode E4M3FN bytes to float64 from the field definition (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = (m / 8.0) * 2.0 ** -6
    nrm = (1.0 + m / 8.0) * np.power(2.0, (e - 7).astype(np.float64))
    mag = np.where(e == 0, sub, nrm)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


_CHUNK = 1 << 18

# The 127 finite non-negative values, codes 0x00..0x7E, increasing.
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALUES = e4m3fn_decode(_POS_CODES)
assert np.all(np.diff(_POS_VALUES) > 0)
assert _POS_VALUES[-1] == E4M3FN_MAX


def e4m3fn_encode(x):
    """Round float32 values in [-448, 448] to E4M3FN, nearest with ties to even.

    Among the finite E4M3FN magnitudes the nearest to |x| is taken (distances in
    float64, exact for these operands); on a tie the code with mantissa LSB 0
    wins. The sign bit is the sign bit of x, so -0.0 and negative values that
    round to zero give 0x80. Values outside [-448, 448] are rejected: the
    quantizer saturates before it encodes.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("e4m3fn_encode: non-finite input")
    if x.size > _CHUNK:  # same result, processed in cache-sized pieces
        flat = x.reshape(-1)
        out = np.empty(flat.shape, np.uint8)
        for i in range(0, flat.size, _CHUNK):
            out[i:i + _CHUNK] = e4m3fn_encode(flat[i:i + _CHUNK])
        return out.reshape(x.shape)
    ax = np.abs(x.astype(np.float64))
    if np.any(ax > E4M3FN_MAX):
        raise ValueError("e4m3fn_encode: |x| > 448 (saturate first)")
    vals = _POS_VALUES
    idx_hi = np.searchsorted(vals, ax, side="left")        # first value >= ax
    idx_hi = np.minimum(idx_hi, len(vals) - 1)
    idx_lo = np.maximum(idx_hi - 1, 0)
    exact = vals[idx_hi] == ax
    d_lo = ax - vals[idx_lo]
    d_hi = vals[idx_hi] - ax
    hi_even = (_POS_CODES[idx_hi] & 1) == 0
    take_hi = exact | (d_hi < d_lo) | ((d_hi == d_lo) & hi_even)
    mag_code = np.where(take_hi, _POS_CODES[idx_hi], _POS_CODES[idx_lo])
    sign = np.signbit(x).astype(np.uint8) << np.uint8(7)
    return (mag_code.astype(np.uint8) | sign).astype(np.uint8)
