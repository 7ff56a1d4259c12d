"""The QuRL W8A8 linear, step by step, in plain numpy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Shapes follow torch.nn.Linear: weights W are [N, K] (output channel n, input
feature k), activations X are [M, K] (token m), outputs Y are [M, N].
Y[m, n] ~= sum_k X[m, k] * W[n, k].

Notation: Q = 127 for INT8 and 448 (the E4M3FN maximum) for FP8; fl32(.) is
IEEE binary32 rounding of one operation. numpy float32 array arithmetic is
exactly that (one correctly-rounded operation per operator, no FMA
contraction), which is why the fp32 steps below are written as one numpy
operator each.
"""

from fractions import Fraction

import numpy as np

from .formats import (
    E4M3FN_MAX,
    bf16_bits_to_f32,
    e4m3fn_decode,
    e4m3fn_encode,
    f32_to_bf16_bits,
)

# Reading of the pages: the quantization step maps the row's absmax to the
# largest code. INT8 is symmetric (+-127, -128 never produced), 2^(b-1) - 1 for
# b = 8; FP8 uses the format's largest finite value.
QMAX = {"int8": 127.0, "fp8": E4M3FN_MAX}


def _check_qt(qt):
    if qt not in QMAX:
        raise ValueError(f"unknown qtype {qt!r}")


# ----------------------------------------------------------------------------
# UAQ: update-aware invariant scaling
# ----------------------------------------------------------------------------

def uaq_reparameterize(W, s, gamma=None, beta=None):
    """One-time UAQ reparameterization (paper notes, "Key designs > UAQ").

    The linear map is unchanged by W X = (W / s)(s X). The weight is divided by
    s (the same scalar for every input column k: "column-wise"), and the factor
    s on the activation side is absorbed by the norm that produces X, whose
    gain (and LayerNorm bias) is multiplied by s. The pages fix s = 1.5
    ("Loss / training strategy").

    Float arrays are processed in fp32 (one division / multiplication each);
    arrays of ``fractions.Fraction`` are processed exactly, which is how the
    invariance itself is checked.
    Returns (W', gamma', beta') with None for absent norm parameters.
    """
    W = np.asarray(W)
    if W.dtype == object:
        s_ = Fraction(s)
        Wp = W / s_
        gp = None if gamma is None else np.asarray(gamma, dtype=object) * s_
        bp = None if beta is None else np.asarray(beta, dtype=object) * s_
        return Wp, gp, bp
    s32 = np.float32(s)
    Wp = np.asarray(W, dtype=np.float32) / s32
    gp = None if gamma is None else np.asarray(gamma, dtype=np.float32) * s32
    bp = None if beta is None else np.asarray(beta, dtype=np.float32) * s32
    return Wp, gp, bp


# ----------------------------------------------------------------------------
# Absmax row quantization (weights per output channel, activations per token)
# ----------------------------------------------------------------------------

def quantize_rows(A, qt):
    """Symmetric absmax quantization of each row of a float32 matrix.

    Per row r (paper notes, "Loss / training strategy": channel-wise weights,
    token-wise activations):
        a_r     = max_k |A[r, k]|                      (exact)
        scale_r = fl32(a_r / Q)
        v       = fl32(A[r, k] / scale_r)
        INT8:  code = clamp(round_half_even(v), -127, 127)
        FP8:   code = E4M3FN(clamp(v, -448, 448)), nearest, ties to even
    A row of zeros gets scale 0 and all codes 0 (reading: the pages are silent).
    Returns (codes, scale): int8 codes, or uint8 E4M3FN bytes; float32 scales.
    """
    _check_qt(qt)
    A = np.ascontiguousarray(A, dtype=np.float32)
    if A.ndim != 2:
        raise ValueError("quantize_rows expects a 2-D matrix")
    if not np.all(np.isfinite(A)):
        raise ValueError("quantize_rows: non-finite input")
    Q = np.float32(QMAX[qt])
    R, K = A.shape
    a = np.abs(A).max(axis=1) if K > 0 else np.zeros(R, np.float32)
    scale = (a / Q).astype(np.float32)
    zero = scale == 0
    safe = np.where(zero, np.float32(1), scale).astype(np.float32)
    v = (A / safe[:, None]).astype(np.float32)
    if qt == "int8":
        codes = np.clip(np.rint(v), -127, 127).astype(np.int8)
        codes[zero] = 0
    else:
        v = np.clip(v, -E4M3FN_MAX, E4M3FN_MAX).astype(np.float32)
        codes = e4m3fn_encode(v)
        codes[zero] = 0
    return codes, scale


def quantize_weights_uaq(W, s, qt, gamma=None, beta=None):
    """theta -> theta_hat for the rollout actor (paper notes, "Overall framework").

    W' = fl32(W / s) (UAQ; s = 1 for the per-step re-quantization of weights
    that were reparameterized once already), then per-output-channel absmax
    quantization of W'. Returns dict(Wq, scale_w, W_scaled, gamma, beta).
    """
    Wp, gp, bp = uaq_reparameterize(np.asarray(W, np.float32), s, gamma, beta)
    codes, scale = quantize_rows(Wp, qt)
    return {"Wq": codes, "scale_w": scale, "W_scaled": Wp, "gamma": gp, "beta": bp}


def quantize_act_per_token(X_bits, act_mult, qt):
    """Per-token absmax quantization of bf16 activations.

    The codes are those of quantize_rows(X). ``act_mult`` carries the UAQ
    factor s onto the activation side for a linear whose input is not produced
    by a norm that absorbed s (reading: with absmax quantization the codes of
    sX equal the codes of X, so s only multiplies the scale):
        scale_x = fl32(fl32(a_m / Q) * act_mult)
    Returns (codes, scale_x).
    """
    X = bf16_bits_to_f32(X_bits)
    codes, scale = quantize_rows(X, qt)
    scale_x = (scale * np.float32(act_mult)).astype(np.float32)
    return codes, scale_x


# ----------------------------------------------------------------------------
# Producers fused with the per-token quantization (the step before the linear)
# ----------------------------------------------------------------------------
#
# Paper notes, "Method > Key designs > UAQ": the activation-side factor s is
# merged into the norm that produces the linear's input (gain gamma' = gamma*s,
# bias beta' = beta*s). The pages do not fix the norm's own arithmetic; the
# reading taken: the per-row statistic is computed in float64 and rounded to
# fp32 once, every later step is fp32 in the order written. The norm output is
# quantized as fp32 (a fused kernel never stores it as bf16).

def _row_stat_f32(x64):
    return np.asarray(x64, np.float64).astype(np.float32)


def norm_folded(H_bits, gamma_s, beta_s=None, eps=1e-6, kind="rms"):
    """Norm of bf16 rows with the UAQ-folded gain (and bias), per row h:

    kind "rms":   ms = sum_k h_k^2 / K                        (float64)
                  r  = fl32(1 / sqrt(ms + eps))               (float64, one rounding;
                                                               eps is an fp32 value)
                  y_k = fl32(fl32(h_k * r) * gamma'_k) [+ beta'_k, fl32]
    kind "layer": mu = fl32(sum_k h_k / K)                    (float64, one rounding)
                  var = sum_k (h_k - mu)^2 / K                (float64, mu as rounded)
                  r  = fl32(1 / sqrt(var + eps))              (float64, one rounding)
                  y_k = fl32(fl32(fl32(h_k - mu) * r) * gamma'_k) [+ beta'_k, fl32]
    Returns (y float32 [M, K], r float32 [M]).
    """
    if kind not in ("rms", "layer"):
        raise ValueError("kind must be 'rms' or 'layer'")
    H = bf16_bits_to_f32(H_bits).astype(np.float32)
    M, K = H.shape
    if K == 0:
        return np.zeros((M, 0), np.float32), np.zeros(M, np.float32)
    g = np.asarray(gamma_s, np.float32)
    H64 = H.astype(np.float64)
    if kind == "rms":
        ms = (H64 * H64).sum(axis=1) / K
        d = H
    else:
        mu = _row_stat_f32(H64.sum(axis=1) / K)
        dev = H64 - mu.astype(np.float64)[:, None]
        ms = (dev * dev).sum(axis=1) / K
        d = (H - mu[:, None]).astype(np.float32)
    r = _row_stat_f32(1.0 / np.sqrt(ms + float(np.float32(eps))))
    y = ((d * r[:, None]).astype(np.float32) * g[None, :]).astype(np.float32)
    if beta_s is not None:
        y = (y + np.asarray(beta_s, np.float32)[None, :]).astype(np.float32)
    return y, r


def norm_quant(H_bits, gamma_s, beta_s=None, eps=1e-6, kind="rms", qt="int8"):
    """The folded norm followed by per-token quantization of its fp32 output.
    s already sits in gamma' (and beta'), so the scale carries no extra factor
    (reading R9's norm-fed case). Returns (codes, scale_x)."""
    y, _ = norm_folded(H_bits, gamma_s, beta_s, eps, kind)
    return quantize_rows(y, qt)


def silu_mul(G_bits, U_bits):
    """SiLU(gate) times up, a = fl32(g * u / (1 + exp(-g))) evaluated in
    float64 from the bf16 inputs (g * u is exact there; exp overflow gives a
    signed zero)."""
    g = bf16_bits_to_f32(G_bits).astype(np.float64)
    u = bf16_bits_to_f32(U_bits).astype(np.float64)
    with np.errstate(over="ignore"):
        a = (g * u) / (1.0 + np.exp(-g))
    return a.astype(np.float32)


def silu_mul_quant(G_bits, U_bits, act_mult, qt):
    """silu_mul followed by per-token quantization; act_mult carries s for the
    down projection, whose input no norm produces (reading R9).
    Returns (codes, scale_x) with scale_x = fl32(fl32(a_m / Q) * act_mult)."""
    a = silu_mul(G_bits, U_bits)
    codes, t = quantize_rows(a, qt)
    return codes, (t * np.float32(act_mult)).astype(np.float32)


# ----------------------------------------------------------------------------
# Quantized product and dequantization
# ----------------------------------------------------------------------------

def acc_int8(Xq, Wq):
    """Exact int32 accumulators acc[m, n] = sum_k Xq[m, k] * Wq[n, k].

    Computed as a float64 matrix product, which is exact here: every product
    and every partial sum is an integer of magnitude <= K * 127^2 < 2^53, so no
    summation order or FMA can round. The result must fit int32 (it does for
    K <= 133152).
    """
    acc = np.asarray(Xq, np.float64) @ np.asarray(Wq, np.float64).T
    if acc.size and np.abs(acc).max() >= 2.0 ** 31:
        raise OverflowError("int8 accumulator exceeds int32")
    return acc.astype(np.int64).astype(np.int32)


def acc_fp8(Xq, Wq):
    """Exact accumulators sum_k dec(Xq[m, k]) * dec(Wq[n, k]) in float64.

    Each E4M3FN value is a multiple of 2^-9 with magnitude <= 448, so a product
    is a multiple of 2^-18 of magnitude < 2^17.61 and a K-term sum stays below
    2^(17.61 + log2 K); for K <= 2^33 every partial sum fits the 53-bit float64
    significand, hence the float64 product is exact in any order.
    """
    dx = e4m3fn_decode(Xq)
    dw = e4m3fn_decode(Wq)
    if np.isnan(dx).any() or np.isnan(dw).any():
        raise ValueError("acc_fp8: NaN code in input")
    return dx @ dw.T


def dequant_epilogue(acc, scale_x, scale_w):
    """y = bf16(fl32(fl32(fl32(acc) * scale_x[m]) * scale_w[n])).

    The order of the two scale multiplications and the absence of FMA are the
    reading taken (the pages do not spell out the epilogue; the output dtype is
    the bf16 of the baseline model). fl32(acc) is round-to-nearest-even of the
    exact accumulator.
    Returns (y_f32, y_bf16_bits).
    """
    a32 = np.asarray(acc, np.float64).astype(np.float32)
    t = (a32 * np.asarray(scale_x, np.float32)[:, None]).astype(np.float32)
    y = (t * np.asarray(scale_w, np.float32)[None, :]).astype(np.float32)
    return y, f32_to_bf16_bits(y)


def w8a8_linear(X_bits, Wq, scale_w, act_mult, qt):
    """One quantized linear: per-token quantization, quantized product, epilogue."""
    _check_qt(qt)
    Xq, sx = quantize_act_per_token(X_bits, act_mult, qt)
    acc = acc_int8(Xq, Wq) if qt == "int8" else acc_fp8(Xq, Wq)
    y32, ybits = dequant_epilogue(acc, sx, scale_w)
    return {"Xq": Xq, "scale_x": sx, "acc": acc, "y_f32": y32, "y": ybits}


# ----------------------------------------------------------------------------
# Decode-layer chain
# ----------------------------------------------------------------------------

def decode_chain(x0_bits, layers, qt):
    """Run a list of quantized linears back to back.

    ``layers`` is a sequence of dicts with keys name, src (``"x0"`` or an earlier
    layer's name), cols (None or (start, stop): the column slice of src taken as
    input), Wq, scale_w, act_mult. Each linear quantizes its bf16 input per
    token and hands its bf16 output on. Returns {name: w8a8_linear result}.
    """
    outs = {}
    for L in layers:
        src = x0_bits if L["src"] == "x0" else outs[L["src"]]["y"]
        if L.get("cols") is not None:
            c0, c1 = L["cols"]
            src = src[:, c0:c1]
        outs[L["name"]] = w8a8_linear(src, L["Wq"], L["scale_w"], L["act_mult"], qt)
    return outs


# ----------------------------------------------------------------------------
# The update-masking experiment (paper notes, "Key designs > UAQ", motivation)
# ----------------------------------------------------------------------------

def _changed(a, b, qt):
    """Positions whose code now stands for a different value.

    INT8: codes differ. FP8 (E4M3FN bytes): codes differ, except that +0
    (0x00) and -0 (0x80) are the same value (reading: a sign change below
    the smallest step is no change of the quantized weight).
    """
    diff = a != b
    if qt == "fp8":
        diff &= ~(((a | b) == 0x80) & ((a & b) == 0))
    return diff


def count_flips(codes_old, codes_new, qt):
    """Number of positions whose code now stands for a different value."""
    _check_qt(qt)
    a = np.asarray(codes_old).view(np.uint8).reshape(-1)
    b = np.asarray(codes_new).view(np.uint8).reshape(-1)
    if a.shape != b.shape:
        raise ValueError("count_flips: shapes differ")
    return int(np.count_nonzero(_changed(a, b, qt)))


def count_flips_rows(codes_old, codes_new, qt):
    """count_flips of each row (output channel) of two [N, K] code matrices."""
    _check_qt(qt)
    a = np.asarray(codes_old).view(np.uint8)
    b = np.asarray(codes_new).view(np.uint8)
    if a.ndim != 2 or a.shape != b.shape:
        raise ValueError("count_flips_rows: two [N, K] matrices of one shape expected")
    return _changed(a, b, qt).sum(axis=1, dtype=np.int64)


def requantize_weights(Wp, qt, codes_old=None):
    """Per-RL-step refresh theta_old -> theta_hat_old (paper notes, "Overall
    framework"; the stored parameter is already W' = W / s under UAQ, so s = 1
    here): per-output-channel quantization of W', and per channel the number
    of codes that changed since the previous refresh (codes_old), if given.
    Returns (codes, scale, row_flips or None)."""
    codes, scale = quantize_rows(Wp, qt)
    flips = None if codes_old is None else count_flips_rows(codes_old, codes, qt)
    return codes, scale, flips


def flip_counts(W, dW, s, qt):
    """Count weight codes changed by a small update, with and without UAQ.

    The pages: RL updates (~1e-7) are far below the quantization step, so the
    quantized actor barely sees them; UAQ divides the stored weight by s (the
    step shrinks by s) while the update on that stored parameter grows by s.
    Where the update lands under UAQ is read three ways:
        base      codes(W + dW)          vs codes(W)
        uaq_same  codes(W/s + dW)        vs codes(W/s)    same-size update
        uaq_pages codes(W/s + s*dW)      vs codes(W/s)    the pages' s*alpha*G
        control   codes(W/s + dW/s)      vs codes(W/s)    same effective update
    All sums and products are fp32. Returns the four counts and the size.
    """
    W = np.asarray(W, np.float32)
    dW = np.asarray(dW, np.float32)
    s32 = np.float32(s)

    def codes(A):
        return quantize_rows(A, qt)[0]

    c0 = codes(W)
    Ws = (W / s32).astype(np.float32)
    cs = codes(Ws)
    out = {
        "base": count_flips(c0, codes((W + dW).astype(np.float32)), qt),
        "uaq_same": count_flips(cs, codes((Ws + dW).astype(np.float32)), qt),
        "uaq_pages": count_flips(cs, codes((Ws + (dW * s32).astype(np.float32)).astype(np.float32)),
                                 qt),
        "control": count_flips(cs, codes((Ws + (dW / s32).astype(np.float32)).astype(np.float32)),
                               qt),
        "n": int(W.size),
    }
    return out


def _fp8_code_step(v):
    """Spacing of E4M3FN values around code-space value v (|v| <= 448)."""
    av = np.abs(v)
    e = np.floor(np.log2(np.maximum(av, 2.0 ** -6)))
    return np.where(av < 2.0 ** -6, 2.0 ** -9, 2.0 ** (e - 3))


def flip_expectation(W, sigma, qt):
    """First-order expected number of changed codes under W + dW, dW ~ N(0, sigma^2).

    Closed form: element (n, k) sits at code-space value v = W[n,k] / scale_n.
    The update moves it by dW[n,k] / scale_n, and moves the row's scale through
    the absmax element, which shifts v by -v * dW[n,kmax] * sign / a_n. The two
    shifts are independent normals, so the total has standard deviation
    sigma * sqrt(1/scale_n^2 + v^2/a_n^2) and crosses a rounding boundary
    (boundaries are spaced one code step h(v) apart, the offset is uniform) with
    probability E|shift| / h(v) = sqrt(2/pi) * sd / h(v). INT8: h = 1; FP8:
    h = the E4M3FN spacing at v. The absmax element itself never moves (its v
    is pinned at +-Q). Valid when sigma is far below one step.
    """
    _check_qt(qt)
    W = np.asarray(W, np.float64)
    Q = QMAX[qt]
    a = np.abs(W).max(axis=1, keepdims=True)
    scale = a / Q
    v = W / scale
    sd = sigma * np.sqrt(1.0 / scale ** 2 + v ** 2 / a ** 2)
    h = np.ones_like(v) if qt == "int8" else _fp8_code_step(v)
    p = np.sqrt(2.0 / np.pi) * sd / h
    p[np.abs(W) == a] = 0.0
    return float(p.sum())


# ----------------------------------------------------------------------------
# Adaptive clipping range with truncated importance sampling (trainer side)
# ----------------------------------------------------------------------------

def acr_tis_loss(logp, logp_prox, logp_behav, adv, mask, eps, C):
    """Per-token ACR objective (paper notes, "Method > Key designs > ACR") as a
    loss, in float64.

    Per token: R = pi / pi_prox = exp(logp - logp_prox) (the clipping ratio,
    against the full-precision old actor), r = pi_prox / pi_behav =
    exp(logp_prox - logp_behav) (full-precision against the quantized actor
    that sampled the token; reading of the pages' r_{i,t}), w = min(r, C)
    (the truncated importance weight), and
        term = min(R A, clip(R, 1 - eps, (1 + eps) / r) A),
        clip(x, lo, hi) = min(max(x, lo), hi)   (hi wins if hi < lo),
        loss = -w term,  dloss/dlogp = -w A R where the first branch is the
        minimum (R inside the clip range, or clipping would raise the term),
        0 where the clipped branch is strictly smaller.
    Masked tokens (mask == 0) give 0 and are not counted.
    Returns (loss [n], grad [n], loss_sum, n_valid, n_clipped) where n_clipped
    counts valid tokens whose gradient the clip removes.
    """
    lp = np.asarray(logp, np.float64)
    lx = np.asarray(logp_prox, np.float64)
    lb = np.asarray(logp_behav, np.float64)
    A = np.asarray(adv, np.float64)
    m = np.asarray(mask).astype(bool)
    R = np.exp(lp - lx)
    r = np.exp(lx - lb)
    w = np.minimum(r, float(C))
    lo, hi = 1.0 - float(eps), (1.0 + float(eps)) / r
    Rc = np.minimum(np.maximum(R, lo), hi)
    u, c = R * A, Rc * A
    unclipped = u <= c
    loss = np.where(m, -w * np.minimum(u, c), 0.0)
    grad = np.where(m & unclipped, -w * u, 0.0)
    return loss, grad, float(loss[m].sum()), int(m.sum()), int((m & ~unclipped).sum())


# ----------------------------------------------------------------------------
# Block-wise FP8 with power-of-two block scales (the block-wise variant the
# pages cite, in the form CDNA4's matrix cores scale natively)
# ----------------------------------------------------------------------------

MX_BLOCK = 32


def mx_exponent(amax):
    """Smallest integer X with amax <= 448 * 2^X (so no element of the block
    saturates), clamped to [-127, 127]; amax = 0 gives -127. Exact: with
    amax = f 2^e, f in [0.5, 1) and 448 = 0.875 2^9, X = e - 9 if f <= 0.875
    else e - 8."""
    a = np.asarray(amax, np.float64)
    f, e = np.frexp(a)
    X = np.where(f <= 0.875, e - 9, e - 8)
    X = np.where(a == 0, -127, X)
    return np.clip(X, -127, 127).astype(np.int16)


def mx_quantize_rows(A, block=MX_BLOCK):
    """Block-wise FP8: every `block` consecutive elements of a row share one
    power-of-two scale 2^X (X = mx_exponent of the block's absmax; E8M0 byte
    X + 127), and each element is the E4M3FN code of fl32(v * 2^-X) (the
    scaling is exact for normal results), nearest with ties to even. Reading:
    the pages cite block-wise FP8 without a block size or scale format; the
    block of 32 and the power-of-two scale are those of the gfx950 scaled MFMA.
    Returns (codes uint8 [R, K], X int16 [R, K / block])."""
    A = np.ascontiguousarray(A, dtype=np.float32)
    R, K = A.shape
    if K % block:
        raise ValueError("K must be a multiple of the block")
    Ab = A.reshape(R, K // block, block).astype(np.float64)
    X = mx_exponent(np.abs(Ab).max(axis=2) if K else np.zeros((R, 0)))
    v = np.ldexp(Ab, -X[:, :, None].astype(np.int64)).astype(np.float32)
    v = np.clip(v, -E4M3FN_MAX, E4M3FN_MAX)
    codes = e4m3fn_encode(v.reshape(R, K))
    return codes, X


def mx_linear(Xc, Xe, Wc, We, block=MX_BLOCK):
    """acc[m, n] = sum_b 2^(Xe[m, b] + We[n, b]) sum_{k in b} x_k w_k with the
    decoded E4M3FN values; every block partial is exact in float64 (products
    are multiples of 2^-18 below 2^17.61, 32 of them), scaled exactly, and the
    blocks are added in float64. Y = bf16_rne(fl32(acc)).
    Returns (acc float64 [M, N], Y bf16 bits)."""
    x = e4m3fn_decode(Xc)
    w = e4m3fn_decode(Wc)
    M, K = x.shape
    N = w.shape[0]
    nb = K // block
    acc = np.zeros((M, N), np.float64)
    for b in range(nb):
        part = x[:, b * block:(b + 1) * block] @ w[:, b * block:(b + 1) * block].T
        acc += np.ldexp(part, (Xe[:, b:b + 1].astype(np.int64) + We[None, :, b].astype(np.int64)))
    return acc, f32_to_bf16_bits(acc.astype(np.float32))

