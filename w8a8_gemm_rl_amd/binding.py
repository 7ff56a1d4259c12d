"""Thin ctypes binding over libqurl_w8a8.so (C ABI in include/qurl_w8a8.h).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the computation runs in the library's kernels. If
the shared library is missing this module raises -- there is no fallback.

Function names mirror the C entry points without the ``qr_`` prefix.
"""

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; QR_LIB_PATH names another build of the same library to
# load instead (the CPU tests use it for the host-sanitizer build).
LIB_PATH = os.environ.get("QR_LIB_PATH") or os.path.join(_HERE, "libqurl_w8a8.so")

QT = {"int8": 0, "fp8": 1}
OUT = {"bf16": 0, "raw": 1}
NORM = {"rms": 0, "layer": 1}
STATUS = {
    0: "QR_OK", -1: "QR_ERR_INVALID_ARG", -2: "QR_ERR_UNSUPPORTED", -3: "QR_ERR_WORKSPACE",
    -4: "QR_ERR_HIP", -5: "QR_ERR_NO_DEVICE",
}
# Every function include/qurl_w8a8.h declares.
EXPORTS = [
    "qr_quantize_weights_uaq", "qr_requantize_weights", "qr_quantize_act_per_token",
    "qr_norm_quant", "qr_silu_mul_quant", "qr_acr_tis_loss", "qr_mx_quantize", "qr_mx_gemm",
    "qr_w8a8_gemm", "qr_w8a8_gemm_quant", "qr_linear_fused", "qr_linear_fused_noalloc",
    "qr_workspace_size", "qr_gemm_plan", "qr_tile_name", "qr_num_tiles", "qr_set_plan_override",
    "qr_set_small_m_override", "qr_set_fuse_override", "qr_last_error", "qr_version", "qr_probe_read", "qr_probe_mfma",
    "qr_probe_copy_stream",
]


class QRError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None
_lock = threading.Lock()

_i64, _f32, _vp, _int, _sz = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_SIGS = {
    "qr_quantize_weights_uaq": (_int, [_vp, _i64, _i64, _i64, _f32, _int, _vp, _vp, _vp, _vp, _vp, _vp]),
    "qr_requantize_weights": (_int, [_vp, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp]),
    "qr_quantize_act_per_token": (_int, [_vp, _i64, _i64, _i64, _f32, _int, _vp, _vp, _vp]),
    "qr_norm_quant": (_int, [_vp, _i64, _i64, _i64, _int, _vp, _vp, _f32, _int, _vp, _vp, _vp]),
    "qr_silu_mul_quant": (_int, [_vp, _vp, _i64, _i64, _i64, _i64, _f32, _int, _vp, _vp, _vp]),
    "qr_acr_tis_loss": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _f32, _f32, _vp, _vp, _vp, _vp, _sz,
                               _vp]),
    "qr_mx_quantize": (_int, [_vp, _i64, _i64, _i64, _int, _vp, _vp, _vp]),
    "qr_mx_gemm": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _vp, _i64, _vp]),
    "qr_w8a8_gemm": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _vp, _i64, _vp, _sz, _vp]),
    "qr_w8a8_gemm_quant": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _vp, _i64, _i64, _i64,
                                  _f32, _vp, _vp, _vp, _sz, _vp]),
    "qr_linear_fused": (_int, [_vp, _i64, _f32, _vp, _vp, _i64, _i64, _i64, _int, _vp, _i64, _vp, _sz, _vp]),
    "qr_linear_fused_noalloc": (_int, [_vp, _i64, _f32, _vp, _vp, _i64, _i64, _i64, _int, _vp, _i64,
                                       _vp]),
    "qr_workspace_size": (_sz, [ctypes.c_char_p, _i64, _i64, _i64, _int]),
    "qr_gemm_plan": (_int, [_i64, _i64, _i64, _int, ctypes.POINTER(_int), ctypes.POINTER(_int),
                            ctypes.POINTER(_int)]),
    "qr_tile_name": (ctypes.c_char_p, [_int]),
    "qr_num_tiles": (_int, []),
    "qr_set_plan_override": (_int, [_int, _int, _int]),
    "qr_set_small_m_override": (_int, [_int]),
    "qr_set_fuse_override": (_int, [_int]),
    "qr_last_error": (ctypes.c_char_p, []),
    "qr_probe_read": (_int, [_vp, _sz, _vp, _i64, _vp]),
    "qr_probe_mfma": (_int, [_int, _int, _int, _vp, _vp, ctypes.POINTER(_int), _vp]),
    "qr_probe_copy_stream": (_int, [_int, _vp, _i64, _i64, _vp, _i64, _i64, _i64, _int, _int, _vp, _i64, _vp]),
    "qr_version": (ctypes.c_char_p, []),
}


def lib():
    """Load (once) and return the shared library; raise if it is not built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is not built: run `python -m w8a8_gemm_rl_amd.build`")
                L = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in _SIGS.items():
                    f = getattr(L, name)
                    f.restype = res
                    f.argtypes = args
                _lib = L
    return _lib


def _check(fn, status):
    if status != 0:
        msg = lib().qr_last_error().decode(errors="replace")
        raise QRError(fn, status, msg)


def _qt(qt):
    if qt not in QT:
        raise ValueError(f"qt must be one of {list(QT)}, got {qt!r}")
    return QT[qt]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on a HIP device")


def _rows(t, name):
    """Leading dimension of a 2-D tensor whose rows are contiguous."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with contiguous rows")
    if t.shape[0] <= 1:  # the row stride of a single row is arbitrary
        return max(t.shape[1], 1)
    return t.stride(0)


def code_dtype(qt):
    return torch.int8 if qt == "int8" else torch.float8_e4m3fn


# ----------------------------------------------------------------------------
# Workspace: one scratch buffer per (device, stream), grown on demand. Calls on
# one stream are ordered, so they may share it; calls on different streams may
# run at the same time and get different buffers. A buffer that is outgrown is
# kept alive (never freed): a HIP graph captured earlier may still write into
# it on every replay, and the caching allocator must not hand its memory to
# another tensor.
# ----------------------------------------------------------------------------
_ws = {}
_ws_retired = []


def workspace(nbytes, device):
    if nbytes == 0:
        return None, 0
    dev = torch.device(device)
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    key = (idx, torch.cuda.current_stream(idx).cuda_stream)
    buf = _ws.get(key)
    if buf is None or buf.numel() < nbytes:
        if buf is not None:
            _ws_retired.append(buf)
        buf = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=torch.device("cuda", idx))
        _ws[key] = buf
    return buf, buf.numel()


# ----------------------------------------------------------------------------
# Entry points
# ----------------------------------------------------------------------------

def version():
    return lib().qr_version().decode()


def num_tiles():
    return lib().qr_num_tiles()


def tile_name(i):
    r = lib().qr_tile_name(i)
    return None if r is None else r.decode()


def set_plan_override(tile=-1, splitk=0, rows=0):
    _check("qr_set_plan_override", lib().qr_set_plan_override(tile, splitk, rows))


def set_small_m_override(rf=0):
    """One-launch decode path of linear_fused at 1-4 tokens: 0 automatic,
    -1 off, 1..5 blocks of 16 * rf output channels (calling thread only)."""
    _check("qr_set_small_m_override", lib().qr_set_small_m_override(rf))


def set_fuse_override(mode=0):
    """w8a8_gemm_quant: 0 separate launches (default), 1 the one-launch
    grid-barrier path where the plan allows (calling thread only)."""
    _check("qr_set_fuse_override", lib().qr_set_fuse_override(mode))


def gemm_plan(M, N, K, qt):
    """(tile, splitk, rows) of the plan qr_w8a8_gemm uses for this shape."""
    t, s, r = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check("qr_gemm_plan", lib().qr_gemm_plan(M, N, K, _qt(qt), ctypes.byref(t), ctypes.byref(s),
                                              ctypes.byref(r)))
    return t.value, s.value, r.value


def workspace_size(fn, M, N, K, qt):
    r = lib().qr_workspace_size(fn.encode(), M, N, K, _qt(qt))
    if r == ctypes.c_size_t(-1).value:
        raise QRError("qr_workspace_size", -1, lib().qr_last_error().decode())
    return r


def quantize_weights_uaq(W, s, qt, Wq=None, scale_w=None, W_scaled=None, gamma=None, beta=None):
    """W [N, K] fp32 (rows contiguous) -> (Wq [N, K], scale_w [N]) on W's device."""
    _need_cuda(W, Wq, scale_w, W_scaled, gamma, beta)
    if W.dtype != torch.float32:
        raise ValueError("W must be float32")
    N, K = W.shape
    ldw = _rows(W, "W")
    if Wq is None:
        Wq = torch.empty((N, K), dtype=code_dtype(qt), device=W.device)
    if scale_w is None:
        scale_w = torch.empty(N, dtype=torch.float32, device=W.device)
    if W_scaled is not None and (W_scaled.shape != W.shape or _rows(W_scaled, "W_scaled") != ldw):
        raise ValueError("W_scaled must have W's shape and row stride")
    with torch.cuda.device(W.device):
        st = lib().qr_quantize_weights_uaq(_ptr(W), N, K, ldw, float(s), _qt(qt), _ptr(Wq),
                                           _ptr(scale_w), _ptr(W_scaled), _ptr(gamma), _ptr(beta),
                                           _stream(W.device))
    _check("qr_quantize_weights_uaq", st)
    return Wq, scale_w


def requantize_weights(Wp, qt, Wq, scale_w=None, row_flips=None):
    """Refresh the codes of stored parameters Wp = W / s [N, K] fp32 in place in Wq.

    With row_flips (an int32 device tensor of N entries) entry n receives the
    number of codes of row n whose value changed. Returns (Wq, scale_w).
    """
    _need_cuda(Wp, Wq, scale_w, row_flips)
    if Wp.dtype != torch.float32:
        raise ValueError("Wp must be float32")
    N, K = Wp.shape
    ldw = _rows(Wp, "Wp")
    if Wq.shape != (N, K) or Wq.dtype != code_dtype(qt) or not Wq.is_contiguous():
        raise ValueError("Wq must be a contiguous [N, K] code tensor of the quantized type")
    if scale_w is None:
        scale_w = torch.empty(N, dtype=torch.float32, device=Wp.device)
    if row_flips is not None and (row_flips.dtype != torch.int32 or row_flips.numel() != N
                                  or not row_flips.is_contiguous()):
        raise ValueError("row_flips must be a contiguous int32 tensor of N entries")
    with torch.cuda.device(Wp.device):
        st = lib().qr_requantize_weights(_ptr(Wp), N, K, ldw, _qt(qt), _ptr(Wq), _ptr(scale_w),
                                         _ptr(row_flips), _stream(Wp.device))
    _check("qr_requantize_weights", st)
    return Wq, scale_w


def norm_quant(H, gamma, qt, beta=None, eps=1e-6, kind="rms", Xq=None, scale_x=None):
    """Norm of bf16 rows H [M, K] with the folded gain gamma (= gamma*s, fp32 [K]) and
    optional folded bias beta, fused with per-token quantization -> (Xq, scale_x)."""
    _need_cuda(H, gamma, beta, Xq, scale_x)
    if H.dtype != torch.bfloat16:
        raise ValueError("H must be bfloat16")
    if kind not in NORM:
        raise ValueError(f"kind must be one of {list(NORM)}")
    M, K = H.shape
    ldh = _rows(H, "H")
    for name, t in (("gamma", gamma), ("beta", beta)):
        if t is not None and (t.dtype != torch.float32 or t.numel() != K or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 tensor of K entries")
    if Xq is None:
        Xq = torch.empty((M, K), dtype=code_dtype(qt), device=H.device)
    if scale_x is None:
        scale_x = torch.empty(M, dtype=torch.float32, device=H.device)
    with torch.cuda.device(H.device):
        st = lib().qr_norm_quant(_ptr(H), M, K, ldh, NORM[kind], _ptr(gamma), _ptr(beta),
                                 float(eps), _qt(qt), _ptr(Xq), _ptr(scale_x), _stream(H.device))
    _check("qr_norm_quant", st)
    return Xq, scale_x


def silu_mul_quant(G, U, act_mult, qt, Xq=None, scale_x=None):
    """SiLU(G) * U for bf16 [M, N] views (rows contiguous, any row strides), fused with
    per-token quantization; scale_x carries act_mult -> (Xq, scale_x)."""
    _need_cuda(G, U, Xq, scale_x)
    if G.dtype != torch.bfloat16 or U.dtype != torch.bfloat16:
        raise ValueError("G and U must be bfloat16")
    if G.shape != U.shape:
        raise ValueError("G and U must have one shape")
    M, N = G.shape
    ldg, ldu = _rows(G, "G"), _rows(U, "U")
    if Xq is None:
        Xq = torch.empty((M, N), dtype=code_dtype(qt), device=G.device)
    if scale_x is None:
        scale_x = torch.empty(M, dtype=torch.float32, device=G.device)
    with torch.cuda.device(G.device):
        st = lib().qr_silu_mul_quant(_ptr(G), _ptr(U), M, N, ldg, ldu, float(act_mult), _qt(qt),
                                     _ptr(Xq), _ptr(scale_x), _stream(G.device))
    _check("qr_silu_mul_quant", st)
    return Xq, scale_x


def acr_tis_loss(logp, logp_prox, logp_behav, adv, mask, eps, C, loss=None, grad=None,
                 with_grad=True):
    """Per-token ACR / TIS loss on fp32 [n] tensors and a uint8 mask ->
    (loss [n], grad [n] or None, sums float64 [3] = loss sum, valid, clipped)."""
    ts = (logp, logp_prox, logp_behav, adv)
    _need_cuda(*ts, mask, loss, grad)
    n = logp.numel()
    for t in ts:
        if t.dtype != torch.float32 or t.numel() != n or not t.is_contiguous():
            raise ValueError("log-probabilities and advantages must be contiguous float32 of one size")
    if mask.dtype != torch.uint8 or mask.numel() != n or not mask.is_contiguous():
        raise ValueError("mask must be a contiguous uint8 tensor of the same size")
    dev = logp.device
    if loss is None:
        loss = torch.empty(n, dtype=torch.float32, device=dev)
    if grad is None and with_grad:
        grad = torch.empty(n, dtype=torch.float32, device=dev)
    sums = torch.empty(3, dtype=torch.float64, device=dev)
    ws, ws_bytes = workspace(workspace_size("qr_acr_tis_loss", n, 0, 0, "int8"), dev)
    with torch.cuda.device(dev):
        st = lib().qr_acr_tis_loss(*(_ptr(t) for t in ts), _ptr(mask), n, float(eps), float(C),
                                   _ptr(loss), _ptr(grad), _ptr(sums), _ptr(ws), ws_bytes,
                                   _stream(dev))
    _check("qr_acr_tis_loss", st)
    return loss, grad, sums


def mx_quantize(A, codes=None, scales=None):
    """Block-wise FP8 of fp32 or bf16 rows A [R, K] -> (codes [R, K] fp8, E8M0 scales uint8
    [ceil(K/128), R, 4]: scales[p, r, j] belongs to 32-element block 4 p + j of row r)."""
    _need_cuda(A, codes, scales)
    if A.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("A must be float32 or bfloat16")
    R, K = A.shape
    lda = _rows(A, "A")
    if codes is None:
        codes = torch.empty((R, K), dtype=torch.float8_e4m3fn, device=A.device)
    if scales is None:
        scales = torch.empty(((K + 127) // 128, R, 4), dtype=torch.uint8, device=A.device)
    with torch.cuda.device(A.device):
        st = lib().qr_mx_quantize(_ptr(A), R, K, lda, int(A.dtype == torch.bfloat16), _ptr(codes),
                                  _ptr(scales), _stream(A.device))
    _check("qr_mx_quantize", st)
    return codes, scales


def mx_gemm(Xq, sx, Wq, sw, out="bf16", Y=None):
    """Block-wise FP8 product: Y [M, N] = bf16(acc) or the fp32 accumulators."""
    _need_cuda(Xq, sx, Wq, sw, Y)
    M, K = Xq.shape
    N = Wq.shape[0]
    P = (K + 127) // 128
    if Wq.shape[1] != K or sx.shape != (P, M, 4) or sw.shape != (P, N, 4):
        raise ValueError("operand shapes do not match")
    for t in (Xq, sx, Wq, sw):
        if not t.is_contiguous():
            raise ValueError("operands must be contiguous")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16 if out == "bf16" else torch.float32,
                        device=Xq.device)
    ldy = _rows(Y, "Y")
    with torch.cuda.device(Xq.device):
        st = lib().qr_mx_gemm(_ptr(Xq), _ptr(sx), _ptr(Wq), _ptr(sw), M, N, K, OUT[out], _ptr(Y),
                              ldy, _stream(Xq.device))
    _check("qr_mx_gemm", st)
    return Y


def quantize_act_per_token(X, act_mult, qt, Xq=None, scale_x=None):
    """X [M, K] bf16 (rows contiguous, any row stride) -> (Xq [M, K], scale_x [M])."""
    _need_cuda(X, Xq, scale_x)
    if X.dtype != torch.bfloat16:
        raise ValueError("X must be bfloat16")
    M, K = X.shape
    ldx = _rows(X, "X")
    if Xq is None:
        Xq = torch.empty((M, K), dtype=code_dtype(qt), device=X.device)
    if scale_x is None:
        scale_x = torch.empty(M, dtype=torch.float32, device=X.device)
    with torch.cuda.device(X.device):
        st = lib().qr_quantize_act_per_token(_ptr(X), M, K, ldx, float(act_mult), _qt(qt), _ptr(Xq),
                                             _ptr(scale_x), _stream(X.device))
    _check("qr_quantize_act_per_token", st)
    return Xq, scale_x


def w8a8_gemm(Xq, scale_x, Wq, scale_w, qt, out="bf16", Y=None, ws=None):
    """Y = dequant(Xq @ Wq^T): bf16 [M, N], or raw int32 / fp32 accumulators."""
    _need_cuda(Xq, scale_x, Wq, scale_w, Y)
    M, K = Xq.shape
    N = Wq.shape[0]
    if Wq.shape[1] != K:
        raise ValueError("Xq and Wq disagree on K")
    if Y is None:
        dt = torch.bfloat16 if out == "bf16" else (torch.int32 if qt == "int8" else torch.float32)
        Y = torch.empty((M, N), dtype=dt, device=Xq.device)
    ldy = _rows(Y, "Y")
    need = workspace_size("qr_w8a8_gemm", M, N, K, qt)
    if ws is None:
        ws, wsb = workspace(need, Xq.device)
    else:
        wsb = ws.numel() * ws.element_size()
    with torch.cuda.device(Xq.device):
        st = lib().qr_w8a8_gemm(_ptr(Xq), _ptr(scale_x), _ptr(Wq), _ptr(scale_w), M, N, K, _qt(qt),
                                OUT[out], _ptr(Y), ldy, _ptr(ws), wsb, _stream(Xq.device))
    _check("qr_w8a8_gemm", st)
    return Y


_wsq = {}


def quant_workspace(nbytes, device):
    """The binding's workspace for qr_w8a8_gemm_quant: one zeroed buffer per
    (device, stream), separate from the other calls' (its header must stay
    as the fused launches leave it); outgrown buffers are kept alive."""
    if nbytes == 0:
        return None, 0
    dev = torch.device(device)
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    key = (idx, torch.cuda.current_stream(idx).cuda_stream)
    buf = _wsq.get(key)
    if buf is None or buf.numel() < nbytes:
        if buf is not None:
            _ws_retired.append(buf)
        buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=torch.device("cuda", idx))
        _wsq[key] = buf
    return buf, buf.numel()


def w8a8_gemm_quant(Xq, scale_x, Wq, scale_w, qt, Y=None, q_cols=None, q_act_mult=1.0,
                    Xq_next=None, scale_x_next=None, ws=None):
    """Y = dequant(Xq @ Wq^T) in bf16, and (q_cols = (c0, c1)) the per-token
    quantization of Y[:, c0:c1] with q_act_mult -> (Y, Xq_next, scale_x_next).
    `ws`, if given, must be a workspace zeroed once when allocated and used
    only by this call."""
    _need_cuda(Xq, scale_x, Wq, scale_w, Y, Xq_next, scale_x_next)
    M, K = Xq.shape
    N = Wq.shape[0]
    if Wq.shape[1] != K:
        raise ValueError("Xq and Wq disagree on K")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=Xq.device)
    ldy = _rows(Y, "Y")
    c0, c1 = (0, 0) if q_cols is None else q_cols
    if q_cols is not None:
        if Xq_next is None:
            Xq_next = torch.empty((M, c1 - c0), dtype=code_dtype(qt), device=Xq.device)
        if scale_x_next is None:
            scale_x_next = torch.empty(M, dtype=torch.float32, device=Xq.device)
    need = workspace_size("qr_w8a8_gemm_quant", M, N, K, qt)
    if ws is None:
        ws, wsb = quant_workspace(need, Xq.device)
    else:
        wsb = ws.numel() * ws.element_size()
    with torch.cuda.device(Xq.device):
        st = lib().qr_w8a8_gemm_quant(_ptr(Xq), _ptr(scale_x), _ptr(Wq), _ptr(scale_w), M, N, K,
                                      _qt(qt), _ptr(Y), ldy, c0, c1 - c0, float(q_act_mult),
                                      _ptr(Xq_next), _ptr(scale_x_next), _ptr(ws), wsb,
                                      _stream(Xq.device))
    _check("qr_w8a8_gemm_quant", st)
    return Y, Xq_next, scale_x_next


def linear_fused(X, act_mult, Wq, scale_w, qt, Y=None, ws=None):
    """One rollout linear: per-token quantization of bf16 X, W8A8 product, bf16 Y."""
    _need_cuda(X, Wq, scale_w, Y)
    if X.dtype != torch.bfloat16:
        raise ValueError("X must be bfloat16")
    M, K = X.shape
    N = Wq.shape[0]
    ldx = _rows(X, "X")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    ldy = _rows(Y, "Y")
    need = workspace_size("qr_linear_fused", M, N, K, qt)
    if ws is None:
        ws, wsb = workspace(need, X.device)
    else:
        wsb = ws.numel() * ws.element_size()
    with torch.cuda.device(X.device):
        st = lib().qr_linear_fused(_ptr(X), ldx, float(act_mult), _ptr(Wq), _ptr(scale_w), M, N, K,
                                   _qt(qt), _ptr(Y), ldy, _ptr(ws), wsb, _stream(X.device))
    _check("qr_linear_fused", st)
    return Y


def linear_fused_noalloc(X, act_mult, Wq, scale_w, qt, Y=None):
    """linear_fused with the library's fixed device scratch instead of a
    workspace: the call allocates nothing (Y must be given to avoid torch's
    own allocation)."""
    _need_cuda(X, Wq, scale_w, Y)
    if X.dtype != torch.bfloat16:
        raise ValueError("X must be bfloat16")
    M, K = X.shape
    N = Wq.shape[0]
    ldx = _rows(X, "X")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    ldy = _rows(Y, "Y")
    with torch.cuda.device(X.device):
        st = lib().qr_linear_fused_noalloc(_ptr(X), ldx, float(act_mult), _ptr(Wq), _ptr(scale_w),
                                           M, N, K, _qt(qt), _ptr(Y), ldy, _stream(X.device))
    _check("qr_linear_fused_noalloc", st)
    return Y


# ----------------------------------------------------------------------------
# Measurement helpers (peaks the chip reaches; not part of the linear)
# ----------------------------------------------------------------------------

def probe_read(buf, sink=None):
    """Enqueue one read of the whole byte buffer `buf` (a contiguous device
    tensor whose size is a multiple of 16 bytes); returns the sink tensor."""
    _need_cuda(buf, sink)
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.empty(2048, dtype=torch.int32, device=buf.device)
    with torch.cuda.device(buf.device):
        st = lib().qr_probe_read(_ptr(buf), nbytes, _ptr(sink), sink.numel(), _stream(buf.device))
    _check("qr_probe_read", st)
    return sink


PROBE_PANEL, PROBE_NO_BARRIER, PROBE_RESIDENT = 1, 2, 4


def probe_copy_stream(tile, Wq, Xq, rows, sink=None, panel=False, barrier=True, resident=False):
    """Enqueue the operand copies GEMM tile `tile` (4, 8 or 10) makes over the
    8-bit code matrices Wq [N, K] and Xq [M, K] (rows contiguous; their row
    strides are passed on) with `rows` weight rows per tile, without the
    matrix work; panel reads Wq's bytes as K panels instead (Wq contiguous),
    barrier=False drops the barrier per K step, resident=True copies K step
    0's bytes at every step (operands resident in L2). Returns the sink
    tensor (one word per block)."""
    _need_cuda(Wq, Xq, sink)
    if Wq.dim() != 2 or Xq.dim() != 2 or Wq.shape[1] != Xq.shape[1]:
        raise ValueError("Wq [N, K] and Xq [M, K] with the same K expected")
    if Wq.element_size() != 1 or Xq.element_size() != 1:
        raise ValueError("8-bit code matrices expected")
    if panel and not Wq.is_contiguous():
        raise ValueError("panel reads need a contiguous Wq")
    (N, K), M = Wq.shape, Xq.shape[0]
    ldw, ldx = _rows(Wq, "Wq"), _rows(Xq, "Xq")
    bm = {4: 256, 8: 128, 10: 256}.get(tile, 1)
    grid = -(-N // max(rows, 1)) * -(-M // bm)
    if sink is None:
        sink = torch.empty(max(grid, 1), dtype=torch.int32, device=Wq.device)
    flags = ((PROBE_PANEL if panel else 0) | (0 if barrier else PROBE_NO_BARRIER)
             | (PROBE_RESIDENT if resident else 0))
    with torch.cuda.device(Wq.device):
        st = lib().qr_probe_copy_stream(tile, _ptr(Wq), N, ldw, _ptr(Xq), M, ldx, K, rows, flags,
                                        _ptr(sink), sink.numel(), _stream(Wq.device))
    _check("qr_probe_copy_stream", st)
    return sink


def probe_mfma(qt, blocks, iters, device="cuda:0", sink=None, ticks=None):
    """Enqueue the MFMA probe; returns (sink, ticks, wall clock rate in kHz)."""
    dev = torch.device(device)
    if sink is None:
        sink = torch.empty(8 * blocks, dtype=torch.int32, device=dev)
    if ticks is None:
        ticks = torch.empty(4 * blocks, dtype=torch.int64, device=dev)
    khz = ctypes.c_int(0)
    with torch.cuda.device(dev):
        st = lib().qr_probe_mfma(_qt(qt), blocks, iters, _ptr(sink), _ptr(ticks), ctypes.byref(khz),
                                 _stream(dev))
    _check("qr_probe_mfma", st)
    return sink, ticks, khz.value
