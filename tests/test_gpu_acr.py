"""GPU parity of the per-token ACR / TIS loss against the float64 oracle.

The device computes in fp32 (exp, one division, products), so losses and
gradients are compared to a relative tolerance of 1e-5; where R lies within
1e-5 (relative) of a clip bound the two precisions may pick different
branches of the min, and the gradient (which jumps there) is compared only
elsewhere. Valid-token counts are exact; clipped-token counts may differ by at
most the number of such tokens; the float64 sums are reproducible bit for bit.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from w8a8_gemm_rl_amd import binding as B
from w8a8_gemm_rl_amd import inputs as I

from gpu_helpers import DEV

pytestmark = pytest.mark.gpu


def _dev(b):
    return {k: torch.from_numpy(v).to(DEV) for k, v in b.items()}


def _near_kink(b, eps):
    R = np.exp(b["logp"].astype(np.float64) - b["logp_prox"])
    r = np.exp(b["logp_prox"].astype(np.float64) - b["logp_behav"])
    return (np.abs(R - (1 - eps)) <= 1e-5 * R) | (np.abs(R - (1 + eps) / r) <= 1e-5 * R)


def _run(b, eps, C, with_grad=True):
    d = _dev(b)
    loss, grad, sums = B.acr_tis_loss(d["logp"], d["logp_prox"], d["logp_behav"], d["adv"],
                                      d["mask"], eps, C, with_grad=with_grad)
    torch.cuda.synchronize()
    return (loss.cpu().numpy(), None if grad is None else grad.cpu().numpy(),
            sums.cpu().numpy())


@pytest.mark.parametrize("n_seq,max_len,C", [(8, 16, I.ACR_C), (3, 37, I.ACR_C),
                                             (64, 1000, float("inf")), (512, 8192, I.ACR_C)])
def test_acr_loss_matches_oracle(n_seq, max_len, C):
    eps = I.ACR_EPS
    b = I.acr_batch(n_seq, max_len, seed=n_seq * 7 + max_len)
    loss, grad, s, nv, nc = O.acr_tis_loss(b["logp"], b["logp_prox"], b["logp_behav"], b["adv"],
                                           b["mask"], eps, C)
    dl, dg, ds = _run(b, eps, C)
    assert np.allclose(dl, loss, rtol=1e-5, atol=1e-7)
    kink = _near_kink(b, eps)
    assert kink.mean() < 1e-3
    ok = ~kink
    assert np.allclose(dg[ok], grad[ok], rtol=1e-5, atol=1e-7)
    assert ds[1] == nv
    assert abs(ds[2] - nc) <= int((kink & (b["mask"] == 1)).sum())
    assert ds[0] == pytest.approx(s, rel=1e-6, abs=1e-6)
    assert not dl[b["mask"] == 0].any() and not dg[b["mask"] == 0].any()
    # the sums are the same bits on a second run
    assert np.array_equal(_run(b, eps, C)[2], ds)


def test_acr_without_gradient_and_masked_batch():
    b = I.acr_batch(4, 33, seed=9)
    dl, dg, ds = _run(b, 0.2, 2.0, with_grad=False)
    assert dg is None
    loss, _, s, nv, _ = O.acr_tis_loss(b["logp"], b["logp_prox"], b["logp_behav"], b["adv"],
                                       b["mask"], 0.2, 2.0)
    assert np.allclose(dl, loss, rtol=1e-5, atol=1e-7) and ds[1] == nv
    b["mask"][:] = 0
    dl, dg, ds = _run(b, 0.2, 2.0)
    assert not dl.any() and not dg.any() and not ds.any()
    # no tokens at all
    e = {k: v[:0] for k, v in b.items()}
    dl, dg, ds = _run(e, 0.2, 2.0)
    assert dl.size == 0 and not ds.any()


def test_acr_rejects_bad_arguments():
    b = _dev(I.acr_batch(2, 8, seed=1))
    args = (b["logp"], b["logp_prox"], b["logp_behav"], b["adv"], b["mask"])
    with pytest.raises(B.QRError):
        B.acr_tis_loss(*args, 1.0, 2.0)  # eps must be < 1
    with pytest.raises(B.QRError):
        B.acr_tis_loss(*args, 0.2, 0.0)  # C must be > 0
    with pytest.raises(ValueError):
        B.acr_tis_loss(*args[:4], b["mask"].float(), 0.2, 2.0)
    # a workspace smaller than qr_workspace_size says is refused
    n = b["logp"].numel()
    loss = torch.empty(n, dtype=torch.float32, device=DEV)
    sums = torch.empty(3, dtype=torch.float64, device=DEV)
    p = [ctypes.c_void_p(t.data_ptr()) for t in args]
    st = B.lib().qr_acr_tis_loss(*p, n, ctypes.c_float(0.2), ctypes.c_float(2.0),
                                 ctypes.c_void_p(loss.data_ptr()), None,
                                 ctypes.c_void_p(sums.data_ptr()), None, 0, None)
    assert st == -3  # QR_ERR_WORKSPACE
