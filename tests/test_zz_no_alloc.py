"""The entry point that allocates nothing, against the one it mirrors.

qr_linear_fused_noalloc runs qr_linear_fused's kernels with their workspace
in the library's fixed per-GPU device array. Its outputs must equal
qr_linear_fused's bit for bit (INT8 and FP8: the same kernels in the same
plan), on two calls in a row, the second with a smaller input (the array
keeps the first call's contents), with no device memory allocated by either
call, and a shape whose workspace exceeds the array is refused with nothing
launched.
"""

import numpy as np
import pytest
import torch

from w8a8_gemm_rl_amd import binding as B
from w8a8_gemm_rl_amd import inputs as I

from gpu_helpers import DEV, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu

# 7B down projection at 256 tokens (split K, the largest 7B workspace), then
# the 7B O projection at 32 tokens (split K, smaller).
SHAPES = [(256, 3584, 18944), (32, 3584, 3584)]


@pytest.mark.parametrize("qt", ["int8", "fp8"])
def test_noalloc_equals_linear_fused_twice(qt):
    B.set_plan_override(-1)
    cases = []
    for i, (M, N, K) in enumerate(SHAPES):
        assert B.gemm_plan(M, N, K, qt)[1] > 1  # partial sums go through the scratch
        X = to_dev_bf16(I.activations(M, K, seed=900 + i, kind="outliers"))
        Wq, sw = B.quantize_weights_uaq(to_dev_f32(I.weights(N, K, 0.02, seed=910 + i)), 1.5, qt)
        ref = B.linear_fused(X, 1.5, Wq, sw, qt)
        Y = torch.full((M, N), 5.0, dtype=torch.bfloat16, device=DEV)
        cases.append((X, Wq, sw, ref, Y))
    torch.cuda.synchronize()
    B.linear_fused_noalloc(cases[0][0], 1.5, cases[0][1], cases[0][2], qt, Y=cases[0][4])
    torch.cuda.synchronize()  # the first call on the device has looked up the array
    for X, Wq, sw, ref, Y in cases:
        Y.fill_(5.0)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info(DEV)[0]
    for X, Wq, sw, ref, Y in cases:  # large, then smaller, back to back
        B.linear_fused_noalloc(X, 1.5, Wq, sw, qt, Y=Y)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info(DEV)[0]
    for X, Wq, sw, ref, Y in cases:
        assert torch.equal(Y.view(torch.int16), ref.view(torch.int16)), (qt, tuple(X.shape))
    assert free1 == free0  # no device memory was allocated by the two calls


def test_noalloc_refuses_shapes_beyond_its_scratch():
    M, N, K = 4096, 512, 18944  # 74 MiB of activation codes: more than the fixed 48 MiB
    assert B.workspace_size("qr_linear_fused", M, N, K, "int8") > 48 << 20
    X = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    Wq = torch.zeros((N, K), dtype=torch.int8, device=DEV)
    sw = torch.ones(N, dtype=torch.float32, device=DEV)
    Y = torch.full((M, N), 3.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(B.QRError) as e:
        B.linear_fused_noalloc(X, 1.5, Wq, sw, "int8", Y=Y)
    assert e.value.status == -3  # QR_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((Y == 3.0).all())  # nothing was launched
