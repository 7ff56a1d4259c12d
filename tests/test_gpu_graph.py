"""HIP-graph capture of the decode chain: every replay must equal the eager result.

The benchmark times graph replays, so the launch path (split-K counters reset
by the kernels themselves, no memset nodes) must give identical outputs on
every replay, with other eager work and synchronizations in between.
"""

import numpy as np
import pytest
import torch

from w8a8_gemm_rl_amd import binding as B
from w8a8_gemm_rl_amd import inputs as I

from gpu_helpers import DEV, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("qt", ["int8", "fp8"])
def test_graph_replays_match_eager(qt):
    M = 32
    shapes = {"a": (1024, 2048), "b": (2048, 1024), "c": (768, 2048)}
    X = to_dev_bf16(I.activations(M, 2048, seed=41, kind="outliers"))
    W = {n: B.quantize_weights_uaq(to_dev_f32(I.weights(N, K, 0.02, seed=50 + i)), 1.5, qt)
         for i, (n, (N, K)) in enumerate(shapes.items())}
    for n, (N, K) in shapes.items():
        assert B.gemm_plan(M, N, K, qt)[1] > 1  # exercise split-K inside the graph
    ws = torch.zeros(4 << 20, dtype=torch.uint8, device=DEV)
    ya = torch.empty((M, 1024), dtype=torch.bfloat16, device=DEV)
    yb = torch.empty((M, 2048), dtype=torch.bfloat16, device=DEV)
    yc = torch.empty((M, 768), dtype=torch.bfloat16, device=DEV)

    def chain():
        B.linear_fused(X, 1.5, *W["a"], qt, Y=ya, ws=ws)
        B.linear_fused(ya, 1.5, *W["b"], qt, Y=yb, ws=ws)
        B.linear_fused(yb, 1.5, *W["c"], qt, Y=yc, ws=ws)

    chain()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (ya, yb, yc)]

    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            chain()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (ya, yb, yc):
            t.zero_()
        junk = torch.randn(1000, device=DEV).sum()  # unrelated eager work
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip((ya, yb, yc), ref):
            assert torch.equal(t.view(torch.int16), r.view(torch.int16)), f"replay {rep}"
        chain()  # eager calls between replays share the workspace
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
