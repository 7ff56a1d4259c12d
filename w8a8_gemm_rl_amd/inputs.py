"""Seeded synthetic inputs and workload shapes for the W8A8 linear.

This module holds no arithmetic of the quantized linear itself: it draws
weights and activations (numpy PCG64, float32 normals), casts activations to
bf16 once with round-to-nearest-even (torch's CPU cast), and names the shapes of
the workloads. Both the GPU path's tests and the CPU oracle take their inputs
from here, so the two sides always see identical bits.

Workloads stand in for the pages' RL rollouts of 7B and 32B models (paper-notes
page, "Key findings": 7B and 32B sizes; the datasets and model weights are not
used). Shapes are nn.Linear [N, K] = [out, in].
"""

import hashlib

import numpy as np

UAQ_S = 1.5  # paper notes, "Loss / training strategy"

# A single linear: X[16, 512] bf16 ~ N(0, 1), W[512, 512] fp32 ~ N(0, 0.02).
SINGLE = dict(M=16, N=512, K=512, qt="int8", s=UAQ_S, seed=0, w_sigma=0.02)
LINEARS_SINGLE = {"linear": (SINGLE["N"], SINGLE["K"])}
CHAIN_SINGLE = [dict(name="linear", src="x0", cols=None)]

# 7B-shaped decoder linears (hidden 3584, intermediate 18944, QKV 4608).
LINEARS_7B = {
    "qkv": (4608, 3584),
    "o": (3584, 3584),
    "gate": (18944, 3584),
    "up": (18944, 3584),
    "down": (3584, 18944),
    "gateup": (37888, 3584),  # gate and up stacked along N (one GEMM, shared input)
}
W_SIGMA_7B = 0.02

# 32B-shaped decoder linears (hidden 5120, intermediate 27648, GQA 40q/8kv, d=128).
LINEARS_32B = {
    "qkv": (7168, 5120),
    "q": (5120, 5120),
    "k": (1024, 5120),
    "v": (1024, 5120),
    "o": (5120, 5120),
    "gate": (27648, 5120),
    "up": (27648, 5120),
    "down": (5120, 27648),
    "gateup": (55296, 5120),  # gate and up stacked along N
}
W_SIGMA_32B = 0.015

# Layer stacks of the whole models (per layer: fused QKV, O, stacked gate+up,
# down), as the per-RL-step weight refresh walks them.
STACK_7B = dict(layers=28, linears=LINEARS_7B, names=("qkv", "o", "gateup", "down"),
                sigma=W_SIGMA_7B)
STACK_32B = dict(layers=64, linears=LINEARS_32B, names=("qkv", "o", "gateup", "down"),
                 sigma=W_SIGMA_32B)

# Decode-layer chains. Each linear names its input: "x0" (the layer input) or
# an earlier linear's bf16 output, optionally a column slice of it. Attention,
# the activation function, residuals and norms are not part of the chain; the
# q slice of the QKV output stands in for the attention output.
CHAIN_7B = [
    dict(name="qkv", src="x0", cols=None),
    dict(name="o", src="qkv", cols=(0, 3584)),
    dict(name="gate", src="o", cols=None),
    dict(name="up", src="o", cols=None),
    dict(name="down", src="up", cols=None),
]
# The same layer with gate and up as one GEMM over the stacked weights
# [W_gate; W_up]: per-channel codes and scales are per row, so its outputs are
# the gate outputs followed by the up outputs, bit for bit.
CHAIN_7B_GATEUP = [
    dict(name="qkv", src="x0", cols=None),
    dict(name="o", src="qkv", cols=(0, 3584)),
    dict(name="gateup", src="o", cols=None),
    dict(name="down", src="gateup", cols=(18944, 37888)),
]
# The same layer with the producers of the linears' inputs: the input norm
# before QKV, the post-attention norm before gate+up (residual adds are not
# modeled: it normalizes the O output), and SiLU(gate) x up before down.
CHAIN_7B_PRODUCERS = [
    dict(name="qkv", src="x0", cols=None, prod="norm"),
    dict(name="o", src="qkv", cols=(0, 3584)),
    dict(name="gateup", src="o", cols=None, prod="norm"),
    dict(name="down", src="gateup", cols=None, prod="silu"),
]
NORM_EPS = 1e-6  # RMSNorm epsilon of the 7B/32B-shaped models
CHAIN_32B = [
    dict(name="q", src="x0", cols=None),
    dict(name="k", src="x0", cols=None),
    dict(name="v", src="x0", cols=None),
    dict(name="o", src="q", cols=None),
    dict(name="gate", src="o", cols=None),
    dict(name="up", src="o", cols=None),
    dict(name="down", src="up", cols=None),
]

# 32B prefill: the same chain shape as the 7B layer with 32B linears (QKV fused).
# The decode layer's variant with q, k and v stacked into one projection over
# [W_q; W_k; W_v] (their shared quantized input, one GEMM; each output column
# still depends only on its own weight row) uses it too.
CHAIN_32B_PREFILL = [
    dict(name="qkv", src="x0", cols=None),
    dict(name="o", src="qkv", cols=(0, 5120)),
    dict(name="gate", src="o", cols=None),
    dict(name="up", src="o", cols=None),
    dict(name="down", src="up", cols=None),
]

DW_SIGMA = 1e-7  # update size, paper notes "Key designs > UAQ" (~1e-7)


def rng(seed):
    return np.random.default_rng(seed)


def normal_f32(shape, sigma, seed):
    """float32 N(0, sigma^2) samples (sigma applied as one fp32 multiply)."""
    x = rng(seed).standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x = (x * np.float32(sigma)).astype(np.float32)
    return x


def bf16_bits(x_f32):
    """One round-to-nearest-even cast float32 -> bf16; returns uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def activations(M, K, seed, kind="normal"):
    """bf16 activation bits [M, K].

    kind:
      "normal"    X ~ N(0, 1)
      "outliers"  N(0, 1) with round(0.01 K) channels, drawn without
                  replacement and fixed across tokens, multiplied by 20
      "heavy"     N(0, 1) times a per-channel lognormal factor exp(z_k),
                  z_k ~ N(0, 1), fixed across tokens
    """
    g = rng(seed)
    x = g.standard_normal((M, K), dtype=np.float32)
    if kind == "outliers":
        n_out = int(round(0.01 * K))
        ch = g.choice(K, size=n_out, replace=False)
        x[:, ch] = (x[:, ch] * np.float32(20.0)).astype(np.float32)
    elif kind == "heavy":
        z = g.standard_normal(K, dtype=np.float32)
        c = np.exp(z.astype(np.float64)).astype(np.float32)
        x = (x * c[None, :]).astype(np.float32)
    elif kind != "normal":
        raise ValueError(kind)
    return bf16_bits(x)


def weights(N, K, sigma, seed):
    """fp32 master weights [N, K] ~ N(0, sigma^2)."""
    return normal_f32((N, K), sigma, seed)


def matrix_seed(cfg_index, idx):
    """Per-matrix seed of the workload recipe: 1000 * config + matrix index."""
    return 1000 * cfg_index + idx


def sha256(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


# Trainer-side token batch for the ACR / TIS loss: n_seq responses of ragged
# length (uniform in [1, max_len]) padded to max_len. Log-probabilities of the
# sampled tokens under the full-precision old actor: -|N(0, 1.5^2)|; the
# quantized actor that sampled them differs by N(0, 0.1^2) (KL between the two
# grows from 0.002 to 0.025 over training on the paper-notes page, "Key designs
# > ACR"); the current policy by N(0, 0.05^2). Advantages: one N(0, 1) value
# per response (group-normalized, as GRPO/DAPO give them), repeated over its
# tokens. Returns float32 arrays [n_seq * max_len] and a uint8 mask.
ACR_EPS = 0.2  # clip epsilon (not on the pages: the common PPO value)
ACR_C = 2.0  # truncation threshold C (the pages defer to FlashRL; not given)


def acr_batch(n_seq, max_len, seed):
    g = rng(seed)
    n = n_seq * max_len
    lens = g.integers(1, max_len + 1, size=n_seq)
    mask = (np.arange(max_len)[None, :] < lens[:, None]).astype(np.uint8).reshape(n)
    prox = (-np.abs(g.standard_normal(n)) * 1.5).astype(np.float32)
    behav = (prox + g.standard_normal(n) * 0.1).astype(np.float32)
    cur = (prox + g.standard_normal(n) * 0.05).astype(np.float32)
    adv = np.repeat(g.standard_normal(n_seq), max_len).astype(np.float32)
    return dict(logp=cur, logp_prox=prox, logp_behav=behav, adv=adv, mask=mask)

