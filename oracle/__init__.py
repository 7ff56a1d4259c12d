"""CPU oracle for the QuRL W8A8 linear -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct numpy statement of what the
quantized-rollout linear computes. Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path (the HIP library
and its Python binding) never does, and shares no code with it.

Sources (pages on "QuRL: Efficient Reinforcement Learning with Quantized
Rollout"):
  * Paper-notes page (ICLR 2026 notes), "Method > Key designs > UAQ": the
    invariant scaling WX = (W/s)(sX), s > 1 applied column-wise to W and
    row-wise to the activation that feeds it, mergeable into the norm.
  * Same page, "Loss / training strategy": channel-wise weight quantization,
    token-wise activation quantization, INT8 or FP8, s = 1.5.
  * Same page, "Method > Overall framework": theta_old is quantized to
    theta_hat_old for every rollout.
  * Same page, "Method > System integration": UAQ is a one-time weight
    preprocessing; INT8/FP8 matmul kernels run the rollout.

Every function states the passage it follows and, where the pages leave a step
open, the reading taken (the full list of readings is kept with the design
notes of the repository).

Floating-point decisions that produce integers (quantized codes) are taken in
IEEE fp32, the precision the GPU path computes them in; accumulations are exact
(float64 holds every partial sum exactly, see ``qurl.acc_int8``/``acc_fp8``).
"""

from .formats import (
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    e4m3fn_decode,
    e4m3fn_encode,
    E4M3FN_MAX,
)
from .qurl import (
    QMAX,
    uaq_reparameterize,
    quantize_rows,
    quantize_weights_uaq,
    quantize_act_per_token,
    acc_int8,
    acc_fp8,
    dequant_epilogue,
    w8a8_linear,
    flip_counts,
    count_flips,
    count_flips_rows,
    norm_folded,
    norm_quant,
    silu_mul,
    silu_mul_quant,
    acr_tis_loss,
    MX_BLOCK,
    mx_exponent,
    mx_quantize_rows,
    mx_linear,
    requantize_weights,
    flip_expectation,
    decode_chain,
)

__all__ = [
    "bf16_bits_to_f32", "f32_to_bf16_bits", "e4m3fn_decode", "e4m3fn_encode",
    "E4M3FN_MAX", "QMAX", "uaq_reparameterize", "quantize_rows",
    "quantize_weights_uaq", "quantize_act_per_token", "acc_int8", "acc_fp8",
    "dequant_epilogue", "w8a8_linear", "flip_counts", "flip_expectation",
    "count_flips", "count_flips_rows",
    "norm_folded", "norm_quant", "silu_mul", "silu_mul_quant", "acr_tis_loss",
    "MX_BLOCK", "mx_exponent", "mx_quantize_rows", "mx_linear", "requantize_weights",
    "decode_chain",
]
