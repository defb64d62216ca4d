"""End-to-end FP8 linear layer (oracle; test infrastructure only).

Definition (page "transformers/integrations/deepgemm.py", ``deepgemm_fp8_fp4_linear``):
the bf16 activations are quantized per token group (``per_token_cast_to_fp8`` with the
float32-scale, gran_k = 128 recipe of ``_select_fp8_cast_kwargs``), multiplied with the
FP8 weight and its 128x128 block scales into an output of the activations' dtype (bf16),
and then, when a bias is given, the bias is added to that output in place
(``output.add_(bias)``): a bf16 + bf16 addition carried out in float32 and rounded once
to bf16.

    out = bf16( float32( bf16(C) ) + float32(bias) )

The quantization and C are the pinned functions of ``quant`` and ``gemm``; only the bias
step is new here. For fp16 activations the layer's output, and C, are fp16 instead
(``linear_f16_ref``).
"""

from __future__ import annotations

import numpy as np

from . import bf16, f16, gemm, quant


def bias_add_bf16(c_bits, bias) -> np.ndarray:
    """bf16 bits of bf16(float32(c) + float32(bias[n])) for c given as bf16 bits [M, N] and
    bias as float32 values that are bf16 values [N]."""
    c = bf16.from_bits(c_bits).astype(np.float32)
    b = np.asarray(bias, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        total = c + b[None, :]  # float32 addition, one rounding
    return bf16.to_bits(total.astype(np.float64))  # exact widening, then one bf16 rounding


def bias_add_f16(c_bits, bias) -> np.ndarray:
    """fp16 bits of fp16(float32(c) + float32(bias[n])): the same step for an fp16 layer."""
    c = f16.from_bits(c_bits).astype(np.float32)
    b = np.asarray(bias, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        total = c + b[None, :]
    return f16.to_bits(total.astype(np.float64))


def linear_f16_ref(x, w_q, w_s, bias=None, rows=None, cols=None):
    """linear_ref for fp16 activations: the output, and the GEMM result before the bias, are fp16
    (the page's output dtype follows the input)."""
    q, s = quant.quant_act_ref(np.asarray(x, dtype=np.float32))
    acc, _ = gemm.gemm_acc_ref(q, s, w_q, w_s, rows, cols)
    c_bits = f16.to_bits(acc)
    if bias is None:
        return c_bits, c_bits, q, s
    b = np.asarray(bias, dtype=np.float32)
    if cols is not None:
        b = b[np.asarray(cols)]
    return bias_add_f16(c_bits, b), c_bits, q, s


def linear_ref(x, w_q, w_s, bias=None, rows=None, cols=None):
    """(out_bits, c_bits, q, s): the layer's bf16 output, the GEMM's bf16 result before the
    bias, and the quantized activations (codes [M, K] and scales [M, K/128]).

    x holds bf16 values (any float dtype); bias is None or bf16 values [N]."""
    q, s = quant.quant_act_ref(np.asarray(x, dtype=np.float32))
    c_bits = gemm.gemm_ref(q, s, w_q, w_s, rows, cols)
    if bias is None:
        return c_bits, c_bits, q, s
    b = np.asarray(bias, dtype=np.float32)
    if cols is not None:
        b = b[np.asarray(cols)]
    return bias_add_bf16(c_bits, b), c_bits, q, s
