"""Block-scaled FP4 matmul by definition: dequantize, then multiply in float64.

Test infrastructure: only tests, the smoke check and the bench's CPU-baseline leg
use this module.

Sources
* "vLLM per-format kernel capability matrix derived from source", section
  THE EMULATION COLUMN: emulation dequantizes the weights, quantizes and
  dequantizes the activations, and computes the linear layer in high precision.
  Here "high precision" is float64 on exact dyadic dequant values.
* "vLLM on the NVIDIA DGX Spark (GB10 / sm_121): A Complete Technical Guide",
  §6.1: effective value = element x block scale x per-tensor scale, combined for
  the product as one alpha.
* "GLM-5.3-Flash on vLLM, on GB10": alpha = weight_scale_2 * input_scale.
* "vLLM on the DGX Spark, the Hard Way: Seven Months of GB10 Field Notes", the
  native-FP4 conditions: a weight-only (W4A16) checkpoint has no FP4
  activations, so its matmul takes the 16-bit activations as they are.

C[m, n] = alpha * sum_k a_hat[m, k] * w_hat[n, k]
  NVFP4 W4A4 : alpha = weight_scale_2 * input_scale, a_hat = NVFP4 QDQ of a under input_scale
  NVFP4 W4A16: alpha = weight_scale_2,                a_hat = a (bf16 values)
  MXFP4 W4A4 : alpha = 1,                             a_hat = MXFP4 QDQ of a
  MXFP4 W4A16: alpha = 1,                             a_hat = a
"""
import numpy as np

from . import quant as Q

W4A4 = "w4a4"
W4A16 = "w4a16"


def alpha(fmt, mode, weight_scale_2=1.0, input_scale=1.0):
    if fmt == Q.MXFP4:
        if float(weight_scale_2) != 1.0 or (mode == W4A4 and float(input_scale) != 1.0):
            raise ValueError("MXFP4 has no per-tensor scales; they must be 1")
        return 1.0
    ws2 = float(Q.check_scale(weight_scale_2, Q.WeightScaleError))
    if mode == W4A16:
        return ws2
    s = float(Q.check_scale(input_scale))
    return ws2 * s


def gemm_w4a4(fmt, a_codes, a_scales, w_codes, w_scales, weight_scale_2=1.0,
              input_scale=1.0):
    """W4A4 on pre-quantized operands (packed codes [M, K/2] / [N, K/2])."""
    al = alpha(fmt, W4A4, weight_scale_2, input_scale)
    a_hat = Q.dequantize_packed(fmt, a_codes, a_scales)
    w_hat = Q.dequantize_packed(fmt, w_codes, w_scales)
    return al * (a_hat @ w_hat.T)


def gemm_w4a16(fmt, a, w_codes, w_scales, weight_scale_2=1.0):
    """W4A16: a holds the 16-bit activation values (as float32/float64)."""
    al = alpha(fmt, W4A16, weight_scale_2)
    w_hat = Q.dequantize_packed(fmt, w_codes, w_scales)
    return al * (np.asarray(a, dtype=np.float64) @ w_hat.T)


def gemm_fused(fmt, a, w_codes, w_scales, weight_scale_2=1.0, input_scale=1.0):
    """W4A4 from 16-bit activations: quantize a under input_scale, then gemm_w4a4."""
    ac, asc = Q.quantize_packed(fmt, a, input_scale)
    return gemm_w4a4(fmt, ac, asc, w_codes, w_scales, weight_scale_2, input_scale)


def gemm_row(fmt, mode, a_row, w_codes, w_scales, weight_scale_2=1.0, input_scale=1.0):
    """One output row (used to check sampled rows of very large problems)."""
    a_row = np.asarray(a_row, dtype=np.float32).reshape(1, -1)
    if mode == W4A16:
        return gemm_w4a16(fmt, a_row, w_codes, w_scales, weight_scale_2)[0]
    return gemm_fused(fmt, a_row, w_codes, w_scales, weight_scale_2, input_scale)[0]


def row_error_bound(a_hat, w_hat, al, rel=2e-3):
    """Per-element tolerance |C - C_ref| <= rel * |alpha| * ||a_hat_m|| * ||w_hat_n||.

    The Cauchy-Schwarz scale of each output; the 2e-3 factor is the stated
    tolerance for GEMM outputs.
    """
    na = np.linalg.norm(np.asarray(a_hat, dtype=np.float64), axis=1)
    nw = np.linalg.norm(np.asarray(w_hat, dtype=np.float64), axis=1)
    return rel * abs(al) * np.outer(na, nw)
