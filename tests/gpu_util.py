"""Helpers shared by the GPU parity tests: device upload, tolerances, problem data.

Tolerances (stated for block-scaled GEMM outputs):
  per element  |C - C_ref| <= 2e-3 * |alpha| * ||a_hat_m|| * ||w_hat_n||  (+ one bf16 ulp of
               C_ref when the output is bf16 and C_ref is the oracle rounded to bf16)
  overall      ||C - C_ref||_F / ||C_ref||_F <= 1e-3
"""
import numpy as np
import torch

import synth
from oracle import formats as OF
from oracle import quant as OQ

DEV = "cuda:0"


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(DEV)


def bf16_dev(x_f32):
    """Round fp32 values to bf16 -> (device bf16 tensor, float32 numpy of the bf16 values)."""
    bits, vals = synth.bf16_bits(x_f32)
    return to_dev(bits.view(np.int16)).view(torch.bfloat16), vals


def round_bf16(x):
    """float64 -> bf16-representable float64 (round to nearest even)."""
    return torch.from_numpy(np.asarray(x, np.float64)).to(torch.float32).to(torch.bfloat16) \
        .to(torch.float64).numpy()


def bf16_ulp(x):
    x = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def check_gemm(got, ref, a_hat, w_hat, alpha, out_bf16, rel=2e-3, frob=1e-3, what=""):
    """got: GPU output (float64 numpy); ref: fp64 oracle output."""
    ref_c = round_bf16(ref) if out_bf16 else ref
    bound = rel * abs(alpha) * np.outer(np.linalg.norm(a_hat, axis=1), np.linalg.norm(w_hat, axis=1))
    if out_bf16:
        bound = bound + bf16_ulp(ref_c)
    err = np.abs(got - ref_c)
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} elements over the per-element bound; "
                           f"worst ratio {float((err / np.maximum(bound, 1e-300)).max()):.3g}")
    den = np.linalg.norm(ref_c)
    if den > 0:
        r = np.linalg.norm(got - ref_c) / den
        assert r <= frob, f"{what}: relative Frobenius error {r:.3g} > {frob}"
    return err


def weights(fmt, N, K, seed, std=0.02, index=0):
    w = synth.normal((N, K), std, seed=seed, role=synth.WEIGHT, index=index)
    codes, scales, ws2 = OQ.quantize_weight(fmt, w)
    return codes, scales, ws2


def dequant(fmt, codes_np, scales_np):
    return OQ.dequantize_packed(fmt, codes_np, scales_np)
