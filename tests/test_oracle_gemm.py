"""Pins for the oracle's block-scaled matmul (CPU only).

Definition: "vLLM per-format kernel capability matrix derived from source", THE
EMULATION COLUMN (dequantize, QDQ the activations, matmul in high precision);
alpha = weight_scale_2 * input_scale from "GLM-5.3-Flash on vLLM, on GB10".

The brute-force test decodes codes with a literal e2m1 list and torch's float8
decoders and sums with exact rationals, so it shares nothing with the oracle but
the packed layout.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import gemm as Gm
from oracle import quant as Q

E2M1_LITERAL = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _lit_e2m1(c):
    v = E2M1_LITERAL[c & 7]
    return -v if c & 8 else v


def _torch_scale(fmt, code):
    dt = torch.float8_e4m3fn if fmt == Q.NVFP4 else torch.float8_e8m0fnu
    return float(torch.tensor([code], dtype=torch.uint8).view(dt).to(torch.float64)[0])


def _rand_operand(rng, fmt, rows, K):
    G = Q.GROUP[fmt]
    codes = rng.integers(0, 16, size=(rows, K), dtype=np.uint8)
    if fmt == Q.NVFP4:
        sc = rng.integers(0x08, 0x70, size=(rows, K // G), dtype=np.uint8)
    else:
        sc = rng.integers(110, 140, size=(rows, K // G), dtype=np.uint8)
    return codes, sc


@pytest.mark.parametrize("fmt", [Q.NVFP4, Q.MXFP4])
def test_w4a4_exact_rational_brute_force(fmt):
    rng = np.random.default_rng(10)
    M, N, K = 3, 5, 64
    G = Q.GROUP[fmt]
    ac, asc = _rand_operand(rng, fmt, M, K)
    wc, wsc = _rand_operand(rng, fmt, N, K)
    ws2, s = (0.75, 0.3125) if fmt == Q.NVFP4 else (1.0, 1.0)
    got = Gm.gemm_w4a4(fmt, F.pack_nibbles(ac), asc, F.pack_nibbles(wc), wsc, ws2, s)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                a = Fraction(_lit_e2m1(ac[m, k])) * Fraction(_torch_scale(fmt, asc[m, k // G]))
                w = Fraction(_lit_e2m1(wc[n, k])) * Fraction(_torch_scale(fmt, wsc[n, k // G]))
                acc += a * w
            exp = acc * Fraction(ws2) * Fraction(float(np.float32(s)))
            assert got[m, n] == pytest.approx(float(exp), rel=1e-15, abs=1e-300)


def test_w4a16_exact_rational_brute_force():
    rng = np.random.default_rng(11)
    M, N, K = 2, 4, 32
    a = rng.standard_normal((M, K)).astype(np.float32)
    wc, wsc = _rand_operand(rng, Q.NVFP4, N, K)
    got = Gm.gemm_w4a16(Q.NVFP4, a, F.pack_nibbles(wc), wsc, 0.5)
    for m in range(M):
        for n in range(N):
            acc = sum(Fraction(float(a[m, k])) * Fraction(_lit_e2m1(wc[n, k]))
                      * Fraction(_torch_scale(Q.NVFP4, wsc[n, k // 16])) for k in range(K))
            assert got[m, n] == pytest.approx(float(acc / 2), rel=1e-14)


@pytest.mark.parametrize("fmt", [Q.NVFP4, Q.MXFP4])
def test_constant_code_closed_form(fmt):
    # every element = code c under scale code sc: C = K * v^2 * alpha
    M, N, K = 4, 6, 128
    G = Q.GROUP[fmt]
    c, scode = 0x5, (0x38 if fmt == Q.NVFP4 else 127)   # 3.0 x 1.0
    codes = np.full((M, K), c, np.uint8)
    sc = np.full((M, K // G), scode, np.uint8)
    wcodes = np.full((N, K), c | 0x8, np.uint8)        # -3.0
    wsc = np.full((N, K // G), scode, np.uint8)
    ws2, s = (2.0, 0.25) if fmt == Q.NVFP4 else (1.0, 1.0)
    got = Gm.gemm_w4a4(fmt, F.pack_nibbles(codes), sc, F.pack_nibbles(wcodes), wsc, ws2, s)
    assert (got == K * 3.0 * -3.0 * ws2 * s).all()


def test_identity_weight_reproduces_activation():
    # W = I (code 2 = 1.0 on the diagonal, scale 1.0): C = alpha * a_hat; a transposed
    # operand or swapped nibbles would scramble it
    K = 64
    rng = np.random.default_rng(12)
    a = rng.standard_normal((3, K)).astype(np.float32)
    w = np.zeros((K, K), np.uint8)
    np.fill_diagonal(w, 0x2)
    wsc = np.full((K, K // 16), 0x38, np.uint8)
    ac, asc = Q.quantize_packed(Q.NVFP4, a, 0.125)
    got = Gm.gemm_w4a4(Q.NVFP4, ac, asc, F.pack_nibbles(w), wsc, 1.0, 0.125)
    assert np.array_equal(got, Q.dequantize_packed(Q.NVFP4, ac, asc) * 0.125)
    got16 = Gm.gemm_w4a16(Q.NVFP4, a, F.pack_nibbles(w), wsc, 1.0)
    assert np.array_equal(got16, a.astype(np.float64))


def test_w4a4_differs_from_w4a16():
    # the fused W4A4 result is the quantized-activation product, not the weight-only one
    rng = np.random.default_rng(13)
    a = rng.standard_normal((4, 256)).astype(np.float32)
    w = (rng.standard_normal((16, 256)) * 0.02).astype(np.float32)
    wc, wsc, ws2 = Q.quantize_weight(Q.NVFP4, w)
    s = float(np.abs(a).max() / 2688.0)
    c44 = Gm.gemm_fused(Q.NVFP4, a, wc, wsc, ws2, s)
    c416 = Gm.gemm_w4a16(Q.NVFP4, a, wc, wsc, ws2)
    rel = np.linalg.norm(c44 - c416) / np.linalg.norm(c416)
    assert rel > 1e-2


def test_mxfp4_rejects_per_tensor_scales():
    with pytest.raises(ValueError):
        Gm.alpha(Q.MXFP4, Gm.W4A4, 1.0, 2.0)
    with pytest.raises(Q.InputScaleError):
        Gm.alpha(Q.NVFP4, Gm.W4A4, 1.0, 0.0)
    assert Gm.alpha(Q.NVFP4, Gm.W4A16, 0.5, 0.0) == 0.5      # weight-only ignores input_scale
