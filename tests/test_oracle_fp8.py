"""Pins for the oracle's MXFP8 and FP8 W8A8 functions (CPU only).

Formats and modes: "vLLM per-format kernel capability matrix derived from source" (the
MX group size of 32, MXFP8 native on gfx95, FP8's per-tensor / 1x128-128x128 block /
rowwise scaling modes).  Each pin is independent of the oracle's own code: torch's
float8 casts and decoders, a hand-worked block in tests/golden, hand-derived scale
constants, and exact rational sums.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import fp8 as O8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_e4m3(y):
    """torch's float8_e4m3fn cast (round to nearest even; valid below 464)."""
    return torch.from_numpy(np.asarray(y, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_cast_below_saturation():
    # every e4m3 value, every midpoint between neighbours and the floats next to them
    v = torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    mids = (v[1:] + v[:-1]) / 2
    pts = np.concatenate([v, mids, np.nextafter(mids, 0).astype(np.float32),
                          np.nextafter(mids, np.float32(1e9)).astype(np.float32)]).astype(np.float32)
    pts = pts[pts <= 448]
    for sgn in (1, -1):
        y = (sgn * pts).astype(np.float32)
        assert np.array_equal(O8.e4m3_encode(y), _torch_e4m3(y))


def test_e4m3_encode_saturates_and_keeps_sign_of_zero():
    assert list(O8.e4m3_encode(np.float32([464, 1e6, -500, 460]))) == [0x7E, 0x7E, 0xFE, 0x7E]
    assert list(O8.e4m3_encode(np.float32([0.0, -0.0, -1e-30]))) == [0x00, 0x80, 0x80]


def test_mxfp8_golden_blocks():
    d = {}
    for line in open(os.path.join(GOLDEN, "mxfp8_blocks.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split(":", 1)
            d[k.strip()] = v.strip()
    x = np.array([float(t) for t in d["x"].split()], dtype=np.float32).reshape(1, -1)
    codes, scales = O8.quantize_mxfp8(x)
    assert [f"{c:02X}" for c in codes[0]] == d["codes"].split()
    assert [int(s) for s in scales[0]] == [int(t) for t in d["scale_codes"].split()]
    # dequantization through torch's float8 decoders (e4m3fn elements, e8m0 scales)
    e = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    s = torch.from_numpy(scales).view(torch.float8_e8m0fnu).double().numpy()
    assert np.array_equal(O8.dequantize_mxfp8(codes, scales), e * np.repeat(s, 32, axis=1))


def test_mxfp8_elements_follow_torch_cast_of_the_scaled_block():
    rng = np.random.default_rng(31)
    x = (rng.standard_normal((16, 256)) * np.exp(rng.uniform(-8, 8, (16, 1)))).astype(np.float32)
    codes, scales = O8.quantize_mxfp8(x)
    E = scales.astype(np.int64) - 127
    amax = np.abs(x).reshape(16, 8, 32).max(-1)
    assert ((amax * np.ldexp(1.0, -E) >= 256) & (amax * np.ldexp(1.0, -E) < 512)).all()
    y = (x.reshape(16, 8, 32) * np.ldexp(1.0, -E)[..., None]).astype(np.float32)
    want = _torch_e4m3(np.clip(y, -448, 448)).reshape(16, 256)
    assert np.array_equal(codes, want)


def test_fp8_dynamic_scale_hand_values():
    # amax / 448 in fp32: 448 -> 1; 1 -> 2^-6 / 7 = 2^-9 * 1.001001001...b, rounded up in
    # the 24th bit: 0x1.24924ap-9; 2.5 -> 2^-8 * (10/7 = 1.0110110110...b): 0x1.6db6dcp-8
    assert O8.dynamic_scale(448.0) == 1.0
    assert float(O8.dynamic_scale(1.0)) == float.fromhex("0x1.24924ap-9")
    assert float(O8.dynamic_scale(2.5)) == float.fromhex("0x1.6db6dcp-8")


@pytest.mark.parametrize("mode", O8.MODES)
def test_fp8_act_quant_is_the_torch_cast_of_the_quotient(mode):
    rng = np.random.default_rng(32)
    x = (rng.standard_normal((8, 256)) * 3).astype(np.float32)
    x[1] = 0.0                                   # a zero row: scale 0, zero codes
    x[2, 5] = -0.0
    codes, s = O8.quantize_act(mode, x, scale=0.05 if mode == O8.PER_TENSOR else None)
    if mode == O8.PER_TENSOR:
        q = x / np.float32(0.05)
    elif mode == O8.ROWWISE:
        amax = np.abs(x).max(1)
        assert np.array_equal(s, (amax / np.float32(448)).astype(np.float32))
        q = x / np.where(s == 0, 1, s)[:, None]
    else:
        amax = np.abs(x).reshape(8, 2, 128).max(-1)
        assert np.array_equal(s, (amax / np.float32(448)).astype(np.float32))
        q = (x.reshape(8, 2, 128) / np.where(s == 0, 1, s)[..., None]).reshape(8, 256)
    q = q.astype(np.float32)
    assert np.abs(q).max() <= 464
    assert np.array_equal(codes, _torch_e4m3(np.clip(q, -448, 448)))
    if mode != O8.PER_TENSOR:
        assert (codes[1] == 0).all()
        assert np.abs(O8.e4m3_decode(codes)).max() == 448      # the row / block maximum maps to 448


def test_fp8_weight_block_scales_cover_128x128_and_a_ragged_edge():
    rng = np.random.default_rng(33)
    w = rng.standard_normal((300, 256)).astype(np.float32)
    codes, s = O8.quantize_weight(O8.BLOCK, w)
    assert s.shape == (3, 2)
    for b in range(3):
        for kb in range(2):
            blk = w[128 * b:128 * b + 128, 128 * kb:128 * kb + 128]
            assert s[b, kb] == np.float32(np.abs(blk).max()) / np.float32(448)
    hat = O8.dequantize_weight(O8.BLOCK, codes, s)
    assert np.abs(hat - w).max() <= np.abs(w).max() / 16        # 3 mantissa bits


def _frac_gemm(a, w):
    return [[sum((Fraction(float(a[m, k])) * Fraction(float(w[n, k])) for k in range(a.shape[1])),
                 Fraction(0)) for n in range(w.shape[0])] for m in range(a.shape[0])]


@pytest.mark.parametrize("mode", O8.MODES + ("mx",))
def test_fp8_gemm_exact_rational_sums(mode):
    rng = np.random.default_rng(34)
    M, N, K = 3, 5, 256
    a = (rng.standard_normal((M, K)) * 2).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.1).astype(np.float32)
    if mode == "mx":
        ac, as_ = O8.quantize_mxfp8(a)
        wc, ws = O8.quantize_mxfp8(w)
        got = O8.gemm_mxfp8(ac, as_, wc, ws)
        a_hat = torch.from_numpy(ac).view(torch.float8_e4m3fn).double().numpy() * \
            np.repeat(torch.from_numpy(as_).view(torch.float8_e8m0fnu).double().numpy(), 32, 1)
        w_hat = torch.from_numpy(wc).view(torch.float8_e4m3fn).double().numpy() * \
            np.repeat(torch.from_numpy(ws).view(torch.float8_e8m0fnu).double().numpy(), 32, 1)
    else:
        ac, as_ = O8.quantize_act(mode, a, scale=0.02)
        wc, ws = O8.quantize_weight(mode, w)
        got = O8.gemm(mode, ac, as_, wc, ws)
        ev = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy()
        if mode == O8.PER_TENSOR:
            a_hat, w_hat = ev(ac) * float(as_), ev(wc) * float(ws)
        elif mode == O8.ROWWISE:
            a_hat, w_hat = ev(ac) * as_[:, None].astype(np.float64), ev(wc) * ws[:, None].astype(np.float64)
        else:
            a_hat = ev(ac) * np.repeat(as_.astype(np.float64), 128, 1)
            w_hat = ev(wc) * np.repeat(np.repeat(ws.astype(np.float64), 128, 1), 128, 0)[:N]
    exact = _frac_gemm(a_hat, w_hat)
    # the float64 matmul rounds its partial sums: within K ulps of the sum of |products|
    bound = K * 2.0 ** -52 * (np.abs(a_hat) @ np.abs(w_hat).T)
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(float(got[m, n])) - exact[m][n]) <= Fraction(float(bound[m, n]))
