"""Pins for oracle/mx.py (CPU only): MX element types e2m1, e2m3, e3m2, e4m3 with e8m0
scales per 32, the 6-bit packing and the mixed-element matmul.

Formats: "vLLM per-format kernel capability matrix derived from source" (group size 32
for MXFP4/MXFP6/MXFP8; MXFP6 weights with MXFP4, MXFP6 or unquantized activations;
MXFP8 native on gfx95).  Each pin stands outside the oracle's code: value lists written
out by hand from the OCP element definitions, hand-worked blocks in tests/golden, torch's
float8 decoders, the MXFP4 and MXFP8 oracles (separate code), big-integer bit
arithmetic, brute-force nearest search and exact rational sums.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import fp8 as O8
from oracle import mx as OX
from oracle import quant as OQ

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# non-negative values of each 6-bit type in code order, written out by hand
E2M3_POS = [0, 0.125, 0.25, 0.375, 0.5, 0.625, 0.75, 0.875,
            1, 1.125, 1.25, 1.375, 1.5, 1.625, 1.75, 1.875,
            2, 2.25, 2.5, 2.75, 3, 3.25, 3.5, 3.75,
            4, 4.5, 5, 5.5, 6, 6.5, 7, 7.5]
E3M2_POS = [0, 0.0625, 0.125, 0.1875, 0.25, 0.3125, 0.375, 0.4375,
            0.5, 0.625, 0.75, 0.875, 1, 1.25, 1.5, 1.75,
            2, 2.5, 3, 3.5, 4, 5, 6, 7,
            8, 10, 12, 14, 16, 20, 24, 28]


def test_six_bit_tables_match_hand_lists():
    assert list(OX.E2M3_TABLE[:32]) == E2M3_POS
    assert list(OX.E2M3_TABLE[32:]) == [-v for v in E2M3_POS]
    assert list(OX.E3M2_TABLE[:32]) == E3M2_POS
    assert list(OX.E3M2_TABLE[32:]) == [-v for v in E3M2_POS]
    assert np.signbit(OX.E2M3_TABLE[32]) and np.signbit(OX.E3M2_TABLE[32])


def test_four_and_eight_bit_tables_match_torch():
    e4 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    fin = ~np.isnan(e4)
    assert np.array_equal(OX.TABLE["e4m3"][fin], e4[fin])
    assert list(OX.TABLE["e2m1"][:8]) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


@pytest.mark.parametrize("elem", OX.ELEMS)
def test_encode_is_brute_force_nearest_with_ties_to_even(elem):
    pos = OX._POS[elem]
    mids = (pos[1:] + pos[:-1]) / 2
    rng = np.random.default_rng(3)
    y = np.concatenate([pos, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                        rng.uniform(0, pos[-1] * 1.2, 500), [pos[-1] * 1.01, 1e30]])
    got = OX.encode(elem, y)
    for v, c in zip(y, got):
        d = np.abs(pos - min(v, pos[-1]))
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert c == want, (elem, v, c, want)
    neg = OX.encode(elem, -y)
    assert np.array_equal(neg, got | OX.SIGN[elem])


def _golden():
    d = {}
    for line in open(os.path.join(GOLDEN, "mxfp6_blocks.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split(":", 1)
            d[k.strip()] = v.strip()
    return d


@pytest.mark.parametrize("blk", ["A", "B", "C", "D", "E"])
def test_mxfp6_golden_blocks(blk):
    d = _golden()
    elem = d[f"elem_{blk}"]
    vals = [float(t) for t in d[f"x_{blk}"].split()]
    x = np.zeros((1, 32), np.float32)
    x[0, :len(vals)] = vals
    codes, scales = OX.quantize(elem, x)
    want = [int(t, 16) for t in d[f"codes_{blk}"].split()]
    assert list(codes[0, :len(want)]) == want
    assert list(codes[0, len(vals):]) == [0] * (32 - len(vals))
    assert int(scales[0, 0]) == int(d[f"scale_{blk}"])


def test_six_bit_packing_golden_and_big_integer_layout():
    d = _golden()
    c = np.zeros((1, 32), np.uint8)
    vals = [int(t) for t in d["pack_codes"].split()]
    c[0, :len(vals)] = vals
    p = OX.pack("e2m3", c)
    assert p.shape == (1, 24)
    assert [f"{b:02X}" for b in p[0, :3]] == d["pack_bytes"].split()
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 64, (3, 96)).astype(np.uint8)
    packed = OX.pack("e3m2", codes)
    for r in range(3):
        for g in range(3):
            big = int.from_bytes(bytes(packed[r, 24 * g:24 * g + 24]), "little")
            for i in range(32):
                assert (big >> (6 * i)) & 63 == codes[r, 32 * g + i]
    assert np.array_equal(OX.unpack("e3m2", packed, 96), codes)


def test_e2m1_and_e4m3_agree_with_the_mxfp4_and_mxfp8_oracles():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((7, 256)) * np.exp(rng.uniform(-8, 8, (7, 1)))).astype(np.float32)
    x[2, :32] = 0.0
    c4, s4 = OX.quantize("e2m1", x)
    r4, rs4 = OQ.quantize_mxfp4(x)
    assert np.array_equal(c4, r4) and np.array_equal(s4, rs4)
    assert np.array_equal(OX.pack("e2m1", c4), OQ.quantize_packed("mxfp4", x)[0])
    c8, s8 = OX.quantize("e4m3", x)
    r8, rs8 = O8.quantize_mxfp8(x)
    assert np.array_equal(c8, r8) and np.array_equal(s8, rs8)


@pytest.mark.parametrize("elem", ["e2m3", "e3m2"])
def test_representable_blocks_round_trip(elem):
    """A block of table values times 2^E, whose largest magnitude sits in the top binade,
    quantizes to itself exactly."""
    rng = np.random.default_rng(11)
    pos = OX._POS[elem]
    top = [i for i, v in enumerate(pos) if v >= 2.0 ** OX.EMAX[elem]]
    for E in (-20, -3, 0, 7):
        idx = rng.integers(0, len(pos), 32)
        idx[5] = top[-1]
        sign = rng.choice([-1.0, 1.0], 32)
        x = (sign * pos[idx] * 2.0 ** E).astype(np.float32).reshape(1, 32)
        codes, scales = OX.quantize(elem, x)
        assert int(scales[0, 0]) == 127 + E
        assert np.array_equal(OX.dequantize(elem, codes, scales), x.astype(np.float64))


@pytest.mark.parametrize("elem", OX.ELEMS)
def test_quantization_error_bound(elem):
    """|x - x_hat| <= half an element step at the block's scale (mantissa bits m): at most
    2^(E + emax - m - 1) for values below the largest element (saturated ones excepted)."""
    mbits = {"e2m1": 1, "e2m3": 3, "e3m2": 2, "e4m3": 3}[elem]
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((16, 128)) * 3).astype(np.float32)
    codes, scales = OX.quantize(elem, x)
    hat = OX.dequantize(elem, codes, scales)
    E = scales.astype(np.int64) - 127
    step = np.repeat(2.0 ** (E + OX.EMAX[elem] - mbits), 32, axis=1)
    top = np.repeat(OX._POS[elem][-1] * 2.0 ** E, 32, axis=1)
    ok = np.abs(x) <= top
    assert np.all(np.abs(x - hat)[ok] <= step[ok] / 2)


def _frac_gemm(a, w):
    return [[sum((Fraction(float(a[m, k])) * Fraction(float(w[n, k])) for k in range(a.shape[1])),
                 Fraction(0)) for n in range(w.shape[0])] for m in range(a.shape[0])]


@pytest.mark.parametrize("ae,we", [("e4m3", "e2m1"), ("e2m3", "e3m2"), ("e2m1", "e2m3"),
                                   ("e3m2", "e4m3")])
def test_mixed_gemm_exact_rational_sums(ae, we):
    rng = np.random.default_rng(21)
    M, N, K = 3, 4, 96
    a = (rng.standard_normal((M, K)) * 2).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    ac, as_ = OX.quantize(ae, a)
    wc, ws = OX.quantize(we, w)
    got = OX.gemm(ae, ac, as_, we, wc, ws)
    # operands decoded a second way: the hand tables / torch's decoders, e8m0 via torch
    dec = {"e2m3": np.array(E2M3_POS + [-v for v in E2M3_POS]),
           "e3m2": np.array(E3M2_POS + [-v for v in E3M2_POS]),
           "e2m1": np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6] * 2) * np.repeat([1, -1], 8),
           "e4m3": torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()}

    def hat(e, c, s):
        sc = torch.from_numpy(s).view(torch.float8_e8m0fnu).double().numpy()
        return dec[e][c] * np.repeat(sc, 32, axis=1)

    exact = _frac_gemm(hat(ae, ac, as_), hat(we, wc, ws))
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(float(got[m, n])) - exact[m][n]) <= \
                Fraction(2.0 ** -45) * (abs(exact[m][n]) + 1)
