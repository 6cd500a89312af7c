"""Pins for the oracle's NVFP4 / MXFP4 quantizers (CPU only).

Formats: "vLLM on the NVIDIA DGX Spark (GB10 / sm_121): A Complete Technical Guide",
§6.1 and §6.4.  The hand-worked blocks in tests/golden pin the rounding rules and
the fp32 operation order; the invariants below pin the scale handling.
"""
import os

import numpy as np
import pytest

from oracle import formats as F
from oracle import quant as Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_golden(name):
    d = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            d[k.strip()] = v.strip()
    x = np.array([float(t) for t in d["x"].split()], dtype=np.float32)
    codes = np.array([int(t, 16) for t in d["codes"].split()], dtype=np.uint8)
    sc = np.array([int(t, 0) for t in d["scale_codes"].split()], dtype=np.uint8)
    deq = np.array([float(t) for t in d["dequant"].split()])
    return d["fmt"], float(d["input_scale"]), x, codes, sc, deq


@pytest.mark.parametrize("name", ["nvfp4_block_s1.txt", "nvfp4_block_s001.txt", "mxfp4_block.txt"])
def test_golden_blocks(name):
    fmt, s, x, codes, sc, deq = load_golden(name)
    q, scales = Q.quantize(fmt, x.reshape(1, -1), s)
    assert list(q[0]) == list(codes)
    assert list(scales[0]) == list(sc)
    got = Q.dequantize(fmt, q, scales)[0]
    assert np.array_equal(got, deq)


def test_nvfp4_scale_power_of_two_invariance():
    # multiplying input_scale by 2**j keeps the element codes and shifts the e4m3
    # exponent by -j (while no scale saturates or underflows); the product
    # (dequant * input_scale) is unchanged.
    rng = np.random.default_rng(3)
    x = rng.standard_normal((8, 64)).astype(np.float32)
    s0 = np.float32(np.abs(x).max() / 2688.0 * 8)
    q0, sc0 = Q.quantize_nvfp4(x, s0)
    d0 = Q.dequantize(Q.NVFP4, q0, sc0) * float(s0)
    for j in (-2, -1, 1, 2):
        s = np.float32(s0 * 2.0 ** j)
        q, sc = Q.quantize_nvfp4(x, s)
        nz = sc0 >= 0x10                          # normal scales, away from the subnormal range
        assert np.array_equal(q, q0)
        assert np.array_equal(sc[nz].astype(int), sc0[nz].astype(int) - 8 * j)
        assert np.allclose(Q.dequantize(Q.NVFP4, q, sc) * float(s), d0, rtol=0, atol=0)


def test_nvfp4_zero_and_saturating_blocks():
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 3] = -0.0
    x[0, 16:] = 1e6            # amax*g/6 far above 448 -> scale saturates to 448
    q, sc = Q.quantize_nvfp4(x, 1.0)
    assert sc[0, 0] == 0 and (q[0, :16] == np.where(np.signbit(x[0, :16]), 8, 0)).all()
    assert sc[0, 1] == 0x7E and (q[0, 16:] == 7).all()


def test_nvfp4_elementwise_error_bound():
    # each dequantized element is within half an e2m1 step of x, except clipping at 6*scale
    rng = np.random.default_rng(4)
    x = rng.standard_normal((16, 256)).astype(np.float32)
    s = np.float32(np.abs(x).max() / 2688.0)
    q, sc = Q.quantize_nvfp4(x, s)
    deq = Q.dequantize(Q.NVFP4, q, sc) * float(s)
    sd = F.E4M3_TABLE[sc].repeat(16, axis=1) * float(s)
    # largest e2m1 gap is 2 (between 4 and 6); half of it bounds the rounding error,
    # plus the block scale's own rounding (<= 1/16 relative) times |x| <= 6.75 * sd
    assert (np.abs(deq - x) <= 1.0 * sd + 1e-7 + 0.07 * np.abs(x)).all()


def test_mxfp4_requant_invariants():
    # dequant -> requant reproduces the dequant values; codes and scale stay the same
    # exactly when the block's largest magnitude code is 6 or 7 (value 4 or 6)
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((32, 128)) * np.exp(rng.uniform(-3, 3, (32, 1)))).astype(np.float32)
    x[0, :32] *= 0.01
    x[1, 32:64] = 0.3
    q, sc = Q.quantize_mxfp4(x)
    d = Q.dequantize(Q.MXFP4, q, sc).astype(np.float32)
    q2, sc2 = Q.quantize_mxfp4(d)
    assert np.array_equal(Q.dequantize(Q.MXFP4, q2, sc2), d.astype(np.float64))
    blk_max_code = (q & 7).reshape(32, 4, 32).max(axis=-1)
    same = (q2.reshape(32, 4, 32) == q.reshape(32, 4, 32)).all(-1) & (sc2 == sc)
    assert np.array_equal(same, blk_max_code >= 6)


def test_mxfp4_max_element_lands_in_top_binade():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((64, 64)).astype(np.float32)
    q, sc = Q.quantize_mxfp4(x)
    amax = np.abs(x).reshape(64, 2, 32).max(-1)
    scale = F.E8M0_TABLE[sc]
    # amax / scale lies in [4, 8): the largest element rounds to 4 or 6 (clipped)
    r = amax / scale
    assert ((r >= 4) & (r < 8)).all()


def test_input_scale_refusal():
    x = np.ones((1, 16), dtype=np.float32)
    for bad in (0.0, -1.0, np.inf, np.nan, 2.0 ** -101, 2.0 ** 101):
        with pytest.raises(Q.InputScaleError):
            Q.quantize_nvfp4(x, bad)
    with pytest.raises(ValueError):
        Q.quantize(Q.MXFP4, np.ones((1, 32), np.float32), 0.5)


def test_weight_quant_uses_full_e4m3_range():
    # weight_scale_2 = fp32(amax / 2688), 2688 = 6 * 448, values worked by hand:
    #   amax 1: 1/2688 = 2^-7 / 21 and 1/21 = 2^-5 * 1.100001100001...b, whose 24th
    #           significant bit onward (1100001...) rounds the 23-bit field up to
    #           10000110000110000110001b: 0x1.861862p-12
    #   amax 3: 3/2688 = 2^-7 / 7 and 1/7 = 2^-3 * 1.001001001...b, rounded up
    #           likewise to 00100100100100100100101b: 0x1.24924ap-10
    for amax, want in ((1.0, "0x1.861862p-12"), (3.0, "0x1.24924ap-10")):
        w = np.zeros((2, 32), np.float32)
        w[1, 5] = -amax
        w[0, 3] = amax / 4
        assert float(Q.weight_scale_2(w)) == float.fromhex(want)
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((64, 128)) * 0.02).astype(np.float32)
    codes, sc, ws2 = Q.quantize_weight(Q.NVFP4, w)
    assert sc.max() == 0x7E                     # the block holding the max uses scale 448
    wd = Q.dequantize_packed(Q.NVFP4, codes, sc) * ws2
    assert np.abs(wd).max() == pytest.approx(np.abs(w).max(), rel=1 / 8)
