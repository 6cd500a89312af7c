"""Pins for the oracle's value tables and encoders (CPU only).

The pages fix e2m1's field widths and its maximum of 6.0 ("vLLM on the NVIDIA DGX
Spark (GB10 / sm_121): A Complete Technical Guide", §6.1) and name e4m3 / e8m0 as
the block-scale types (§6.1, §6.4).  Everything else is checked against torch's
float8 decoders (a library routine), literal value sets, brute force and
invariants -- never against the oracle's own formulas.
"""
import itertools

import numpy as np
import pytest
import torch

from oracle import formats as F

# The e2m1 value set (OCP MX spec, e2m1 table); its maximum 6.0 is the pages'.
E2M1_LITERAL = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_table_literal_and_symmetry():
    assert list(F.E2M1_TABLE[:8]) == E2M1_LITERAL
    assert F.E2M1_TABLE.max() == 6.0                   # the pages' stated maximum
    for c in range(8):
        assert F.E2M1_TABLE[c + 8] == -F.E2M1_TABLE[c]
    assert np.signbit(F.E2M1_TABLE[8])                 # 0x8 is -0


def test_e2m1_one_mantissa_bit():
    # every positive value is 1.0 or 1.5 times a power of two: one mantissa bit
    for v in F.E2M1_TABLE[1:8]:
        m, e = np.frexp(v)
        assert 2 * m in (1.0, 1.5)


def test_e4m3_decode_matches_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = F.E4M3_TABLE
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], ours[ok])
    assert np.nanmax(ours) == 448.0


def test_e8m0_decode_matches_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ref), np.isnan(F.E8M0_TABLE))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], F.E8M0_TABLE[ok])


def _e4m3_probe_values():
    pos = F.E4M3_TABLE[:0x7F]
    mids = (pos[1:] + pos[:-1]) / 2
    rng = np.random.default_rng(1)
    rand = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(464.0), 20000))
    near = np.concatenate([np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(1e9))])
    vals = np.concatenate([pos, mids, rand, near, [0.0, 2.0 ** -10, 3 * 2.0 ** -11, 464.0]])
    return vals.astype(np.float32)


def test_e4m3_encode_matches_torch_rne_below_464():
    v = _e4m3_probe_values()
    v = v[v <= 464.0]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.e4m3_encode_pos(v), ref)


def test_e4m3_encode_saturates():
    v = np.array([464.0, 464.01, 480.0, 1e6, 3.0e38, np.inf], dtype=np.float32)
    assert (F.e4m3_encode_pos(v) == 0x7E).all()


def test_e4m3_tiny_values():
    # below half the smallest subnormal -> 0; the tie at 2**-10 -> 0 (even code)
    v = np.array([0.0, 1e-30, 2.0 ** -11, 2.0 ** -10, np.nextafter(np.float32(2.0 ** -10), 1)],
                 dtype=np.float32)
    assert list(F.e4m3_encode_pos(v)) == [0, 0, 0, 0, 1]


# the tie list: midpoints go to the neighbour with the even code (mantissa bit 0)
E2M1_TIES = [(0.25, 0x0), (0.75, 0x2), (1.25, 0x2), (1.75, 0x4), (2.5, 0x4), (3.5, 0x6),
             (5.0, 0x6)]


@pytest.mark.parametrize("y,code", E2M1_TIES)
def test_e2m1_ties_to_even(y, code):
    assert F.e2m1_encode(np.float32(y)) == code
    assert F.e2m1_encode(np.float32(-y)) == code | 0x8


def test_e2m1_encode_brute_force_nearest():
    # dense grid incl. every midpoint and its neighbours: result is a nearest value
    grid = np.linspace(0, 8, 8193).astype(np.float32)
    mids = [(a + b) / 2 for a, b in zip(E2M1_LITERAL[:-1], E2M1_LITERAL[1:])]
    extra = np.array(mids + [np.nextafter(np.float32(m), np.float32(0)) for m in mids]
                     + [np.nextafter(np.float32(m), np.float32(9)) for m in mids], np.float32)
    ys = np.concatenate([grid, extra])
    codes = F.e2m1_encode(ys)
    lit = np.array(E2M1_LITERAL)
    for y, c in zip(ys.astype(np.float64), codes):
        assert c < 8
        d = np.abs(lit - min(y, 6.0))
        assert d[c] == d.min(), (y, c)


def test_e2m1_encode_monotone_and_signed():
    ys = np.sort(np.random.default_rng(2).uniform(-10, 10, 5000)).astype(np.float32)
    vals = F.E2M1_TABLE[F.e2m1_encode(ys)]
    assert (np.diff(vals) >= 0).all()
    assert (F.e2m1_encode(np.float32(-0.0)) == 0x8)
    assert (F.e2m1_encode(np.float32(0.0)) == 0x0)
    assert F.e2m1_encode(np.float32(100.0)) == 0x7
    assert F.e2m1_encode(np.float32(-np.inf)) == 0xF


def test_e2m1_round_trip_all_codes():
    for c in range(16):
        assert F.e2m1_encode(np.float32(F.E2M1_TABLE[c])) == c


def test_mx_scale_exponent_examples():
    # floor(log2 amax) - 2 from the float bits; subnormals and zero clamp to -127
    cases = {1.0: -2, 6.0: 0, 7.99: 0, 8.0: 1, 20.0: 2, 0.5: -3, 2.0 ** -130: -127, 0.0: -127,
             2.0 ** 127 * 1.5: 125}
    for a, e in cases.items():
        assert F.mx_scale_exponent(np.float64(a)) == e, a


def test_pack_nibbles_low_first():
    codes = np.array([[0x1, 0x2, 0xA, 0xF]], dtype=np.uint8)
    assert list(F.pack_nibbles(codes)[0]) == [0x21, 0xFA]
    for a, b in itertools.product(range(16), repeat=2):
        p = F.pack_nibbles(np.array([[a, b]], dtype=np.uint8))
        assert list(F.unpack_nibbles(p)[0]) == [a, b]
