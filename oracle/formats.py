"""Element and scale formats of block-scaled FP4, written from their definitions.

Test infrastructure (see the package docstring): only tests, the smoke check and the
bench's CPU-baseline leg use this module.

Sources
* "vLLM on the NVIDIA DGX Spark (GB10 / sm_121): A Complete Technical Guide",
  §6.1 (NVFP4 format): elements are e2m1 -- two exponent bits, one mantissa bit,
  largest value 6.0 -- packed two per byte; one FP8 e4m3 block scale per 16
  contiguous elements along K; an fp32 global scale on top.
* Same guide, §6.4 (NVFP4 vs MXFP4 table): MXFP4 uses the same e2m1 element with
  32-element blocks and an exponent-only e8m0 scale.
* The pages do not spell out bias, subnormals or NaN codes.  E2M1's bias of 1
  follows from its stated maximum (6 = 1.5 * 2**2 needs the top exponent code 3 to
  mean 2**2).  E4M3 is read as the OCP "e4m3fn" variant (bias 7, no infinities,
  S.1111.111 is NaN, largest finite 448); E8M0 as the OCP MX scale (2**(c-127),
  0xFF is NaN).  The capability matrix's "WHAT IS NATIVE ON AMD" section notes the
  FNUZ variant on gfx94x parts; the target here is gfx950, which uses OCP.

Every encoder is "nearest finite value, ties to the even code", with magnitudes
above the largest finite value saturating to it.  Those are the plain meanings of
round-to-nearest-even and satfinite.  The pages state no rounding rule; this is the
reading taken.
"""
import numpy as np

# ----------------------------------------------------------------------------------
# value tables (closed form from the bit fields)
# ----------------------------------------------------------------------------------


def e2m1_value(code):
    """Value of a 4-bit e2m1 code: sign | 2-bit exponent (bias 1) | 1-bit mantissa."""
    c = int(code) & 0xF
    s = -1.0 if c & 0x8 else 1.0
    e = (c >> 1) & 0x3
    m = c & 0x1
    if e == 0:  # subnormal: 2**(1-bias) * (m/2)
        mag = m * 0.5
    else:
        mag = 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return s * mag


def e4m3_value(code):
    """Value of an OCP e4m3fn byte (bias 7, no infinities, 0x7F/0xFF are NaN)."""
    c = int(code) & 0xFF
    s = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:  # subnormal: 2**(1-7) * (m/8)
        mag = m * 2.0 ** -9
    else:
        mag = 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return s * mag


def e8m0_value(code):
    """Value of an E8M0 (exponent-only) scale byte: 2**(c-127); 0xFF is NaN."""
    c = int(code) & 0xFF
    if c == 0xFF:
        return float("nan")
    return 2.0 ** (c - 127)


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E8M0_TABLE = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)

E2M1_MAX = 6.0
E4M3_MAX = 448.0

# non-negative finite magnitudes, indexed by code (increasing with the code)
_E2M1_POS = E2M1_TABLE[:8].copy()          # codes 0..7
_E4M3_POS = E4M3_TABLE[:0x7F].copy()       # codes 0..0x7E (0x7F is NaN)


# ----------------------------------------------------------------------------------
# encoders: nearest finite value, ties to the even code, saturate above the maximum
# ----------------------------------------------------------------------------------


def _nearest_code(mag, table):
    """Codes of the nearest table entries to the non-negative magnitudes ``mag``.

    ``table`` holds the finite non-negative values in code order (increasing).
    Ties go to the even code; magnitudes above the last entry saturate to it.
    Arithmetic is float64, which is exact for every tie that can occur (the inputs
    are float32 and the table entries are short dyadic numbers).
    """
    mag = np.asarray(mag, dtype=np.float64)
    if np.isnan(mag).any():
        raise ValueError("NaN is outside the quantizer's contract")
    if (mag < 0).any():
        raise ValueError("magnitudes must be non-negative")
    n = table.shape[0]
    top = table[-1]
    m = np.minimum(mag, top)                       # satfinite
    hi = np.searchsorted(table, m, side="left")     # first entry >= m
    hi = np.clip(hi, 0, n - 1)
    lo = np.clip(hi - 1, 0, n - 1)
    d_lo = m - table[lo]
    d_hi = table[hi] - m
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(m == table[hi], hi, code)       # exact hits (incl. 0 -> code 0)
    return code.astype(np.uint8)


def e2m1_encode(x):
    """fp32 values -> 4-bit e2m1 codes (uint8 0..15); sign bit = signbit(x)."""
    x = np.asarray(x, dtype=np.float32)
    mag = np.abs(x.astype(np.float64))
    code = _nearest_code(mag, _E2M1_POS)
    sign = np.signbit(x).astype(np.uint8) << 3
    return (code | sign).astype(np.uint8)


def e4m3_encode_pos(y):
    """Non-negative fp32 values -> e4m3fn codes (RNE, satfinite at 448)."""
    y = np.asarray(y, dtype=np.float32)
    return _nearest_code(y.astype(np.float64), _E4M3_POS)


def mx_scale_exponent(amax):
    """E8M0 block-scale exponent for MXFP4 blocks with maximum magnitude ``amax``.

    The pages only say the MXFP4 scale is exponent-only.  The reading taken is the
    OCP MX rule: E = floor(log2(amax)) - emax_elem, with emax_elem = 2 for e2m1
    (its largest value is 1.5 * 2**2), clamped to the E8M0 range [-127, 127]; an
    all-zero block gets E = -127 (code 0).  floor(log2) is read off frexp exactly.
    """
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)                  # amax = f * 2**e, f in [0.5, 1)
    floor_log2 = e.astype(np.int64) - 1
    E = floor_log2 - 2
    E = np.where(amax == 0, -127, E)
    return np.clip(E, -127, 127).astype(np.int64)


# ----------------------------------------------------------------------------------
# nibble packing: element 2i in the low nibble of byte i, element 2i+1 in the high
# ----------------------------------------------------------------------------------


def pack_nibbles(codes):
    """uint8 codes [..., K] (0..15) -> packed bytes [..., K/2], low nibble = even k."""
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.shape[-1] % 2:
        raise ValueError("K must be even to pack two codes per byte")
    lo = codes[..., 0::2] & 0xF
    hi = codes[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """packed bytes [..., K/2] -> codes [..., K]."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out
