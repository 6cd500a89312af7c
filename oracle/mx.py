"""MX block formats with any element type the gfx950 scaled MFMA takes, by definition:
MXFP4 (e2m1), MXFP6 (e2m3 or e3m2) and MXFP8 (e4m3); quantize, pack, dequantize and
multiply in float64, the two operands of a matmul free to use different element types.

Test infrastructure: only tests, the smoke check and the bench's CPU-baseline leg use
this module.

Sources ("vLLM per-format kernel capability matrix derived from source"):
* its group-size note: MXFP4, MXFP6 and MXFP8 all use blocks of 32 elements along K with
  an exponent-only (e8m0) scale;
* MXFP6: MXFP6 weights are accepted with MXFP4, MXFP6 or unquantized activations -- the
  two operands of one matmul need not share an element type;
* MXFP8 / WHAT IS NATIVE ON AMD: MXFP8 is native on gfx95 parts;
* THE EMULATION COLUMN: the product is defined by dequantizing both operands and
  multiplying in high precision.

Readings where the pages are silent (listed in the design notes):
* MXFP6 names two element types, both read from the OCP MX definitions: e2m3 (bias 1,
  three mantissa bits, largest 7.5) and e3m2 (bias 3, two mantissa bits, largest 28),
  neither with infinities or NaN.
* Block scale: the OCP MX rule E = floor(log2 amax) - emax(element), clamped to
  [-127, 127], an all-zero block E = -127; emax is 2 (e2m1, e2m3), 4 (e3m2), 8 (e4m3).
  Elements: nearest value of x * 2**-E, ties to the even code, saturating at the
  element's largest value, sign of x kept (negative zero included).
* Packing (a storage choice, not on the pages): e2m1 two per byte, low nibble first;
  e4m3 one per byte; e2m3 / e3m2 32 elements in 24 bytes, element i at bits
  [6 i, 6 i + 6) of the little-endian 192-bit group.
"""
import numpy as np

from . import formats as F

ELEMS = ("e2m1", "e2m3", "e3m2", "e4m3")
BITS = {"e2m1": 4, "e2m3": 6, "e3m2": 6, "e4m3": 8}
EMAX = {"e2m1": 2, "e2m3": 2, "e3m2": 4, "e4m3": 8}
GROUP = 32


def e2m3_value(code):
    """6-bit e2m3: sign (bit 5) | 2-bit exponent, bias 1 | 3-bit mantissa."""
    c = int(code) & 0x3F
    s = -1.0 if c & 0x20 else 1.0
    e, m = (c >> 3) & 0x3, c & 0x7
    mag = m / 8.0 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 8.0)
    return s * mag


def e3m2_value(code):
    """6-bit e3m2: sign (bit 5) | 3-bit exponent, bias 3 | 2-bit mantissa."""
    c = int(code) & 0x3F
    s = -1.0 if c & 0x20 else 1.0
    e, m = (c >> 2) & 0x7, c & 0x3
    mag = m / 4.0 * 2.0 ** -2 if e == 0 else 2.0 ** (e - 3) * (1.0 + m / 4.0)
    return s * mag


E2M3_TABLE = np.array([e2m3_value(c) for c in range(64)], dtype=np.float64)
E3M2_TABLE = np.array([e3m2_value(c) for c in range(64)], dtype=np.float64)
TABLE = {"e2m1": F.E2M1_TABLE, "e2m3": E2M3_TABLE, "e3m2": E3M2_TABLE, "e4m3": F.E4M3_TABLE}
SIGN = {"e2m1": 0x8, "e2m3": 0x20, "e3m2": 0x20, "e4m3": 0x80}
# non-negative finite magnitudes in code order (e4m3: 0x7F is NaN)
_POS = {"e2m1": F.E2M1_TABLE[:8], "e2m3": E2M3_TABLE[:32], "e3m2": E3M2_TABLE[:32],
        "e4m3": F.E4M3_TABLE[:0x7F]}


def _check_elem(elem):
    if elem not in ELEMS:
        raise ValueError(f"unknown MX element type {elem!r}")


def encode(elem, y, sign_src=None):
    """Codes of the exact float64 values y (nearest, ties to even, saturating); the sign
    bit is the sign bit of ``sign_src`` (default y)."""
    _check_elem(elem)
    y = np.asarray(y, dtype=np.float64)
    code = F._nearest_code(np.abs(y), _POS[elem])
    neg = np.signbit(y if sign_src is None else np.asarray(sign_src))
    return (code | np.where(neg, SIGN[elem], 0)).astype(np.uint8)


def scale_exponent(elem, amax):
    """floor(log2 amax) - emax(elem), clamped to [-127, 127]; amax == 0 -> -127."""
    _check_elem(elem)
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)                       # amax = f * 2**e, f in [0.5, 1)
    E = (e.astype(np.int64) - 1) - EMAX[elem]
    E = np.where(amax == 0, -127, E)
    return np.clip(E, -127, 127).astype(np.int64)


def quantize(elem, x):
    """fp32 x [R, K] -> (element codes uint8 [R, K], e8m0 scale codes uint8 [R, K/32])."""
    x = np.asarray(x, dtype=np.float32)
    R, K = x.shape
    if K % GROUP:
        raise ValueError(f"K={K} is not a multiple of {GROUP}")
    xb = x.reshape(R, K // GROUP, GROUP)
    E = scale_exponent(elem, np.abs(xb).max(axis=-1))
    y = xb.astype(np.float64) * np.ldexp(1.0, -E)[..., None]        # exact power of two
    return encode(elem, y, xb).reshape(R, K), (E + 127).astype(np.uint8)


def dequantize(elem, codes, scales):
    """Element codes [R, K] (unpacked) and e8m0 codes [R, K/32] -> float64 values."""
    codes = np.asarray(codes, dtype=np.uint8)
    R, K = codes.shape
    v = TABLE[elem][codes].reshape(R, K // GROUP, GROUP)
    return (v * F.E8M0_TABLE[np.asarray(scales, dtype=np.uint8)][..., None]).reshape(R, K)


def pack(elem, codes):
    """Element codes [R, K] -> packed bytes [R, K * bits / 8]."""
    codes = np.asarray(codes, dtype=np.uint8)
    if elem == "e4m3":
        return codes.copy()
    if elem == "e2m1":
        return F.pack_nibbles(codes)
    R, K = codes.shape
    g = codes.reshape(R, K // GROUP, GROUP).astype(np.uint64) & 0x3F
    out = np.zeros((R, K // GROUP, 24), dtype=np.uint8)
    for i in range(GROUP):                      # element i -> bits [6 i, 6 i + 6)
        bit = 6 * i
        byte, sh = bit // 8, bit % 8
        out[..., byte] |= ((g[..., i] << np.uint64(sh)) & 0xFF).astype(np.uint8)
        if sh > 2:                              # spills into the next byte
            out[..., byte + 1] |= (g[..., i] >> np.uint64(8 - sh)).astype(np.uint8)
    return out.reshape(R, K // GROUP * 24)


def unpack(elem, packed, K):
    packed = np.asarray(packed, dtype=np.uint8)
    if elem == "e4m3":
        return packed.copy()
    if elem == "e2m1":
        return F.unpack_nibbles(packed)
    R = packed.shape[0]
    g = packed.reshape(R, K // GROUP, 24).astype(np.uint64)
    out = np.empty((R, K // GROUP, GROUP), dtype=np.uint8)
    for i in range(GROUP):
        bit = 6 * i
        byte, sh = bit // 8, bit % 8
        v = g[..., byte] >> np.uint64(sh)
        if sh > 2:
            v |= g[..., byte + 1] << np.uint64(8 - sh)
        out[..., i] = (v & 0x3F).astype(np.uint8)
    return out.reshape(R, K)


def gemm(a_elem, a_codes, a_scales, w_elem, w_codes, w_scales):
    """out[m, n] = sum_k a_hat[m, k] w_hat[n, k] in float64 (unpacked codes)."""
    return dequantize(a_elem, a_codes, a_scales) @ dequantize(w_elem, w_codes, w_scales).T
