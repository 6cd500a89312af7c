"""NVFP4 and MXFP4 quantize / dequantize, written from the format definitions.

Test infrastructure: only tests, the smoke check and the bench's CPU-baseline leg
use this module.

Sources
* "vLLM on the NVIDIA DGX Spark (GB10 / sm_121): A Complete Technical Guide",
  §6.1 (NVFP4 format): the value of an element is the e2m1 element times its fp8
  e4m3 block scale (one per 16 elements along K) times an fp32 global scale.
* Same guide, §6.4 (NVFP4 vs MXFP4 table): MXFP4 has 32-element blocks and an e8m0
  scale, and no per-tensor scale.
* Same guide, §4.3 (b12x): the fused MoE quantizes BF16 activations to FP4 inside
  the kernel -- the activation quantizer below is that step.
* "GLM-5.3-Flash on vLLM, on GB10": the stored per-tensor scales are dequant
  multipliers (alpha = weight_scale_2 * input_scale).  The guide's §6.1 writes the
  kernel's alpha as a reciprocal of "global scales"; those global scales are read
  as the quantize-direction multipliers g = 1 / input_scale.  Only this reading
  makes a zero input_scale give alpha = 0, which is the GLM page's failure.

Readings where the pages are silent (each also listed in the design notes):
* block scale choice (NVFP4): sf = fp32(fp32(amax * g) / 6), rounded to e4m3 RNE
  with saturation at 448; elements are scaled by r = fp32(g / scale) and rounded to
  e2m1 RNE with saturation at 6; an all-zero scale gives zero elements that keep
  the sign of x.  The fp32 operation order is a chosen convention (parity
  unpinned by the pages), pinned by the hand-worked examples in tests/golden.
* block scale choice (MXFP4): the OCP MX rule, see formats.mx_scale_exponent.
* input_scale must be finite and lie in [2**-100, 2**100]; outside that range the
  scaled values can overflow or leave the normal fp32 range, and the call is
  refused (the zero scale of the GLM page is the case that matters).
"""
import numpy as np

from . import formats as F

NVFP4 = "nvfp4"
MXFP4 = "mxfp4"
GROUP = {NVFP4: 16, MXFP4: 32}

SCALE_MIN = 2.0 ** -100
SCALE_MAX = 2.0 ** 100


class InputScaleError(ValueError):
    """A W4A4 activation scale that is zero, negative, non-finite or out of range."""


class WeightScaleError(ValueError):
    """A weight_scale_2 that is zero, negative, non-finite or out of range."""


def check_scale(s, exc=InputScaleError):
    s = float(np.float32(s))
    if not np.isfinite(s) or not (SCALE_MIN <= s <= SCALE_MAX):
        raise exc(f"scale {s!r} is not a finite value in [2**-100, 2**100]")
    return np.float32(s)


def _rows(x, group):
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("expected a [rows, K] matrix")
    R, K = x.shape
    if K % group:
        raise ValueError(f"K={K} is not a multiple of the block size {group}")
    return x, R, K


def quantize_nvfp4(x, input_scale):
    """NVFP4 quantization of fp32 values x [R, K] under a per-tensor scale.

    Returns (codes uint8 [R, K] in 0..15, scale codes uint8 [R, K/16]).
    All scale arithmetic is fp32 with correctly rounded operations, in this order:
      g  = 1 / s                       (once)
      sf = (amax * g) / 6              per 16-element block
      sc = e4m3(sf), sd = value(sc)
      r  = g / sd,  q = e2m1(x * r)    (q = signed zero when sd == 0)
    """
    s = check_scale(input_scale)
    x, R, K = _rows(x, 16)
    g = np.float32(1.0) / s
    xb = x.reshape(R, K // 16, 16)
    amax = np.abs(xb).max(axis=-1)                         # exact in fp32
    sf = (amax * g) / np.float32(6.0)                      # two fp32 roundings
    sc = F.e4m3_encode_pos(sf)
    sd = F.E4M3_TABLE[sc].astype(np.float32)               # exact
    zero = sd == 0
    with np.errstate(divide="ignore"):
        r = np.where(zero, np.float32(0.0), g / np.where(zero, np.float32(1.0), sd))
    r = r.astype(np.float32)
    y = (xb * r[..., None]).astype(np.float32)            # fp32 product
    q = F.e2m1_encode(y)
    signed_zero = (np.signbit(xb).astype(np.uint8) << 3)
    q = np.where(zero[..., None], signed_zero, q).astype(np.uint8)
    return q.reshape(R, K), sc.astype(np.uint8)


def quantize_mxfp4(x):
    """MXFP4 quantization of fp32 values x [R, K] (no per-tensor scale).

    Returns (codes uint8 [R, K], scale codes uint8 [R, K/32]) with
      E = clamp(floor(log2(amax)) - 2, -127, 127), q = e2m1(x * 2**-E), code = E + 127.
    """
    x, R, K = _rows(x, 32)
    xb = x.reshape(R, K // 32, 32)
    amax = np.abs(xb).max(axis=-1)
    E = F.mx_scale_exponent(amax)
    y = xb.astype(np.float64) * np.ldexp(1.0, -E)[..., None]    # exact power-of-two scaling
    q = _e2m1_encode_f64(y, xb)
    return q.reshape(R, K), (E + 127).astype(np.uint8)


def _e2m1_encode_f64(y, x_sign_src):
    """e2m1 codes of exact float64 values y, sign bit taken from x."""
    code = F._nearest_code(np.abs(y), F._E2M1_POS)
    sign = np.signbit(x_sign_src).astype(np.uint8) << 3
    return (code | sign).astype(np.uint8)


def quantize(fmt, x, input_scale=1.0):
    """Dispatch on format.  MXFP4 has no per-tensor scale: input_scale must be 1."""
    if fmt == NVFP4:
        return quantize_nvfp4(x, input_scale)
    if fmt == MXFP4:
        if float(input_scale) != 1.0:
            raise ValueError("MXFP4 carries no per-tensor scale; input_scale must be 1")
        return quantize_mxfp4(x)
    raise ValueError(f"unknown format {fmt!r}")


def block_scale_values(fmt, scale_codes):
    """Decoded block scales (float64)."""
    sc = np.asarray(scale_codes, dtype=np.uint8)
    if fmt == NVFP4:
        v = F.E4M3_TABLE[sc]
    elif fmt == MXFP4:
        v = F.E8M0_TABLE[sc]
    else:
        raise ValueError(fmt)
    if np.isnan(v).any():
        raise ValueError("NaN block scale code")
    return v


def dequantize(fmt, codes, scale_codes):
    """Exact dequantized values (float64) of codes [R, K] with block scales [R, K/G].

    The per-tensor scale is not applied here: it is part of the GEMM's alpha.
    """
    G = GROUP[fmt]
    codes = np.asarray(codes, dtype=np.uint8)
    R, K = codes.shape
    elem = F.E2M1_TABLE[codes & 0xF]
    sv = block_scale_values(fmt, scale_codes).reshape(R, K // G)
    return (elem.reshape(R, K // G, G) * sv[..., None]).reshape(R, K)


def weight_scale_2(w):
    """Per-tensor NVFP4 weight scale: fp32(amax(W) / (6 * 448)).

    This puts the largest block scale at the top of the e4m3 range, so the largest
    weight maps to 6 * 448 in the scaled domain.  (Reading: the pages give the
    per-tensor scale's role, not its calibration; this is the usual choice.)
    """
    w = np.asarray(w, dtype=np.float32)
    amax = np.float32(np.abs(w).max())
    s = amax / np.float32(6.0 * 448.0)
    return check_scale(s, WeightScaleError)


def quantize_weight(fmt, w):
    """Offline weight quantization (the synthetic checkpoint), not the hot path.

    NVFP4: (packed codes [N, K/2], scale codes [N, K/16], weight_scale_2).
    MXFP4: (packed codes [N, K/2], scale codes [N, K/32], 1.0).
    """
    if fmt == NVFP4:
        ws2 = weight_scale_2(w)
        q, sc = quantize_nvfp4(w, ws2)
        return F.pack_nibbles(q), sc, float(ws2)
    q, sc = quantize_mxfp4(w)
    return F.pack_nibbles(q), sc, 1.0


def quantize_packed(fmt, x, input_scale=1.0):
    """Activation quantization with packed output: (codes [R, K/2], scales [R, K/G])."""
    q, sc = quantize(fmt, x, input_scale)
    return F.pack_nibbles(q), sc


def dequantize_packed(fmt, packed, scale_codes):
    return dequantize(fmt, F.unpack_nibbles(packed), scale_codes)
