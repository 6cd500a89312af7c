"""MXFP8 and FP8 W8A8 by definition: quantize, dequantize, multiply in float64.

Test infrastructure: only tests, the smoke check and the bench's CPU-baseline leg use
this module.

Sources ("vLLM per-format kernel capability matrix derived from source"):
* its group-size note: MXFP4, MXFP6 and MXFP8 all use blocks of 32 elements;
* MXFP8 and WHAT IS NATIVE ON AMD: MXFP8 is the MX format with a native AMD path on
  gfx95 parts; its elements are FP8 e4m3 with an exponent-only (e8m0) block scale, as
  in every MX format;
* FP8, THREE SCALING MODES: per-tensor scales; block scales in the 1x128 (activations)
  / 128x128 (weights) layout; rowwise scales -- per token for activations, per output
  channel for weights, computed dynamically.  A part without per-token support falls
  back to per-tensor scaling silently on the page's engine; here every mode is asked
  for explicitly and none turns into another;
* the same page notes that gfx94-class parts use the FNUZ e4m3 variant; gfx950 uses
  OCP e4m3fn, the variant of formats.E4M3_TABLE.
The matrix itself is the emulation definition (THE EMULATION COLUMN): dequantize both
operands and multiply in high precision.

Readings where the pages are silent (listed in the design notes):
* MXFP8 block scale: the OCP MX rule with emax(e4m3) = 8: E = floor(log2 amax) - 8,
  clamped to [-127, 127], zero blocks E = -127; elements e4m3(x * 2**-E), rounded to
  nearest even, saturating at 448.
* FP8 dynamic scales (rowwise, block): s = fp32(amax / 448), so the largest magnitude
  maps to 448; elements e4m3(fp32(x / s)), nearest even, saturating at 448, sign kept;
  a block whose amax is 0 gets s = 0 and all-zero codes.  Per-tensor scales are given.
* blocks: activations 1 x 128 along K; weights 128 x 128 (rows n / 128, K / 128), the
  last block along N holding the rows that exist.
"""
import numpy as np

from . import formats as F

PER_TENSOR = "per_tensor"
ROWWISE = "rowwise"
BLOCK = "block"
MODES = (PER_TENSOR, ROWWISE, BLOCK)
BLK = 128          # FP8 block edge (1 x 128 activations, 128 x 128 weights)
MX_GROUP = 32      # MX block along K
E4M3_EMAX = 8      # largest e4m3 exponent: 448 = 1.75 * 2**8


def e4m3_encode(y):
    """fp32 values -> e4m3fn codes: nearest even, saturating at 448, sign bit = signbit."""
    y = np.asarray(y, dtype=np.float32)
    code = F.e4m3_encode_pos(np.abs(y))
    return (code | (np.signbit(y).astype(np.uint8) << 7)).astype(np.uint8)


def e4m3_decode(codes):
    return F.E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


# ----------------------------------------------------------------------------------
# MXFP8
# ----------------------------------------------------------------------------------


def mxfp8_scale_exponent(amax):
    """OCP MX scale exponent for e4m3 elements: floor(log2 amax) - 8, in [-127, 127]."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)                   # amax = f * 2**e, f in [0.5, 1)
    E = (e.astype(np.int64) - 1) - E4M3_EMAX
    E = np.where(amax == 0, -127, E)
    return np.clip(E, -127, 127).astype(np.int64)


def quantize_mxfp8(x):
    """fp32 x [R, K] -> (e4m3 codes uint8 [R, K], e8m0 scale codes uint8 [R, K/32])."""
    x = np.asarray(x, dtype=np.float32)
    R, K = x.shape
    if K % MX_GROUP:
        raise ValueError(f"K={K} is not a multiple of {MX_GROUP}")
    xb = x.reshape(R, K // MX_GROUP, MX_GROUP)
    E = mxfp8_scale_exponent(np.abs(xb).max(axis=-1))
    y = xb.astype(np.float64) * np.ldexp(1.0, -E)[..., None]       # exact
    codes = e4m3_encode(y.astype(np.float32))                       # exact conversion
    return codes.reshape(R, K), (E + 127).astype(np.uint8)


def dequantize_mxfp8(codes, scales):
    codes = np.asarray(codes, dtype=np.uint8)
    R, K = codes.shape
    s = F.E8M0_TABLE[np.asarray(scales, dtype=np.uint8)]
    return (e4m3_decode(codes).reshape(R, K // MX_GROUP, MX_GROUP) * s[..., None]).reshape(R, K)


def gemm_mxfp8(a_codes, a_scales, w_codes, w_scales):
    """C = a_hat @ w_hat^T in float64 (MX formats carry no per-tensor scale: alpha = 1)."""
    return dequantize_mxfp8(a_codes, a_scales) @ dequantize_mxfp8(w_codes, w_scales).T


# ----------------------------------------------------------------------------------
# FP8 W8A8 with per-tensor, rowwise or block scales
# ----------------------------------------------------------------------------------


def _quantize_by(x, s):
    """e4m3 codes of fp32 x divided by fp32 scales s (broadcast); s == 0 -> zero codes."""
    x = np.asarray(x, dtype=np.float32)
    s = np.asarray(s, dtype=np.float32)
    zero = s == 0
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        # one fp32 division; a quotient beyond fp32 becomes inf and saturates like any
        # value above 448
        y = (x / np.where(zero, np.float32(1.0), s)).astype(np.float32)
    y = np.where(zero, np.copysign(np.float32(0.0), x), y)
    return e4m3_encode(y.astype(np.float32))


def dynamic_scale(amax):
    """fp32(amax / 448) for fp32 amax."""
    return (np.asarray(amax, dtype=np.float32) / np.float32(F.E4M3_MAX)).astype(np.float32)


def quantize_act(mode, x, scale=None):
    """Activations x [M, K] (fp32 values of the bf16 input).

    per_tensor: codes = e4m3(x / scale), scale given (host fp32 > 0)
    rowwise:    scales [M] = amax(row) / 448, codes = e4m3(x / scales[m])
    block:      scales [M, K/128] = amax over 1 x 128 / 448
    Returns (codes uint8 [M, K], scales float32 or the given scalar)."""
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    if mode == PER_TENSOR:
        s = np.float32(scale)
        if not np.isfinite(s) or s <= 0:
            raise ValueError("per-tensor scale must be finite and positive")
        return _quantize_by(x, s), s
    if mode == ROWWISE:
        s = dynamic_scale(np.abs(x).max(axis=1))
        return _quantize_by(x, s[:, None]), s
    if mode == BLOCK:
        if K % BLK:
            raise ValueError(f"K={K} is not a multiple of {BLK}")
        xb = x.reshape(M, K // BLK, BLK)
        s = dynamic_scale(np.abs(xb).max(axis=-1))
        return _quantize_by(xb, s[..., None]).reshape(M, K), s
    raise ValueError(mode)


def quantize_weight(mode, w, scale=None):
    """Weights w [N, K] fp32.  per_tensor: given scale (default amax / 448); rowwise:
    per output channel [N]; block: [ceil(N/128), K/128] over 128 x 128 blocks."""
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    if mode == PER_TENSOR:
        s = dynamic_scale(np.abs(w).max()) if scale is None else np.float32(scale)
        return _quantize_by(w, s), np.float32(s)
    if mode == ROWWISE:
        return quantize_act(ROWWISE, w)
    if mode == BLOCK:
        if K % BLK:
            raise ValueError(f"K={K} is not a multiple of {BLK}")
        nb = -(-N // BLK)
        s = np.zeros((nb, K // BLK), dtype=np.float32)
        codes = np.empty((N, K), dtype=np.uint8)
        for b in range(nb):
            blk = w[b * BLK:(b + 1) * BLK].reshape(-1, K // BLK, BLK)
            s[b] = dynamic_scale(np.abs(blk).max(axis=(0, 2)))
            codes[b * BLK:(b + 1) * BLK] = _quantize_by(blk, s[b][None, :, None]).reshape(-1, K)
        return codes, s
    raise ValueError(mode)


def dequantize_act(mode, codes, scales):
    v = e4m3_decode(codes)
    M, K = v.shape
    if mode == PER_TENSOR:
        return v * float(scales)
    if mode == ROWWISE:
        return v * np.asarray(scales, np.float64)[:, None]
    return (v.reshape(M, K // BLK, BLK) * np.asarray(scales, np.float64)[..., None]).reshape(M, K)


def dequantize_weight(mode, codes, scales):
    v = e4m3_decode(codes)
    N, K = v.shape
    if mode in (PER_TENSOR, ROWWISE):
        return dequantize_act(mode, codes, scales)
    s = np.repeat(np.asarray(scales, np.float64), BLK, axis=0)[:N]          # [N, K/128]
    return (v.reshape(N, K // BLK, BLK) * s[..., None]).reshape(N, K)


def gemm(mode, a_codes, a_scales, w_codes, w_scales):
    """out[m, n] = sum_k a_hat[m, k] w_hat[n, k], float64, each operand dequantized with
    its own scales (the per-tensor product of the two scales is the GEMM's alpha)."""
    return dequantize_act(mode, a_codes, a_scales) @ dequantize_weight(mode, w_codes, w_scales).T
