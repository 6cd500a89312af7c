"""GPU parity of the FP8 family (fp8_quantize_act, fp8_quantize_weight, fp8_gemm)
against oracle/fp8.py.

Definitions ("vLLM per-format kernel capability matrix derived from source"): MXFP8 =
e4m3 elements with an e8m0 scale per 32 along K (the MX group-size note, the MXFP8
section); FP8 W8A8 with per-tensor, rowwise or 1x128 / 128x128 block scales (FP8, THREE
SCALING MODES); the matmul is the emulation definition (THE EMULATION COLUMN).

Quantization: codes and scales bit-exact.  Matmul tolerance, from the arithmetic: the
e4m3 MFMA's inner sum was measured to stay within 1.4e-4 of the sum of |products| of one
instruction, so it is bounded here by 2^-12 * sum_k |a_hat w_hat|; fp32 accumulation over
K adds at most K * 2^-24 of the same sum; the output rounding adds 2^-23 |C| (fp32) or one
bf16 ulp.  That per-element bound is also below the 2e-3 * ||a_hat_m|| * ||w_hat_n|| bound
of the FP4 tests (the sum of |products| is at most the product of the norms).
"""
import numpy as np
import pytest
import torch

import block_scaled_fp4_quantize_amd as F
from block_scaled_fp4_quantize_amd import tensors as T
import synth
from oracle import fp8 as O8
from tests.gpu_util import DEV, bf16_dev, bf16_ulp, round_bf16, to_dev

pytestmark = pytest.mark.gpu

MODES = {"mx": F.FP8_MX, "per_tensor": F.FP8_PER_TENSOR, "rowwise": F.FP8_ROWWISE,
         "block": F.FP8_BLOCK}
ORACLE_MODE = {"per_tensor": O8.PER_TENSOR, "rowwise": O8.ROWWISE, "block": O8.BLOCK}


def oracle_quant(mode, x, weight, scale=None):
    """(codes, scales) of the oracle for fp32 values x."""
    if mode == "mx":
        return O8.quantize_mxfp8(x)
    f = O8.quantize_weight if weight else O8.quantize_act
    return f(ORACLE_MODE[mode], x, scale)


def oracle_hat(mode, codes, scales, weight):
    if mode == "mx":
        return O8.dequantize_mxfp8(codes, scales)
    f = O8.dequantize_weight if weight else O8.dequantize_act
    return f(ORACLE_MODE[mode], codes, scales)


def act_tensor_scale(x):
    """A per-tensor activation scale that lets the top 2% of the values saturate."""
    return float(np.float32(np.quantile(np.abs(x), 0.98)) / np.float32(300.0))


def edge_values(shape, seed):
    """Values on e4m3 rounding decisions (midpoints of the e4m3 grid times powers of two),
    signed zeros, bf16 subnormals, huge values, and whole zero rows / blocks."""
    rng = np.random.default_rng(seed)
    n = int(np.prod(shape))
    mant = (1.0 + (rng.integers(0, 8, n) + 0.5) / 8.0)
    v = (mant * 2.0 ** rng.integers(-20, 12, n) * rng.choice([-1.0, 1.0], n)).astype(np.float32)
    sel = rng.random(n)
    v[sel < 0.04] = 0.0
    v[(sel >= 0.04) & (sel < 0.07)] = -0.0
    sub = (sel >= 0.07) & (sel < 0.09)
    v[sub] = (rng.integers(1, 127, sub.sum()) * 2.0 ** -133).astype(np.float32)
    big = (sel >= 0.09) & (sel < 0.095)
    v[big] = np.float32(3.0e38)
    v = v.reshape(shape)
    v[0] = 0.0                                  # an all-zero row (zero dynamic scale)
    if shape[0] > 2:
        v[2, :shape[1] // 2] = -0.0             # a row half negative zeros
    return v


def run_act(mode, x_f32, ts=1.0, ldx_pad=0):
    M, K = x_f32.shape
    xd, xv = bf16_dev(np.pad(x_f32, ((0, 0), (0, ldx_pad))))
    xd = xd[:, :K] if ldx_pad else xd
    codes, scales = T.fp8_quantize_act_t(MODES[mode], xd, ts)
    torch.cuda.synchronize()
    rc, rs = oracle_quant(mode, xv[:, :K], False, ts if mode == "per_tensor" else None)
    return codes.cpu().numpy(), None if scales is None else scales.cpu().numpy(), rc, rs


def assert_same(got_c, got_s, rc, rs, mode):
    if mode != "per_tensor":
        gs = np.asarray(got_s)
        rs = np.asarray(rs)
        if mode != "mx":          # fp32 scales: compare bit patterns
            gs, rs = gs.view(np.uint32), rs.astype(np.float32).view(np.uint32)
        assert np.array_equal(gs, rs), f"{mode}: scales differ at {np.argwhere(gs != rs)[:5]}"
    bad = np.argwhere(got_c != rc)
    assert bad.size == 0, f"{mode}: {len(bad)} codes differ, first at {bad[:5]}"


ACT_SHAPES = [(1, 128), (3, 256), (37, 512), (64, 4096), (2, 6144), (5, 96), (7, 72)]


@pytest.mark.parametrize("shape", ACT_SHAPES)
@pytest.mark.parametrize("mode", list(MODES))
def test_act_quant_bit_exact(mode, shape):
    M, K = shape
    if K % {"mx": 32, "block": 128}.get(mode, 8):
        # K is not a multiple of this mode's block: refused on the host, nothing written
        xd = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
        codes = torch.full((M, K), 0x5A, dtype=torch.uint8, device=DEV)
        scales = torch.zeros((M, K // 8 + 1), dtype=torch.float32, device=DEV)
        st = F.fp8_quantize_act(MODES[mode], xd, M, K, K, 1.0, codes, scales, check=False)
        assert st == F.FP4_ERR_SHAPE
        assert bool((codes == 0x5A).all())
        return
    x = synth.normal((M, K), seed=3, role=synth.ACT, index=M * K)
    x = synth.with_outliers(x, 0.01, 20.0, seed=3, index=M)
    ts = act_tensor_scale(x) if mode == "per_tensor" else 1.0
    assert_same(*run_act(mode, x, ts), mode)


@pytest.mark.parametrize("mode", list(MODES))
def test_act_quant_edge_values(mode):
    x = edge_values((9, 1024), seed=5)
    ts = 2.0 ** -6 if mode == "per_tensor" else 1.0
    assert_same(*run_act(mode, x, ts), mode)


@pytest.mark.parametrize("mode", list(MODES))
def test_act_quant_strided_rows(mode):
    x = synth.normal((6, 256), seed=7, role=synth.ACT, index=1)
    ts = 0.01 if mode == "per_tensor" else 1.0
    assert_same(*run_act(mode, x, ts, ldx_pad=24), mode)


@pytest.mark.parametrize("shape", [(300, 384), (128, 256), (1, 128), (257, 1024)])
@pytest.mark.parametrize("mode", list(MODES))
def test_weight_quant_bit_exact(mode, shape):
    N, K = shape
    w = synth.normal((N, K), 0.02, seed=11, role=synth.WEIGHT, index=N)
    if N > 5:
        w[5] = 0.0                              # an all-zero output channel
    ts = float(np.float32(np.abs(w).max()) / np.float32(448.0)) if mode == "per_tensor" else 1.0
    codes, scales = T.fp8_quantize_weight_t(MODES[mode], to_dev(w), ts)
    torch.cuda.synchronize()
    rc, rs = oracle_quant(mode, w, True, ts if mode == "per_tensor" else None)
    assert_same(codes.cpu().numpy(), None if scales is None else scales.cpu().numpy(), rc, rs, mode)


# ---- matmul -----------------------------------------------------------------------------


def operands(mode, M, N, K, seed, outliers=True):
    """Oracle-quantized operands (the GEMM test takes none of its inputs from the device
    quantizer): returns host codes/scales, tensor scales and the dequantized operands."""
    a = synth.normal((M, K), seed=seed, role=synth.ACT, index=M)
    if outliers:
        a = synth.with_outliers(a, 0.01, 20.0, seed=seed, index=M)
    _, av = synth.bf16_bits(a)
    w = synth.normal((N, K), 0.02, seed=seed, role=synth.WEIGHT, index=N)
    ats = act_tensor_scale(av) if mode == "per_tensor" else None
    wts = float(np.float32(np.abs(w).max()) / np.float32(448.0)) if mode == "per_tensor" else None
    ac, asc = oracle_quant(mode, av, False, ats)
    wc, wsc = oracle_quant(mode, w, True, wts)
    return ac, asc, ats, wc, wsc, wts


def dev_scales(mode, s):
    if mode == "per_tensor":
        return None
    return to_dev(np.ascontiguousarray(s, dtype=np.uint8 if mode == "mx" else np.float32))


def run_gemm(mode, ac, asc, ats, wc, wsc, wts, out_dtype):
    out = T.fp8_gemm_t(MODES[mode], to_dev(ac), dev_scales(mode, asc), to_dev(wc),
                       dev_scales(mode, wsc), ats or 1.0, wts or 1.0, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def check_fp8_gemm(got, a_hat, w_hat, out_bf16, K, what):
    ref = a_hat @ w_hat.T
    mag = np.abs(a_hat) @ np.abs(w_hat).T
    bound = (2.0 ** -12 + K * 2.0 ** -24) * mag
    if out_bf16:
        ref_c = round_bf16(ref)
        bound = bound + bf16_ulp(ref_c)
    else:
        ref_c = ref
        bound = bound + 2.0 ** -23 * np.abs(ref)
    err = np.abs(got - ref_c)
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} elements over the bound, first at "
                           f"{np.argwhere(bad)[:3].tolist()}, worst ratio "
                           f"{float((err / np.maximum(bound, 1e-300)).max()):.3g}")
    den = np.linalg.norm(ref_c)
    if den > 0:
        r = np.linalg.norm(got - ref_c) / den
        assert r <= 1e-3, f"{what}: relative Frobenius error {r:.3g}"


GEMM_SHAPES = [(1, 8, 128), (5, 40, 256), (32, 300, 384), (33, 64, 128), (130, 300, 512),
               (257, 520, 1024), (20, 1000, 640)]


@pytest.mark.parametrize("shape", GEMM_SHAPES)
@pytest.mark.parametrize("mode", list(MODES))
def test_gemm_small(mode, shape):
    M, N, K = shape
    ac, asc, ats, wc, wsc, wts = operands(mode, M, N, K, seed=M + N)
    a_hat = oracle_hat(mode, ac, asc if mode != "per_tensor" else ats, False)
    w_hat = oracle_hat(mode, wc, wsc if mode != "per_tensor" else wts, True)
    for od in (torch.bfloat16, torch.float32):
        got = run_gemm(mode, ac, asc, ats, wc, wsc, wts, od)
        check_fp8_gemm(got, a_hat, w_hat, od == torch.bfloat16, K,
                       f"{mode} M={M} N={N} K={K} {od}")


@pytest.mark.parametrize("mode", list(MODES))
def test_gemm_zero_rows_and_blocks(mode):
    """All-zero activation rows (zero dynamic scales) give exact zeros."""
    M, N, K = 40, 64, 256
    ac, asc, ats, wc, wsc, wts = operands(mode, M, N, K, seed=17, outliers=False)
    a = np.zeros((M, K), np.float32)
    ac2, asc2 = oracle_quant(mode, a, False, ats)
    ac[3], ac[35] = ac2[3], ac2[35]
    if mode == "mx":
        asc[3], asc[35] = asc2[3], asc2[35]
    elif mode in ("rowwise", "block"):
        asc[3], asc[35] = 0.0, 0.0
    got = run_gemm(mode, ac, asc, ats, wc, wsc, wts, torch.float32)
    assert np.all(got[3] == 0) and np.all(got[35] == 0)
    a_hat = oracle_hat(mode, ac, asc if mode != "per_tensor" else ats, False)
    w_hat = oracle_hat(mode, wc, wsc if mode != "per_tensor" else wts, True)
    check_fp8_gemm(got, a_hat, w_hat, False, K, f"{mode} zero rows")


@pytest.mark.parametrize("mode", list(MODES))
def test_gemm_strided_output(mode):
    M, N, K = 70, 96, 256
    ac, asc, ats, wc, wsc, wts = operands(mode, M, N, K, seed=23)
    big = torch.full((M, N + 5), 7.0, dtype=torch.float32, device=DEV)
    out = big[:, :N]
    T.fp8_gemm_t(MODES[mode], to_dev(ac), dev_scales(mode, asc), to_dev(wc),
                 dev_scales(mode, wsc), ats or 1.0, wts or 1.0, out=out)
    torch.cuda.synchronize()
    b = big.cpu().numpy()
    assert np.all(b[:, N:] == 7.0), "the call wrote outside its output rows"
    a_hat = oracle_hat(mode, ac, asc if mode != "per_tensor" else ats, False)
    w_hat = oracle_hat(mode, wc, wsc if mode != "per_tensor" else wts, True)
    check_fp8_gemm(b[:, :N].astype(np.float64), a_hat, w_hat, False, K, f"{mode} strided")


# ---- the benchmarked sizes: device quantizer + GEMM, sampled rows ------------------------

FULL = [("mx", 32, 14336, 4096), ("rowwise", 32, 14336, 4096), ("mx", 8192, 4096, 4096),
        ("block", 8192, 4096, 4096), ("per_tensor", 8192, 4096, 4096)]


@pytest.mark.parametrize("mode,M,N,K", FULL)
def test_full_size_sampled(mode, M, N, K):
    """The device chain at the benchmarked sizes (activation quantization then GEMM);
    the device codes of sampled rows are checked bit-exact, their outputs to the bound."""
    a = synth.normal((M, K), seed=29, role=synth.ACT, index=M)
    a = synth.with_outliers(a, 0.01, 20.0, seed=29, index=M)
    w = synth.normal((N, K), 0.02, seed=29, role=synth.WEIGHT, index=N)
    ad, av = bf16_dev(a)
    wts = float(np.float32(np.abs(w).max()) / np.float32(448.0)) if mode == "per_tensor" else 1.0
    ats = act_tensor_scale(av[:256]) if mode == "per_tensor" else 1.0
    m = MODES[mode]
    wc, ws = T.fp8_quantize_weight_t(m, to_dev(w), wts)
    ac, asc = T.fp8_quantize_act_t(m, ad, ats)
    out = T.fp8_gemm_t(m, ac, asc, wc, ws, ats, wts)
    torch.cuda.synchronize()
    rng = np.random.default_rng(31)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, min(M, 24), replace=False)]))
    rwc, rws = oracle_quant(mode, w, True, wts if mode == "per_tensor" else None)
    assert_same(wc.cpu().numpy(), None if ws is None else ws.cpu().numpy(), rwc, rws, mode)
    rac, ras = oracle_quant(mode, av[rows], False, ats if mode == "per_tensor" else None)
    gac = ac.cpu().numpy()[rows]
    gas = None if asc is None else asc.cpu().numpy()[rows]
    assert_same(gac, gas, rac, ras, mode)
    a_hat = oracle_hat(mode, rac, ras, False)
    w_hat = oracle_hat(mode, rwc, rws, True)
    got = out.float().cpu().numpy().astype(np.float64)[rows]
    check_fp8_gemm(got, a_hat, w_hat, True, K, f"{mode} M={M} N={N} K={K}")
