"""GPU parity of the MX family of any element type (mx_quantize_act, mx_quantize_weight,
mx_gemm) against oracle/mx.py.

Definitions ("vLLM per-format kernel capability matrix derived from source"): MXFP4,
MXFP6 and MXFP8 use 32-element blocks with e8m0 scales (the group-size note); MXFP6
weights take MXFP4, MXFP6 or other activations (the MXFP6 section); the matmul is the
emulation definition (THE EMULATION COLUMN).

Quantization: packed codes and scales bit-exact.  Matmul tolerance, from the arithmetic:
the scaled MFMA's inner sum stays within 2^-12 of the sum of |products| of one
instruction (1.4e-4 was the largest seen for e4m3 operands), fp32 accumulation over K
adds at most K * 2^-24 of that sum, and the output rounding adds 2^-23 |C| (fp32) or
one bf16 ulp.  That bound is below the 2e-3 * ||a_hat_m|| * ||w_hat_n|| bound of the FP4
tests.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp4_quantize_amd as F
from block_scaled_fp4_quantize_amd import tensors as T
import synth
from oracle import mx as OX
from tests.gpu_util import DEV, bf16_dev, to_dev
from tests.test_gpu_fp8 import check_fp8_gemm, edge_values

pytestmark = pytest.mark.gpu

ELEMS = list(OX.ELEMS)


def oracle_packed(elem, x):
    codes, scales = OX.quantize(elem, x)
    return OX.pack(elem, codes), scales, codes


def assert_bit_exact(got_c, got_s, want_c, want_s, what):
    assert np.array_equal(got_s, want_s), f"{what}: scales differ at {np.argwhere(got_s != want_s)[:5]}"
    bad = np.argwhere(got_c != want_c)
    assert bad.size == 0, f"{what}: {len(bad)} code bytes differ, first at {bad[:5]}"


@pytest.mark.parametrize("shape", [(1, 32), (3, 96), (37, 512), (64, 4096), (2, 6144)])
@pytest.mark.parametrize("elem", ELEMS)
def test_act_quant_bit_exact(elem, shape):
    M, K = shape
    x = synth.normal((M, K), seed=41, role=synth.ACT, index=M * K)
    x = synth.with_outliers(x, 0.01, 20.0, seed=41, index=M)
    xd, xv = bf16_dev(x)
    codes, scales = T.mx_quantize_t(elem, xd)
    torch.cuda.synchronize()
    wc, ws, _ = oracle_packed(elem, xv)
    assert_bit_exact(codes.cpu().numpy(), scales.cpu().numpy(), wc, ws, f"{elem} {shape}")


@pytest.mark.parametrize("elem", ELEMS)
def test_act_quant_edge_values_and_strides(elem):
    x = edge_values((9, 1024), seed=43)
    pad = np.pad(x, ((0, 0), (0, 40)))
    xd, xv = bf16_dev(pad)
    codes, scales = T.mx_quantize_t(elem, xd[:, :1024])
    torch.cuda.synchronize()
    wc, ws, _ = oracle_packed(elem, xv[:, :1024])
    assert_bit_exact(codes.cpu().numpy(), scales.cpu().numpy(), wc, ws, f"{elem} edges")


@pytest.mark.parametrize("shape", [(300, 384), (1, 128), (257, 1024)])
@pytest.mark.parametrize("elem", ELEMS)
def test_weight_quant_bit_exact(elem, shape):
    N, K = shape
    w = synth.normal((N, K), 0.02, seed=47, role=synth.WEIGHT, index=N)
    if N > 5:
        w[5, :64] = 0.0
    codes, scales = T.mx_quantize_t(elem, to_dev(w))
    torch.cuda.synchronize()
    wc, ws, _ = oracle_packed(elem, w)
    assert_bit_exact(codes.cpu().numpy(), scales.cpu().numpy(), wc, ws, f"{elem} weights {shape}")


def operands(ae, we, M, N, K, seed):
    a = synth.with_outliers(synth.normal((M, K), seed=seed, role=synth.ACT, index=M), 0.01, 20.0,
                            seed=seed, index=M)
    _, av = synth.bf16_bits(a)
    w = synth.normal((N, K), 0.02, seed=seed, role=synth.WEIGHT, index=N)
    apk, asc, acodes = oracle_packed(ae, av)
    wpk, wsc, wcodes = oracle_packed(we, w)
    return apk, asc, wpk, wsc, OX.dequantize(ae, acodes, asc), OX.dequantize(we, wcodes, wsc)


PAIRS = [(a, w) for a in ELEMS for w in ELEMS]


@pytest.mark.parametrize("shape", [(1, 40, 128), (32, 300, 384), (33, 64, 256), (130, 520, 512)])
@pytest.mark.parametrize("ae,we", PAIRS)
def test_gemm_pairs(ae, we, shape):
    M, N, K = shape
    apk, asc, wpk, wsc, a_hat, w_hat = operands(ae, we, M, N, K, seed=M + N + K)
    for od in (torch.bfloat16, torch.float32):
        out = T.mx_gemm_t(ae, we, to_dev(apk), to_dev(asc), to_dev(wpk), to_dev(wsc), out_dtype=od)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        check_fp8_gemm(got, a_hat, w_hat, od == torch.bfloat16, K, f"{ae} x {we} {shape} {od}")


def test_gemm_strided_output_and_zero_blocks():
    M, N, K = 70, 96, 256
    apk, asc, wpk, wsc, a_hat, w_hat = operands("e2m3", "e3m2", M, N, K, seed=53)
    zero_c, zero_s, zc = oracle_packed("e2m3", np.zeros((1, K), np.float32))
    apk[4], asc[4] = zero_c[0], zero_s[0]
    a_hat[4] = 0.0
    big = torch.full((M, N + 3), 5.0, dtype=torch.float32, device=DEV)
    T.mx_gemm_t("e2m3", "e3m2", to_dev(apk), to_dev(asc), to_dev(wpk), to_dev(wsc), out=big[:, :N])
    torch.cuda.synchronize()
    b = big.cpu().numpy()
    assert np.all(b[:, N:] == 5.0), "the call wrote outside its output rows"
    assert np.all(b[4, :N] == 0.0)
    check_fp8_gemm(b[:, :N].astype(np.float64), a_hat, w_hat, False, K, "strided")


FULL = [("e4m3", "e2m1", 32, 14336, 4096), ("e2m3", "e2m3", 8192, 4096, 4096),
        ("e2m1", "e3m2", 8192, 4096, 4096), ("e4m3", "e2m3", 8, 14336, 4096)]


@pytest.mark.parametrize("ae,we,M,N,K", FULL)
def test_full_size_sampled(ae, we, M, N, K):
    """The device chain at the benchmarked sizes: both quantizations on the device, their
    codes checked bit-exact (weights in full, activations on sampled rows), the GEMM
    checked on the sampled rows."""
    a = synth.with_outliers(synth.normal((M, K), seed=59, role=synth.ACT, index=M), 0.01, 20.0,
                            seed=59, index=M)
    w = synth.normal((N, K), 0.02, seed=59, role=synth.WEIGHT, index=N)
    ad, av = bf16_dev(a)
    wc, ws = T.mx_quantize_t(we, to_dev(w))
    ac, asc = T.mx_quantize_t(ae, ad)
    out = T.mx_gemm_t(ae, we, ac, asc, wc, ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(61)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, min(M, 24), replace=False)]))
    rwc, rws, rw_codes = oracle_packed(we, w)
    assert_bit_exact(wc.cpu().numpy(), ws.cpu().numpy(), rwc, rws, f"{we} weights")
    rac, ras, ra_codes = oracle_packed(ae, av[rows])
    assert_bit_exact(ac.cpu().numpy()[rows], asc.cpu().numpy()[rows], rac, ras, f"{ae} rows")
    got = out.float().cpu().numpy().astype(np.float64)[rows]
    check_fp8_gemm(got, OX.dequantize(ae, ra_codes, ras), OX.dequantize(we, rw_codes, rws), True, K,
                   f"{ae} x {we} M={M} N={N} K={K}")
