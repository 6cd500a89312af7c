"""GPU checks of the one-time weight preparation (fp4_prepare_weights) and of fp4_gemm
reading prepared weights.

Source: "vLLM on the NVIDIA DGX Spark (GB10 / sm_121): A Complete Technical Guide", §4.3
(scale factors converted to the MMA layout once, when the weights are loaded) and §5.3
(the block scales repacked for the dequant kernel).  The prepared layout is checked
byte for byte against a repack written here from its definition; matmuls on prepared
weights must equal those on row-major weights bit for bit (the same kernels and
arithmetic, only the addresses of the weight loads differ) and match the oracle to the
GEMM tolerance; a NaN block scale is refused.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp4_quantize_amd as F
from block_scaled_fp4_quantize_amd import tensors as T
import synth
from oracle import gemm as OG
from oracle import quant as OQ
from tests.gpu_util import DEV, bf16_dev, check_gemm, dequant, to_dev, weights

pytestmark = pytest.mark.gpu

FMTS = {"nvfp4": F.FP4_NVFP4, "mxfp4": F.FP4_MXFP4}


def host_prepared(codes, N, K):
    """The layout's definition: blocks of 16 rows x 64 bytes (128 elements), ordered by
    row block then K block; piece 16 q + r of a block = bytes 16 q .. 16 q + 15 of row r."""
    c = np.asarray(codes).reshape(N // 16, 16, K // 128, 4, 16)      # [g, r, s, q, byte]
    return np.ascontiguousarray(c.transpose(0, 2, 3, 1, 4)).reshape(-1)


def prepare(fmt, wc, ws, N, K):
    out = torch.empty(F.fp4_prepared_weight_bytes(N, K), dtype=torch.uint8, device=DEV)
    chk = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    st = F.fp4_prepare_weights(FMTS[fmt], wc, ws, N, K, out, chk, check=False)
    return out, st


@pytest.mark.parametrize("fmt", list(FMTS))
@pytest.mark.parametrize("N,K", [(16, 128), (48, 512), (4096, 4096)])
def test_prepared_layout(fmt, N, K):
    wc, ws, _ = weights(fmt, N, K, seed=N + K)
    out, st = prepare(fmt, to_dev(wc), to_dev(ws), N, K)
    torch.cuda.synchronize()
    assert st == F.FP4_OK
    assert np.array_equal(out.cpu().numpy(), host_prepared(wc, N, K))


@pytest.mark.parametrize("fmt", list(FMTS))
def test_nan_scale_refused(fmt):
    N, K = 32, 256
    wc, ws, _ = weights(fmt, N, K, seed=3)
    ws = ws.copy()
    ws[7, 3] = 0xFF if fmt == "mxfp4" else 0x7F        # e8m0 NaN / e4m3 NaN
    _, st = prepare(fmt, to_dev(wc), to_dev(ws), N, K)
    assert st == F.FP4_ERR_WEIGHT_SCALE
    if fmt == "nvfp4":
        ws[7, 3] = 0xFF                                  # negative-signed NaN too
        _, st = prepare(fmt, to_dev(wc), to_dev(ws), N, K)
        assert st == F.FP4_ERR_WEIGHT_SCALE


@pytest.mark.parametrize("fmt", list(FMTS))
@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (5, 48, 512), (16, 64, 1024), (17, 80, 256),
                                   (32, 14336, 4096), (64, 96, 384), (8, 256, 4096)])
def test_gemm_on_prepared_weights(fmt, M, N, K):
    f = FMTS[fmt]
    wc, ws, ws2 = weights(fmt, N, K, seed=M + N)
    wcd, wsd = to_dev(wc), to_dev(ws)
    wp, st = prepare(fmt, wcd, wsd, N, K)
    assert st == F.FP4_OK
    a = synth.with_outliers(synth.normal((M, K), seed=M, role=synth.ACT, index=K), 0.01, 20.0,
                            seed=M, index=N)
    ad, av = bf16_dev(a)
    s = float(np.float32(np.abs(av).max()) / np.float32(2688.0)) if fmt == "nvfp4" else 1.0
    ac, asc = T.quantize_act(fmt, ad, s)
    outs = []
    for w_codes, flags in ((wcd, 0), (wp, F.FP4_FLAG_PREPARED_WEIGHTS)):
        out = torch.empty((M, N), dtype=torch.float32, device=DEV)
        st = F.fp4_gemm(f, F.FP4_W4A4, M, N, K, None, 0, ac, asc, w_codes, wsd, ws2, s, out, N,
                        F.FP4_OUT_F32, flags, None, 0, check=False)
        assert st == F.FP4_OK
        outs.append(out)
    # the fused activation quantization path reads the prepared weights too
    fused, st = T.gemm(fmt, "w4a4", wp.view(N, K // 2), wsd, a_bf16=ad, weight_scale_2=ws2,
                       input_scale=s, out_dtype=torch.float32, flags=F.FP4_FLAG_PREPARED_WEIGHTS)
    assert st == F.FP4_OK
    torch.cuda.synchronize()
    plain, prep = outs[0].cpu().numpy(), outs[1].cpu().numpy()
    assert np.array_equal(plain.view(np.uint32), prep.view(np.uint32))
    assert np.array_equal(plain.view(np.uint32), fused.cpu().numpy().view(np.uint32))
    rows = np.unique(np.linspace(0, M - 1, min(M, 8)).astype(int))
    ac_r, as_r = OQ.quantize_packed(fmt, av[rows], s)
    ref = OG.alpha(fmt, OG.W4A4, ws2, s) * (dequant(fmt, ac_r, as_r) @ dequant(fmt, wc, ws).T)
    check_gemm(prep[rows].astype(np.float64), ref, dequant(fmt, ac_r, as_r), dequant(fmt, wc, ws),
               OG.alpha(fmt, OG.W4A4, ws2, s), False, what=f"{fmt} prepared M={M} N={N} K={K}")


def test_noalloc_gemm_on_prepared_weights():
    M, N, K = 8, 64, 512
    wc, ws, _ = weights("mxfp4", N, K, seed=9)
    wcd, wsd = to_dev(wc), to_dev(ws)
    wp, st = prepare("mxfp4", wcd, wsd, N, K)
    assert st == F.FP4_OK
    ad, _ = bf16_dev(synth.normal((M, K), seed=9, role=synth.ACT))
    o1 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    o2 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    F.fp4_gemm_noalloc(F.FP4_MXFP4, F.FP4_W4A4, M, N, K, ad, K, None, None, wcd, wsd, 1.0, 1.0,
                       o1, N, F.FP4_OUT_F32, 0)
    F.fp4_gemm_noalloc(F.FP4_MXFP4, F.FP4_W4A4, M, N, K, ad, K, None, None, wp, wsd, 1.0, 1.0,
                       o2, N, F.FP4_OUT_F32, F.FP4_FLAG_PREPARED_WEIGHTS)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
