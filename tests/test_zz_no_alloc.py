"""fp4_gemm_noalloc, the allocation-free variant of fp4_gemm (for callers that
cannot allocate device memory), against fp4_gemm itself through the C ABI.

Both run the same kernels, so their outputs must agree bit for bit (stricter than the
GEMM tolerance, which the GEMM tests already hold fp4_gemm to).  Two calls in a row,
the second smaller than the first, so that what the first left in the shared scratch
array cannot leak into the second; a call too large for the array is refused before
any launch.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp4_quantize_amd as F
import synth
from tests.gpu_util import DEV, bf16_dev, to_dev, weights

pytestmark = pytest.mark.gpu


def _pair(fmt, M, N, K, seed, out_dtype=torch.bfloat16):
    """(fp4_gemm output, fp4_gemm_noalloc output) for one fused W4A4 problem."""
    wc, ws, ws2 = weights(fmt, N, K, seed)
    ad, av = bf16_dev(synth.normal((M, K), seed=seed, role=synth.ACT, index=M))
    s = float(np.float32(np.abs(av).max()) / np.float32(2688.0)) if fmt == "nvfp4" else 1.0
    wcd, wsd = to_dev(wc), to_dev(ws)
    od = F.FP4_OUT_F32 if out_dtype == torch.float32 else F.FP4_OUT_BF16
    ref = torch.full((M, N), float("nan"), dtype=out_dtype, device=DEV)
    need = F.fp4_gemm_workspace_size(fmt, "w4a4", M, K, 1)
    wsb = torch.empty(need, dtype=torch.uint8, device=DEV)
    st = F.fp4_gemm(fmt, "w4a4", M, N, K, ad, K, None, None, wcd, wsd, ws2, s, ref, N, od, 0,
                    wsb, need)
    assert st == F.FP4_OK
    got = torch.full((M, N), float("nan"), dtype=out_dtype, device=DEV)
    st = F.fp4_gemm_noalloc(fmt, "w4a4", M, N, K, ad, K, None, None, wcd, wsd, ws2, s, got, N, od)
    assert st == F.FP4_OK
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_noalloc_equals_fp4_gemm_two_calls(fmt):
    # a prefill-shaped call (tiled kernel), then a smaller decode-shaped one
    for M, N, K, od in ((320, 512, 2048, torch.bfloat16), (7, 256, 1024, torch.float32)):
        ref, got = _pair(fmt, M, N, K, seed=M + N, out_dtype=od)
        assert torch.equal(ref, got), f"{fmt} M={M} N={N} K={K}"
        assert not torch.isnan(got).any()



@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_noalloc_big_tile_relayout_two_calls(fmt):
    # dense shapes on the 4-wave 256 x 256 tile: fp4_gemm with the plain fused workspace
    # reads the block scales row by row, fp4_gemm_noalloc first re-lays them in stage
    # order into the scratch array (after the quantized activations); same bits.  The
    # second call is smaller than the first.
    for M, N, K in ((2300, 7324, 384), (2049, 7324, 128)):
        ref, got = _pair(fmt, M, N, K, seed=M + N + 1, out_dtype=torch.float32)
        assert F.fp4_last_kernel() == f"big_{fmt}_256"
        assert torch.equal(ref.view(torch.int32), got.view(torch.int32)), f"{fmt} M={M} N={N} K={K}"
        assert not torch.isnan(got).any()

def test_noalloc_prequantized_and_weight_only_need_no_scratch():
    fmt, M, N, K = "nvfp4", 12, 128, 512
    wc, ws, ws2 = weights(fmt, N, K, 5)
    ad, av = bf16_dev(synth.normal((M, K), seed=5, role=synth.ACT))
    wcd, wsd = to_dev(wc), to_dev(ws)
    a = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    b = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    F.fp4_gemm(fmt, "w4a16", M, N, K, ad, K, None, None, wcd, wsd, ws2, 0.0, a, N)
    F.fp4_gemm_noalloc(fmt, "w4a16", M, N, K, ad, K, None, None, wcd, wsd, ws2, 0.0, b, N)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_noalloc_refuses_calls_beyond_the_scratch():
    # NVFP4 M = 8192, K = 8192 needs 4 MiB more than the 32 MiB array: refused on the
    # host with FP4_ERR_WORKSPACE, nothing launched, the output left as it was
    M, N, K = 8192, 16, 8192
    assert F.fp4_gemm_workspace_size("nvfp4", "w4a4", M, K, 1) > (32 << 20)
    ad = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    wcd = torch.zeros((N, K // 2), dtype=torch.uint8, device=DEV)
    wsd = torch.full((N, K // 16), 0x38, dtype=torch.uint8, device=DEV)
    out = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=DEV)
    st = F.fp4_gemm_noalloc("nvfp4", "w4a4", M, N, K, ad, K, None, None, wcd, wsd, 1.0, 1.0,
                            out, N, check=False)
    assert st == F.FP4_ERR_WORKSPACE, F.status_str(st)
    torch.cuda.synchronize()
    assert (out == 7.0).all()
