"""GPU parity of fp4_gemm against the oracle (dequantize, QDQ, matmul in float64).

Definition: "vLLM per-format kernel capability matrix derived from source", THE
EMULATION COLUMN; alpha = weight_scale_2 * input_scale ("GLM-5.3-Flash on vLLM, on
GB10"); W4A16 = bf16 activations x dequantized weights ("vLLM on the DGX Spark, the
Hard Way: Seven Months of GB10 Field Notes", native-FP4 conditions).
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


def problem(fmt, M, N, K, seed, outliers=False):
    wc, ws, ws2 = weights(fmt, N, K, seed)
    a = synth.normal((M, K), seed=seed, role=synth.ACT, index=M)
    if outliers:
        a = synth.with_outliers(a, seed=seed)
    ad, av = bf16_dev(a)
    s = float(np.float32(np.abs(av).max()) / np.float32(2688.0)) if fmt == "nvfp4" else 1.0
    return wc, ws, ws2, ad, av, s


def run_and_check(fmt, mode, M, N, K, seed=0, out_dtype=torch.bfloat16, prequant=False,
                  outliers=False, rows=None):
    wc, ws, ws2, ad, av, s = problem(fmt, M, N, K, seed, outliers)
    wcd, wsd = to_dev(wc), to_dev(ws)
    if mode == "w4a16":
        out, st = T.gemm(fmt, mode, wcd, wsd, a_bf16=ad, weight_scale_2=ws2, out_dtype=out_dtype)
    elif prequant:
        ac, asc = T.quantize_act(fmt, ad, s)
        out, st = T.gemm(fmt, mode, wcd, wsd, a_codes=ac, a_scales=asc, weight_scale_2=ws2,
                         input_scale=s, out_dtype=out_dtype)
    else:
        out, st = T.gemm(fmt, mode, wcd, wsd, a_bf16=ad, weight_scale_2=ws2, input_scale=s,
                         out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert st == F.FP4_OK
    got = out.float().cpu().numpy().astype(np.float64)
    rows = np.arange(M) if rows is None else np.asarray(rows)
    w_hat = dequant(fmt, wc, ws)
    if mode == "w4a16":
        a_hat = av[rows].astype(np.float64)
        al = OG.alpha(fmt, OG.W4A16, ws2)
    else:
        ac_r, as_r = OQ.quantize_packed(fmt, av[rows], s)
        a_hat = dequant(fmt, ac_r, as_r)
        al = OG.alpha(fmt, OG.W4A4, ws2, s)
    ref = al * (a_hat @ w_hat.T)
    check_gemm(got[rows], ref, a_hat, w_hat, al, out_dtype == torch.bfloat16,
               what=f"{fmt} {mode} M={M} N={N} K={K}")
    if out_dtype == torch.float32:
        r = np.linalg.norm(got[rows] - ref) / max(np.linalg.norm(ref), 1e-300)
        assert r < 1e-5, f"fp32 accumulation error {r:.3g} is larger than expected"
    return out


SMALL = [(1, 16, 128), (5, 37, 256), (33, 50, 512), (17, 24, 384), (2, 8, 16), (3, 40, 96),
         (6, 20, 48), (40, 64, 1024)]


@pytest.mark.parametrize("shape", SMALL)
@pytest.mark.parametrize("fmt,mode", [("nvfp4", "w4a4"), ("mxfp4", "w4a4"), ("nvfp4", "w4a16"),
                                      ("mxfp4", "w4a16")])
def test_small_shapes(fmt, mode, shape):
    M, N, K = shape
    if K % OQ.GROUP[fmt]:
        # K not a multiple of the block size (MXFP4 K = 16, 48): refused on the host
        # with FP4_ERR_SHAPE before any launch, the canary output left as it was
        G = OQ.GROUP[fmt]
        wcd = torch.zeros((N, K // 2), dtype=torch.uint8, device=DEV)
        wsd = torch.full((N, (K + G - 1) // G), 127, dtype=torch.uint8, device=DEV)
        ad, _ = bf16_dev(synth.normal((M, K), seed=1, role=synth.ACT))
        out = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=DEV)
        ws = torch.empty(4096, dtype=torch.uint8, device=DEV)
        st = F.fp4_gemm(fmt, mode, M, N, K, ad, K, None, None, wcd, wsd, 1.0, 1.0, out, N,
                        F.FP4_OUT_BF16, 0, ws, 4096, check=False)
        assert st == F.FP4_ERR_SHAPE, F.status_str(st)
        ac = torch.zeros((M, K // 2), dtype=torch.uint8, device=DEV)
        asc = torch.full((M, (K + G - 1) // G), 127, dtype=torch.uint8, device=DEV)
        st = F.fp4_quantize_act(fmt, ad, M, K, K, 1.0, ac, asc, check=False)
        assert st == F.FP4_ERR_SHAPE, F.status_str(st)
        torch.cuda.synchronize()
        assert (out == 7.0).all()
        return
    run_and_check(fmt, mode, M, N, K, seed=sum(shape))
    run_and_check(fmt, mode, M, N, K, seed=sum(shape) + 1, out_dtype=torch.float32)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_prequantized_equals_fused(fmt):
    # fused activation quantization gives the same bits as quantize-then-GEMM
    M, N, K = 24, 48, 512
    a = run_and_check(fmt, "w4a4", M, N, K, seed=9, prequant=True)
    b = run_and_check(fmt, "w4a4", M, N, K, seed=9, prequant=False)
    assert torch.equal(a, b)


def test_nvfp4_w4a16_linear_small_config():
    # weights [256, 512] N(0, 0.02) -> NVFP4, activations [4, 512] bf16 N(0, 1), seed 0
    run_and_check("nvfp4", "w4a16", 4, 256, 512, seed=0)
    run_and_check("nvfp4", "w4a16", 4, 256, 512, seed=0, out_dtype=torch.float32)


@pytest.fixture(scope="module")
def decode_problem():
    fmt, N, K = "mxfp4", 14336, 4096
    wc, ws, _ = weights(fmt, N, K, seed=0)
    a = synth.with_outliers(synth.normal((32, K), seed=0, role=synth.ACT), seed=0)
    return wc, ws, a


@pytest.mark.parametrize("M", [1, 8, 32])
def test_mxfp4_w4a4_decode_full_size(decode_problem, M):
    # weights [14336, 4096] -> MXFP4; activations = the first M rows of [32, 4096]
    # N(0, 1) with 1% x20 outliers, quantized on the fly
    wc, ws, a = decode_problem
    ad, av = bf16_dev(a[:M])
    out, st = T.gemm("mxfp4", "w4a4", to_dev(wc), to_dev(ws), a_bf16=ad)
    torch.cuda.synchronize()
    assert st == F.FP4_OK
    ac, asc = OQ.quantize_packed("mxfp4", av, 1.0)
    a_hat, w_hat = dequant("mxfp4", ac, asc), dequant("mxfp4", wc, ws)
    ref = a_hat @ w_hat.T
    check_gemm(out.float().cpu().numpy().astype(np.float64), ref, a_hat, w_hat, 1.0, True,
               what=f"decode M={M}")


# more than 64 activation rows and K % 128 == 0: the LDS-tiled kernel (128-row
# tiles; 128 x 128 for NVFP4, 128 x 256 for MXFP4), with ragged rows and columns
TILED = [(65, 40, 128), (130, 256, 1024), (200, 300, 512), (257, 513, 384), (64 + 128 + 1, 17, 256)]


@pytest.mark.parametrize("shape", TILED)
@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_tiled_shapes(fmt, shape):
    M, N, K = shape
    run_and_check(fmt, "w4a4", M, N, K, seed=sum(shape))
    name = F.fp4_last_kernel()
    assert name.startswith("tile_" + fmt), name
    assert name == {"nvfp4": "tile_nvfp4_m128_n128", "mxfp4": "tile_mxfp4_m128"}[fmt], name
    run_and_check(fmt, "w4a4", M, N, K, seed=sum(shape) + 1, out_dtype=torch.float32,
                  prequant=True)


# Uniformly drawn bytes: every e2m1 code, and block scales over the whole finite range
# (NVFP4: e4m3 codes of either sign, subnormals included, only the NaN codes 0x7F /
# 0xFF left out; MXFP4: e8m0 2^-20 .. 2^20), through each kernel family -- resident
# (1 row), streaming (32 rows), LDS tile (more than 64 rows), generic (K not a
# multiple of 128) -- against the oracle's dequantization of the same bytes.
RAW = [(1, 272, 1024), (32, 200, 1024), (96, 384, 512), (20, 72, 96)]


@pytest.mark.parametrize("shape", RAW)
@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_raw_codes(fmt, shape):
    M, N, K = shape
    G = OQ.GROUP[fmt]
    rng = np.random.default_rng(sum(shape) + (fmt == "nvfp4"))

    def scales(rows):
        if fmt == "nvfp4":
            c = rng.integers(0, 256, (rows, K // G), dtype=np.uint8)
            c[(c & 0x7F) == 0x7F] ^= 1
            return c
        return rng.integers(107, 148, (rows, K // G), dtype=np.uint8)

    wc, ws = rng.integers(0, 256, (N, K // 2), dtype=np.uint8), scales(N)
    ac, asc = rng.integers(0, 256, (M, K // 2), dtype=np.uint8), scales(M)
    out, st = T.gemm(fmt, "w4a4", to_dev(wc), to_dev(ws), a_codes=to_dev(ac),
                     a_scales=to_dev(asc), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert st == F.FP4_OK
    a_hat, w_hat = dequant(fmt, ac, asc), dequant(fmt, wc, ws)
    check_gemm(out.cpu().numpy().astype(np.float64), a_hat @ w_hat.T, a_hat, w_hat, 1.0,
               False, what=f"raw {fmt} M={M} N={N} K={K} ({F.fp4_last_kernel()})")


# dense problems with at least 256 tiles of 256 x 256: the 4-wave 256 x 256 tile, with K
# of 1, 3, 5, 8 and 17 stages of 128 (fewer stages than its four stage buffers, and
# more), ragged rows and columns; the oracle checks the first and last 300 rows and
# 200 sampled ones
TILED_256 = [(2300, 7324, 128), (2049, 7324, 384), (4096, 4096, 1024), (4096, 4096, 640),
             (4352, 4096, 2176)]


@pytest.mark.parametrize("shape", TILED_256)
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_tiled_256_shapes(fmt, shape):
    M, N, K = shape
    rng = np.random.default_rng(sum(shape))
    rows = np.unique(np.concatenate([np.arange(300), np.arange(M - 300, M),
                                     rng.choice(M, 200, replace=False)]))
    run_and_check(fmt, "w4a4", M, N, K, seed=sum(shape), rows=rows)
    assert F.fp4_last_kernel() == f"big_{fmt}_256"
    run_and_check(fmt, "w4a4", M, N, K, seed=sum(shape) + 1, out_dtype=torch.float32,
                  prequant=True, rows=rows)


@pytest.mark.parametrize("shape", [(2300, 7324, 384), (4352, 4096, 2176)])
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_big_tile_scale_paths_bitwise(fmt, shape):
    # the 256 x 256 tile reads its block scales either from the stage-ordered copy that
    # fp4_gemm writes into a large enough workspace, or row by row: same bits
    M, N, K = shape
    wc, ws, ws2, ad, av, s = problem(fmt, M, N, K, seed=M)
    wcd, wsd = to_dev(wc), to_dev(ws)
    ac, asc = T.quantize_act(fmt, ad, s)
    need = F.fp4_gemm_workspace_size_mnk(fmt, "w4a4", M, N, K, 0)
    assert need > 0
    outs = []
    for wsb in (torch.empty(need, dtype=torch.uint8, device=DEV),
                torch.empty(16, dtype=torch.uint8, device=DEV)):
        out, st = T.gemm(fmt, "w4a4", wcd, wsd, a_codes=ac, a_scales=asc, weight_scale_2=ws2,
                         input_scale=s, out_dtype=torch.float32, workspace=wsb)
        assert st == F.FP4_OK and F.fp4_last_kernel() == f"big_{fmt}_256"
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))
    # the fused path with its own workspace gives the same bits as well
    out, st = T.gemm(fmt, "w4a4", wcd, wsd, a_bf16=ad, weight_scale_2=ws2, input_scale=s,
                     out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert st == F.FP4_OK and torch.equal(out.view(torch.int32), outs[0].view(torch.int32))



@pytest.mark.parametrize("pad", [8, 3])
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_big_tile_strided_output(fmt, pad):
    # the 256 x 256 tile into a bf16 output with row stride N + pad: 16-byte stores when
    # the stride keeps rows aligned (pad 8; N % 8 == 4 leaves a partial piece at the
    # end of each row), element stores otherwise (pad 3); the columns past N keep their
    # canary and the first N equal the contiguous output bit for bit
    M, N, K = 2300, 7324, 384
    wc, ws, ws2, ad, av, s = problem(fmt, M, N, K, seed=N + pad)
    wcd, wsd = to_dev(wc), to_dev(ws)
    ac, asc = T.quantize_act(fmt, ad, s)
    ref, st = T.gemm(fmt, "w4a4", wcd, wsd, a_codes=ac, a_scales=asc, weight_scale_2=ws2,
                     input_scale=s, out_dtype=torch.bfloat16)
    assert st == F.FP4_OK
    ldo = N + pad
    canary = torch.tensor(-7.25, dtype=torch.bfloat16)
    out = torch.full((M, ldo), float(canary), dtype=torch.bfloat16, device=DEV)
    need = F.fp4_gemm_workspace_size_mnk(fmt, "w4a4", M, N, K, 0)
    wsb = torch.empty(need, dtype=torch.uint8, device=DEV)
    st = F.fp4_gemm(fmt, "w4a4", M, N, K, None, K, ac, asc, wcd, wsd, ws2, s, out, ldo,
                    F.FP4_OUT_BF16, 0, wsb, need)
    assert st == F.FP4_OK and F.fp4_last_kernel() == f"big_{fmt}_256"
    torch.cuda.synchronize()
    assert torch.equal(out[:, :N].view(torch.int16), ref.view(torch.int16))
    assert bool((out[:, N:] == canary).all())

# at most 64 activation rows: the resident-activation kernel whenever the scale rows
# are whole 16-byte pieces and the activations fit in LDS (ring of 8, 16 or 32 K
# steps; K = 6144 refills the ring once), otherwise the streaming kernel.  The 4 waves
# split K 1, 2 or 4 ways depending on M, N and K: (3, 40, 1024) one way, (16, 100,
# 2048) two ways, (1, 300, 6144) four ways with 12 steps a wave, and (5, 72, 4352) and
# (4, 72, 4352) (NVFP4) two even and four uneven ranges (8 and 9 steps)
RESIDENT = [(1, 300, 6144), (16, 100, 2048), (17, 64, 768), (32, 520, 4096), (50, 70, 1536),
            (64, 33, 512), (3, 40, 1024), (5, 72, 4352), (4, 72, 4352)]


def resident_ksplit(M, N, K):
    ns, ks, kmax = K // 128, 1, 4 if M <= 4 else 2
    while ks < kmax and ns // (2 * ks) >= 8 and -(-N // (16 * (4 // ks))) < 512:
        ks *= 2
    return ks


def resident_expected(fmt, M, N, K):
    G = 16 if fmt == "nvfp4" else 32
    if M > 16:
        return False    # two-tile blocks take the streaming kernel
    mt, ks = 1, resident_ksplit(M, N, K)
    kb = lambda b: (b + 1023) // 1024 * 1024
    arows = 4 if ks == 4 else 16 * mt
    lds = (arows * (kb(K // 2) + 16) + kb(arows * (K // G)) + kb(64 // ks * (K // G))
           + (ks - 1) * (4 // ks) * mt * 1024)
    return K % 128 == 0 and (K // G) % 16 == 0 and lds <= 160 * 1024


@pytest.mark.parametrize("shape", RESIDENT)
@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_resident_shapes(fmt, shape):
    M, N, K = shape
    if K % OQ.GROUP[fmt]:
        pytest.skip("K not a multiple of the block size")
    run_and_check(fmt, "w4a4", M, N, K, seed=sum(shape) + 7)
    name = F.fp4_last_kernel()
    if resident_expected(fmt, M, N, K):
        assert name == f"resident_{fmt}_m16", name
    else:
        assert name.startswith(("stream_", "rowblock_")), name
    run_and_check(fmt, "w4a4", M, N, K, seed=sum(shape) + 8, out_dtype=torch.float32,
                  prequant=True)


# 17..64 rows: the streaming kernel over many weight tiles with a ragged last one, one
# 32-row block and two
STREAM = [(20, 9990, 512), (40, 5000, 256)]


@pytest.mark.parametrize("shape", STREAM)
@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_stream_wide(fmt, shape):
    M, N, K = shape
    run_and_check(fmt, "w4a4", M, N, K, seed=sum(shape) + 3)
    assert F.fp4_last_kernel() == f"stream_{fmt}_m32", F.fp4_last_kernel()
    run_and_check(fmt, "w4a4", M, N, K, seed=sum(shape) + 4, out_dtype=torch.float32,
                  prequant=True)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_tiled_strided_output_canaries(fmt):
    # output rows with a stride that is not a multiple of 4 take the scalar stores;
    # the padding columns and the row after the output stay untouched
    M, N, K = 150, 70, 256
    wc, ws, ws2, ad, av, s = problem(fmt, M, N, K, 21)
    wcd, wsd = to_dev(wc), to_dev(ws)
    ref, _ = T.gemm(fmt, "w4a4", wcd, wsd, a_bf16=ad, weight_scale_2=ws2, input_scale=s)
    big = torch.full((M + 1, N + 3), -7.0, dtype=torch.bfloat16, device=DEV)
    out = big[:M, :N]
    _, st = T.gemm(fmt, "w4a4", wcd, wsd, a_bf16=ad, weight_scale_2=ws2, input_scale=s, out=out)
    torch.cuda.synchronize()
    assert st == F.FP4_OK
    assert F.fp4_last_kernel().startswith("tile_")
    assert torch.equal(out, ref)
    assert (big[M] == -7.0).all() and (big[:, N:] == -7.0).all()


def test_mxfp4_w4a4_prefill_full_size_sampled_rows():
    # MXFP4 at the prefill shape; 64 sampled rows incl. first and last
    fmt, M, N, K = "mxfp4", 8192, 4096, 4096
    rng = np.random.default_rng(1)
    rows = np.concatenate([[0, M - 1], rng.choice(np.arange(1, M - 1), 62, replace=False)])
    run_and_check(fmt, "w4a4", M, N, K, seed=1, rows=np.sort(rows))


def test_nvfp4_w4a4_prefill_full_size_sampled_rows():
    # [8192, 4096] x [4096, 4096]^T, fused quantization, bf16 out; the oracle checks
    # 96 sampled rows (rows are independent) including the first and last
    fmt, M, N, K = "nvfp4", 8192, 4096, 4096
    rng = np.random.default_rng(0)
    rows = np.concatenate([[0, M - 1], rng.choice(np.arange(1, M - 1), 94, replace=False)])
    run_and_check(fmt, "w4a4", M, N, K, seed=0, rows=np.sort(rows))


def test_w4a4_is_not_weight_only():
    # the W4A4 result matches the W4A4 oracle and not the W4A16 one
    fmt, M, N, K = "nvfp4", 8, 64, 512
    wc, ws, ws2, ad, av, s = problem(fmt, M, N, K, 11)
    out, _ = T.gemm(fmt, "w4a4", to_dev(wc), to_dev(ws), a_bf16=ad, weight_scale_2=ws2,
                    input_scale=s, out_dtype=torch.float32)
    got = out.cpu().numpy().astype(np.float64)
    ref44 = OG.gemm_fused(fmt, av, wc, ws, ws2, s)
    ref416 = OG.gemm_w4a16(fmt, av, wc, ws, ws2)
    d44 = np.linalg.norm(got - ref44) / np.linalg.norm(ref44)
    d416 = np.linalg.norm(got - ref416) / np.linalg.norm(ref416)
    assert d44 < 1e-5 and d416 > 1e-2


def test_zero_input_scale_refused_or_explicit_fallback():
    fmt, M, N, K = "nvfp4", 4, 32, 256
    wc, ws, ws2, ad, av, _ = problem(fmt, M, N, K, 12)
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    st = F.fp4_gemm(F.FP4_NVFP4, F.FP4_W4A4, M, N, K, ad, K, None, None, to_dev(wc),
                    to_dev(ws), ws2, 0.0, out, N, F.FP4_OUT_F32, 0, None, 0, check=False)
    torch.cuda.synchronize()
    assert st == F.FP4_ERR_INPUT_SCALE
    assert torch.isnan(out).all()                      # nothing was written
    wcd, wsd = to_dev(wc), to_dev(ws)
    st = F.fp4_gemm(F.FP4_NVFP4, F.FP4_W4A4, M, N, K, ad, K, None, None, wcd, wsd, ws2, 0.0,
                    out, N, F.FP4_OUT_F32, F.FP4_FLAG_ALLOW_W4A16_FALLBACK, None, 0, check=False)
    torch.cuda.synchronize()
    assert st == F.FP4_OK_FELL_BACK_W4A16
    ref = OG.gemm_w4a16(fmt, av, wc, ws, ws2)
    assert np.linalg.norm(out.cpu().numpy() - ref) / np.linalg.norm(ref) < 1e-5


def test_deterministic_canaries_and_two_streams():
    fmt, M, N, K = "mxfp4", 40, 96, 1024
    wc, ws, _, ad, av, _ = problem(fmt, M, N, K, 13)
    wcd, wsd = to_dev(wc), to_dev(ws)
    big = torch.full((M + 1, N + 8), float("nan"), dtype=torch.float32, device=DEV)
    out = big[:M, :N]
    T.gemm(fmt, "w4a4", wcd, wsd, a_bf16=ad, out=out)
    torch.cuda.synchronize()
    first = out.clone()
    assert torch.isnan(big[M]).all() and torch.isnan(big[:, N:]).all()
    # the same problem on two streams at once, next to a different one, stays bitwise equal
    wc2, ws2_, _, ad2, _, _ = problem("nvfp4", 64, 128, 512, 14)
    w2d, s2d = to_dev(wc2), to_dev(ws2_)
    ref2, _ = T.gemm("nvfp4", "w4a16", w2d, s2d, a_bf16=ad2)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for i in range(4):
        with torch.cuda.stream(s1 if i % 2 == 0 else s2):
            o1, _ = T.gemm(fmt, "w4a4", wcd, wsd, a_bf16=ad, out_dtype=torch.float32)
            o2, _ = T.gemm("nvfp4", "w4a16", w2d, s2d, a_bf16=ad2)
            outs.append((o1, o2))
    torch.cuda.synchronize()
    for o1, o2 in outs:
        assert torch.equal(o1, first)
        assert torch.equal(o2, ref2)


# W4A16 for many rows (bf16 activations x FP4 weights decoded exactly to bf16): the
# LDS-tiled bf16-MFMA kernel above 64 rows with K a multiple of 128 ("vLLM on the DGX
# Spark, the Hard Way: Seven Months of GB10 Field Notes": weight-only checkpoints are
# what costs prefill).  Ragged rows and columns, one to several stages of K.
W4A16_TILED = [(65, 256, 128), (130, 300, 512), (257, 520, 1024), (96, 40, 384), (200, 256, 4096)]


@pytest.mark.parametrize("shape", W4A16_TILED)
@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_w4a16_tiled_shapes(fmt, shape):
    M, N, K = shape
    run_and_check(fmt, "w4a16", M, N, K, seed=sum(shape))
    assert F.fp4_last_kernel() == "w4a16_tile_" + fmt, F.fp4_last_kernel()
    run_and_check(fmt, "w4a16", M, N, K, seed=sum(shape) + 1, out_dtype=torch.float32)
    # below the tiled kernel's size and for K % 128 != 0 the row-block kernel runs
    run_and_check(fmt, "w4a16", 64, N, K, seed=1)
    assert F.fp4_last_kernel().startswith("rowblock_"), F.fp4_last_kernel()


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_w4a16_tiled_strided_activations_and_output(fmt):
    M, N, K = 150, 264, 640
    wc, ws, ws2 = weights(fmt, N, K, seed=5)
    a = synth.normal((M, K + 24), seed=5, role=synth.ACT)
    ad, av = bf16_dev(a)
    big = torch.full((M, N + 8), -3.0, dtype=torch.float32, device=DEV)
    out, st = T.gemm(fmt, "w4a16", to_dev(wc), to_dev(ws), a_bf16=ad[:, :K], weight_scale_2=ws2,
                     out=big[:, :N])
    torch.cuda.synchronize()
    assert st == F.FP4_OK and F.fp4_last_kernel() == "w4a16_tile_" + fmt
    b = big.cpu().numpy()
    assert (b[:, N:] == -3.0).all()
    a_hat = av[:, :K].astype(np.float64)
    w_hat = dequant(fmt, wc, ws)
    al = OG.alpha(fmt, OG.W4A16, ws2)
    check_gemm(b[:, :N].astype(np.float64), al * (a_hat @ w_hat.T), a_hat, w_hat, al, False,
               what=f"{fmt} w4a16 strided")


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_w4a16_prefill_full_size_sampled_rows(fmt):
    # [8192, 4096] bf16 x [4096, 4096] FP4 weights, bf16 out; 64 sampled rows incl. the
    # first and the last
    M, N, K = 8192, 4096, 4096
    rng = np.random.default_rng(7)
    rows = np.concatenate([[0, M - 1], rng.choice(np.arange(1, M - 1), 62, replace=False)])
    run_and_check(fmt, "w4a16", M, N, K, seed=7, rows=np.sort(rows))
    assert F.fp4_last_kernel() == "w4a16_tile_" + fmt
