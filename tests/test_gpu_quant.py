"""GPU parity of fp4_quantize_act / fp4_quantize_weight against the oracle:
codes and scales must be bit-exact.

Formats: "vLLM on the NVIDIA DGX Spark (GB10 / sm_121): A Complete Technical Guide",
§6.1 (NVFP4) and §6.4 (MXFP4); in-kernel activation quantization, §4.3.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp4_quantize_amd as F
from block_scaled_fp4_quantize_amd import tensors as T
import synth
from oracle import quant as OQ
from tests.gpu_util import DEV, bf16_dev, to_dev

pytestmark = pytest.mark.gpu


def edge_values(n, seed):
    """Values that sit on rounding decisions: e2m1 midpoints times powers of two,
    signed zeros, bf16 subnormals, huge values, plus noise."""
    rng = np.random.default_rng(seed)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.5, 1.0, 4.0])
    base = rng.choice(mids, n) * 2.0 ** rng.integers(-8, 8, n) * rng.choice([-1, 1], n)
    v = base.astype(np.float32)
    sel = rng.random(n)
    v[sel < 0.05] = 0.0
    v[(sel >= 0.05) & (sel < 0.08)] = -0.0
    sub = (sel >= 0.08) & (sel < 0.1)
    v[sub] = (rng.integers(1, 127, sub.sum()) * 2.0 ** -133).astype(np.float32)   # bf16 subnormals
    big = (sel >= 0.1) & (sel < 0.11)
    v[big] = np.float32(3.0e38)
    noise = sel >= 0.6
    v[noise] = rng.standard_normal(noise.sum()).astype(np.float32)
    return v


def run_quant(fmt, x_f32, s, ldx_pad=0):
    M, K = x_f32.shape
    xd, xv = bf16_dev(np.pad(x_f32, ((0, 0), (0, ldx_pad))))
    xd = xd[:, :K] if ldx_pad else xd
    codes, scales = T.quantize_act(fmt, xd, s)
    torch.cuda.synchronize()
    ref_c, ref_s = OQ.quantize_packed(fmt, xv[:, :K], s)
    return codes.cpu().numpy(), scales.cpu().numpy(), ref_c, ref_s


SHAPES = [(1, 32), (3, 64), (5, 96), (37, 512), (64, 4096), (2, 6144)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("fmt,s", [("nvfp4", 1.0), ("nvfp4", 0.01), ("nvfp4", 3.7e-4),
                                   ("mxfp4", 1.0)])
def test_act_quant_bit_exact(fmt, s, shape):
    M, K = shape
    x = synth.normal((M, K), seed=1, role=synth.ACT, index=M * K)
    x = synth.with_outliers(x, 0.01, 20.0, seed=1, index=M)
    c, sc, rc, rs = run_quant(fmt, x, s)
    assert np.array_equal(sc, rs), f"scale codes differ at {np.argwhere(sc != rs)[:5]}"
    assert np.array_equal(c, rc), f"codes differ at {np.argwhere(c != rc)[:5]}"


@pytest.mark.parametrize("fmt,s", [("nvfp4", 1.0), ("nvfp4", 1.0 / 64), ("mxfp4", 1.0)])
def test_act_quant_edge_values(fmt, s):
    x = edge_values(64 * 256, seed=3).reshape(64, 256)
    c, sc, rc, rs = run_quant(fmt, x, s)
    assert np.array_equal(sc, rs)
    assert np.array_equal(c, rc)


def test_act_quant_ragged_k_and_stride():
    # K = 16 (one NVFP4 block), K = 48 (three), and a row stride larger than K
    for fmt, K in (("nvfp4", 16), ("nvfp4", 48), ("mxfp4", 32), ("mxfp4", 96)):
        x = synth.normal((7, K), seed=4, role=synth.ACT, index=K)
        c, sc, rc, rs = run_quant(fmt, x, 0.05 if fmt == "nvfp4" else 1.0, ldx_pad=8)
        assert np.array_equal(sc, rs) and np.array_equal(c, rc), (fmt, K)


def test_act_quant_golden_blocks():
    from tests.test_oracle_quant import load_golden
    for name in ("nvfp4_block_s1.txt", "nvfp4_block_s001.txt", "mxfp4_block.txt"):
        fmt, s, x, codes, sc, _ = load_golden(name)
        xd, _ = bf16_dev(x.reshape(1, -1))
        gc, gs = T.quantize_act(fmt, xd, s)
        got = np.zeros(x.size, np.uint8)
        b = gc.cpu().numpy()[0]
        got[0::2], got[1::2] = b & 0xF, b >> 4
        assert list(got) == list(codes), name
        assert list(gs.cpu().numpy()[0]) == list(sc), name


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_weight_quant_fp32_bit_exact(fmt):
    w = synth.normal((96, 512), 0.02, seed=5, role=synth.WEIGHT)
    ref_c, ref_s, ws2 = OQ.quantize_weight(fmt, w)
    c, s = T.quantize_weight(fmt, to_dev(w), ws2)
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy(), ref_s)
    assert np.array_equal(c.cpu().numpy(), ref_c)


def test_full_size_activations():
    # decode activations [32, 4096] with 1% x20 outliers (MXFP4) and prefill
    # activations [8192, 4096] under input_scale = amax / 2688 (NVFP4)
    x = synth.with_outliers(synth.normal((32, 4096), seed=0, role=synth.ACT), seed=0)
    c, sc, rc, rs = run_quant("mxfp4", x, 1.0)
    assert np.array_equal(sc, rs) and np.array_equal(c, rc)
    a = synth.normal((8192, 4096), seed=0, role=synth.ACT, index=3)
    _, av = synth.bf16_bits(a)
    s = float(np.float32(np.abs(av).max()) / np.float32(2688.0))
    c, sc, rc, rs = run_quant("nvfp4", a, s)
    assert np.array_equal(sc, rs) and np.array_equal(c, rc)


def test_quant_is_deterministic_and_leaves_canaries():
    x = synth.normal((33, 512), seed=6, role=synth.ACT)
    xd, _ = bf16_dev(x)
    codes = torch.full((34, 256), 0xA5, dtype=torch.uint8, device=DEV)
    scales = torch.full((34, 32), 0x5A, dtype=torch.uint8, device=DEV)
    F.fp4_quantize_act(F.FP4_NVFP4, xd, 33, 512, 512, 0.02, codes, scales)
    first = codes.clone(), scales.clone()
    for _ in range(3):
        F.fp4_quantize_act(F.FP4_NVFP4, xd, 33, 512, 512, 0.02, codes, scales)
    torch.cuda.synchronize()
    assert torch.equal(first[0], codes) and torch.equal(first[1], scales)
    assert (codes[33] == 0xA5).all() and (scales[33] == 0x5A).all()
