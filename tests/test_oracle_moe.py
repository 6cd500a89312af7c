"""Pins for the oracle's router, dispatch bookkeeping and MoE chain (CPU only).

Stages: "vLLM on the NVIDIA DGX Spark (GB10 / sm_121): A Complete Technical Guide",
§7.1 and §4.3.  Refusal rule: "GLM-5.3-Flash on vLLM, on GB10".
"""
import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import gemm as Gm
from oracle import moe as Mo
from oracle import quant as Q
import synth


def test_topk_invariants():
    logits = synth.normal((50, 32), seed=1, role=synth.LOGITS)
    ids, w = Mo.topk_softmax(logits, 8)
    for t in range(50):
        assert len(set(ids[t])) == 8
        order = np.argsort(-logits[t].astype(np.float64), kind="stable")[:8]
        assert list(ids[t]) == list(order)
    assert np.allclose(w.sum(1), 1.0, atol=1e-15)
    p = torch.softmax(torch.from_numpy(logits).double(), dim=1).numpy()
    pk = np.take_along_axis(p, ids.astype(np.int64), 1)
    assert np.allclose(w, pk / pk.sum(1, keepdims=True), rtol=1e-13)
    _, w_raw = Mo.topk_softmax(logits, 8, renormalize=False)
    assert np.allclose(w_raw, pk, rtol=1e-13)


def test_topk_ties_go_to_lower_index():
    logits = np.array([[1.0, 3.0, 3.0, 0.0, 3.0]], np.float32)
    ids, w = Mo.topk_softmax(logits, 2)
    assert list(ids[0]) == [1, 2]
    assert w[0, 0] == w[0, 1] == 0.5


def test_permute_is_stable_counting_sort():
    rng = np.random.default_rng(20)
    T, k, E = 37, 4, 9
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    off, rows, inv = Mo.permute(ids, E)
    flat = ids.reshape(-1)
    assert off[0] == 0 and off[-1] == T * k
    assert np.array_equal(np.diff(off), np.bincount(flat, minlength=E))
    for e in range(E):
        seg = rows[off[e]:off[e + 1]]
        assert (flat[seg] == e).all() and (np.diff(seg) > 0).all()
    assert np.array_equal(rows[inv], np.arange(T * k))


def _expert(rng, fmt, H, I, a13=1.0, a2=1.0):
    w13 = (rng.standard_normal((2 * I, H)) * 0.05).astype(np.float32)
    w2 = (rng.standard_normal((H, I)) * 0.05).astype(np.float32)
    c13, s13, ws13 = Q.quantize_weight(fmt, w13)
    c2, s2, ws2 = Q.quantize_weight(fmt, w2)
    return Mo.Expert(c13, s13, c2, s2, ws13, ws2, a13, a2)


def _lit_dequant(fmt, packed, sc):
    lit = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    codes = F.unpack_nibbles(packed).astype(np.int64)
    v = np.array(lit)[codes & 7] * np.where(codes & 8, -1.0, 1.0)
    dt = torch.float8_e4m3fn if fmt == Q.NVFP4 else torch.float8_e8m0fnu
    s = torch.from_numpy(sc).view(dt).double().numpy()
    G = Q.GROUP[fmt]
    return v * np.repeat(s, G, axis=1)


@pytest.mark.parametrize("fmt", [Q.NVFP4, Q.MXFP4])
def test_single_expert_w4a16_written_out(fmt):
    # E = 1, k = 1, weight 1: the layer is gate/up -> SiLU(gate)*up -> bf16 -> down,
    # computed here with torch in float64 from literal decodes
    rng = np.random.default_rng(21)
    T, H, I = 5, 64, 32
    ex = _expert(rng, fmt, H, I)
    _, x = synth.bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1))
    got = Mo.moe(fmt, Gm.W4A16, x, ids, w, [ex])
    W13 = torch.from_numpy(_lit_dequant(fmt, ex.w13_codes, ex.w13_scales) * ex.w13_scale_2)
    W2 = torch.from_numpy(_lit_dequant(fmt, ex.w2_codes, ex.w2_scales) * ex.w2_scale_2)
    gu = torch.from_numpy(x).double() @ W13.T
    h = torch.nn.functional.silu(gu[:, :I]) * gu[:, I:]
    h = h.float().to(torch.bfloat16).double()
    y = h @ W2.T
    assert np.allclose(got, y.numpy(), rtol=1e-12, atol=1e-12)


def test_identical_experts_reduce_to_one():
    rng = np.random.default_rng(22)
    T, H, I, E, k = 6, 64, 32, 4, 3
    ex = _expert(rng, Q.MXFP4, H, I)
    x = rng.standard_normal((T, H)).astype(np.float32)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = Mo.topk_softmax(logits, k)
    got = Mo.moe(Q.MXFP4, Gm.W4A4, x, ids, w, [ex] * E)
    one = Mo.moe(Q.MXFP4, Gm.W4A4, x, np.zeros((T, 1), np.int32), np.ones((T, 1)), [ex])
    assert np.allclose(got, one, rtol=1e-12, atol=1e-12)


def test_expert_relabeling_invariance():
    rng = np.random.default_rng(23)
    T, H, I, E, k = 7, 64, 32, 5, 2
    exps = [_expert(rng, Q.NVFP4, H, I, 0.01, 0.002) for _ in range(E)]
    x = rng.standard_normal((T, H)).astype(np.float32)
    ids, w = Mo.topk_softmax(rng.standard_normal((T, E)).astype(np.float32), k)
    perm = rng.permutation(E)
    inv = np.argsort(perm)
    a = Mo.moe(Q.NVFP4, Gm.W4A4, x, ids, w, exps)
    b = Mo.moe(Q.NVFP4, Gm.W4A4, x, inv[ids].astype(np.int32), w, [exps[p] for p in perm])
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def test_zero_activation_scale_refused_and_buggy_zeroes_experts():
    rng = np.random.default_rng(24)
    T, H, I, E, k = 4, 64, 32, 3, 2
    exps = [_expert(rng, Q.NVFP4, H, I, 0.01, 0.002) for _ in range(E)]
    shared = _expert(rng, Q.NVFP4, H, I, 0.01, 0.002)
    exps[1].a13_scale = 0.0
    x = rng.standard_normal((T, H)).astype(np.float32)
    ids = np.array([[1, 0], [1, 2], [0, 2], [1, 0]], np.int32)
    w = np.full((T, k), 0.5)
    with pytest.raises(Q.InputScaleError):
        Mo.moe(Q.NVFP4, Gm.W4A4, x, ids, w, exps, shared)
    for e in exps:
        e.a13_scale = 0.0
    buggy = Mo.moe(Q.NVFP4, Gm.W4A4, x, ids, w, exps, shared, buggy=True)
    only_shared = Mo.expert_forward(Q.NVFP4, Gm.W4A4, x, shared)
    assert np.array_equal(buggy, only_shared)          # the routed experts contribute zero


def test_token_subset_matches_full():
    rng = np.random.default_rng(25)
    T, H, I, E, k = 9, 64, 32, 4, 2
    exps = [_expert(rng, Q.MXFP4, H, I) for _ in range(E)]
    x = rng.standard_normal((T, H)).astype(np.float32)
    ids, w = Mo.topk_softmax(rng.standard_normal((T, E)).astype(np.float32), k)
    full = Mo.moe(Q.MXFP4, Gm.W4A4, x, ids, w, exps)
    sub = Mo.moe(Q.MXFP4, Gm.W4A4, x, ids, w, exps, tokens=[7, 2])
    assert np.allclose(sub, full[[7, 2]], rtol=1e-13, atol=1e-13)
