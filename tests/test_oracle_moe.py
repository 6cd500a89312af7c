"""Pins for the oracle's router, dispatch bookkeeping and MoE chain (CPU only).

Stages: "vLLM on the NVIDIA DGX Spark (GB10 / sm_121): A Complete Technical Guide",
§7.1 and §4.3.  Refusal rule: "GLM-5.3-Flash on vLLM, on GB10".
"""
import os

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


# ----------------------------------------------------------------------------------
# W4A4 expert chain written out independently of oracle.quant / oracle.gemm: block
# scales through torch's float8 casts and decoders, elements by a brute-force nearest
# search over the literal e2m1 magnitudes, products with torch in float64.
# ----------------------------------------------------------------------------------

_E2M1_LIT = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _lit_e2m1(y, sign_src):
    """e2m1 codes of float64 magnitudes |y|: nearest literal value, a tie to the even
    code (both candidates of a tie are adjacent, one even and one odd); sign of sign_src."""
    d = np.abs(np.abs(y)[..., None] - _E2M1_LIT)
    cand = d == d.min(-1, keepdims=True)
    even = cand & (np.arange(8) % 2 == 0)
    code = np.where(even.any(-1), np.argmax(even, -1), np.argmax(cand, -1))
    return (code | (np.signbit(sign_src).astype(np.int64) << 3)).astype(np.int64)


def _lit_value(code):
    return _E2M1_LIT[code & 7] * np.where(code & 8, -1.0, 1.0)


def _lit_qdq_nvfp4(x, s):
    """Dequantized NVFP4 values of fp32 rows x under the activation scale s:
    g = 1/s, per 16-block sf = (amax g)/6 in fp32, scale = e4m3(sf) via torch's cast,
    r = g/scale, element = nearest e2m1 of fp32(x r)."""
    xt = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    R, K = xt.shape
    g = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(s, dtype=torch.float32)
    xb = xt.view(R, K // 16, 16)
    amax = xb.abs().amax(-1)
    sf = (amax * g) / torch.tensor(6.0, dtype=torch.float32)
    assert float(sf.max()) < 464.0             # torch's cast returns NaN from 464 on
    sd = sf.to(torch.float8_e4m3fn).to(torch.float32)
    r = torch.where(sd > 0, g / torch.where(sd > 0, sd, torch.ones_like(sd)), torch.zeros_like(sd))
    y = (xb * r[..., None]).numpy().astype(np.float64)
    code = _lit_e2m1(y, xb.numpy())
    return (_lit_value(code) * sd.numpy().astype(np.float64)[..., None]).reshape(R, K)


def _lit_qdq_mxfp4(x):
    """Dequantized MXFP4 values: per 32-block E = floor(log2 amax) - 2 (from frexp),
    element = nearest e2m1 of x 2^-E, value = element 2^E."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    R, K = x.shape
    xb = x.reshape(R, K // 32, 32)
    amax = np.abs(xb).max(-1)
    _, ex = np.frexp(amax)                     # amax = m 2^ex, m in [0.5, 1)
    E = np.where(amax > 0, np.clip(ex - 1 - 2, -127, 127), -127)
    code = _lit_e2m1(xb * np.ldexp(1.0, -E)[..., None], xb)
    return (_lit_value(code) * np.ldexp(1.0, E)[..., None]).reshape(R, K)


def _chain_written_out(fmt, x, ex):
    """One W4A4 expert: x_hat (under a13) -> gate/up * alpha13 -> SiLU(gate)*up in
    float64 -> rounded to fp32 -> h_hat (under a2) -> down * alpha2."""
    nv = fmt == Q.NVFP4
    qdq = (lambda v, s: _lit_qdq_nvfp4(v, s)) if nv else (lambda v, s: _lit_qdq_mxfp4(v))
    W13 = torch.from_numpy(_lit_dequant(fmt, ex.w13_codes, ex.w13_scales))
    W2 = torch.from_numpy(_lit_dequant(fmt, ex.w2_codes, ex.w2_scales))
    al13 = ex.w13_scale_2 * ex.a13_scale if nv else 1.0
    al2 = ex.w2_scale_2 * ex.a2_scale if nv else 1.0
    I = W2.shape[1]
    gu = al13 * (torch.from_numpy(qdq(x, ex.a13_scale)) @ W13.T)
    h = torch.nn.functional.silu(gu[:, :I]) * gu[:, I:]
    h32 = h.numpy().astype(np.float32)
    return al2 * (torch.from_numpy(qdq(h32, ex.a2_scale)) @ W2.T).numpy()


@pytest.mark.parametrize("fmt", [Q.NVFP4, Q.MXFP4])
def test_w4a4_layer_written_out(fmt):
    # three routed experts (top-2) and a shared one; NVFP4 experts each carry their
    # own a13 != a2, at ratios that are not powers of two (a power-of-two change of
    # an activation scale leaves the output unchanged, so it would pin nothing)
    rng = np.random.default_rng(26)
    T, H, I, E, k = 6, 64, 32, 3, 2
    _, x = synth.bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    exps = [_expert(rng, fmt, H, I) for _ in range(E)]
    shared = _expert(rng, fmt, H, I)
    if fmt == Q.NVFP4:
        base13 = float(np.abs(x).max()) / 2688.0
        for e, ex in enumerate(exps + [shared]):
            ex.a13_scale = float(np.float32(base13 * (1.0 + 0.3 * e)))
            h = Mo.expert_h(fmt, Gm.W4A4, x, ex)
            ex.a2_scale = float(np.float32(float(np.abs(h).max()) / 2688.0 * (1.7 + 0.2 * e)))
            assert ex.a13_scale != ex.a2_scale
    ids = np.array([[0, 1], [2, 0], [1, 2], [0, 2], [1, 0], [2, 1]], np.int32)
    w = np.array([[0.7, 0.3], [0.6, 0.4], [0.55, 0.45], [0.8, 0.2], [0.5, 0.5], [0.9, 0.1]])
    got = Mo.moe(fmt, Gm.W4A4, x, ids, w, exps, shared)
    want = _chain_written_out(fmt, x, shared)                # the shared expert, weight 1
    ys = [_chain_written_out(fmt, x, ex) for ex in exps]
    for t in range(T):
        for j in range(k):
            want[t] += w[t, j] * ys[ids[t, j]][t]
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
    # the routed experts matter and the shared expert enters with weight exactly 1
    assert not np.allclose(got, _chain_written_out(fmt, x, shared), rtol=1e-3)
    alone = Mo.moe(fmt, Gm.W4A4, x, ids, w, exps)
    assert np.allclose(got - alone, _chain_written_out(fmt, x, shared),
                       rtol=1e-12, atol=1e-12 * np.abs(want).max())


def _load_requant_golden(name):
    d = {}
    with open(os.path.join(os.path.dirname(__file__), "golden", name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                key, v = line.split(":", 1)
                d[key.strip()] = v.strip()
    h = np.array([float(t) for t in d["h"].split()], dtype=np.float64)
    codes = np.array([int(t, 16) for t in d["codes"].split()], dtype=np.uint8)
    sc = np.array([int(t, 0) for t in d["scale_codes"].split()], dtype=np.uint8)
    deq = np.array([float(t) for t in d["dequant"].split()])
    return d["fmt"], float(d["a2_scale"]), h, codes, sc, deq


@pytest.mark.parametrize("name", ["nvfp4_requant_h.txt", "mxfp4_requant_h.txt"])
def test_golden_requant_through_down_projection(name):
    # expert_down takes float64 h; through an identity W2 (e2m1 1.0 on the diagonal,
    # block scale 1, weight_scale_2 1) its output is alpha2 x the requantized h, so
    # the hand-worked block pins the fp32 rounding of h, the scale it is quantized
    # under and alpha2
    fmt, a2, h, codes, sc, deq = _load_requant_golden(name)
    n = h.size
    G = Q.GROUP[fmt]
    diag = np.zeros((n, n), np.uint8)
    np.fill_diagonal(diag, 2)                              # e2m1 code 2 = 1.0
    one = 0x38 if fmt == Q.NVFP4 else 127                  # block scale 1.0
    ex = Mo.Expert(None, None, F.pack_nibbles(diag), np.full((n, n // G), one, np.uint8),
                   w2_scale_2=1.0, a2_scale=a2)
    q, s = Q.quantize(fmt, h.astype(np.float32).reshape(1, -1), a2)
    assert list(q[0]) == list(codes) and list(s[0]) == list(sc)
    y = Mo.expert_down(fmt, Gm.W4A4, h.reshape(1, -1), ex)[0]
    assert np.array_equal(y, a2 * deq)


def test_requant_input_is_fp32():
    # The intermediate h is an fp32 value when it is requantized ("vLLM on the NVIDIA DGX
    # Spark (GB10 / sm_121): A Complete Technical Guide", §4.3: SwiGLU between the GEMMs,
    # quantized inside the kernel).  h = 2.5 + 1e-9 rounds to 2.5 in fp32, the midpoint of
    # the e2m1 values 2 and 3, which ties to the even code (2.0); quantized in float64 it
    # would round up to 3.0.  MXFP4 block with amax 4: scale exponent floor(log2 4) - 2 = 0.
    h = np.zeros((1, 32), np.float64)
    h[0, 0] = 4.0
    h[0, 1] = 2.5 + 1e-9
    codes, scales = Q.quantize(Q.MXFP4, h)
    assert scales[0, 0] == 127
    d = Q.dequantize(Q.MXFP4, codes, scales)
    assert d[0, 1] == 2.0 and d[0, 0] == 4.0
    # the down projection sees the same: identity-like weights pick h's second element
    I, H = 32, 32
    w2 = np.zeros((H, I), np.float32)
    w2[0, 1] = 1.0
    w2c, w2s, _ = Q.quantize_weight(Q.MXFP4, w2)
    w13 = np.zeros((2 * I, H), np.float32)
    w13c, w13s, _ = Q.quantize_weight(Q.MXFP4, w13)
    ex = Mo.Expert(w13c, w13s, w2c, w2s)
    y = Mo.expert_down(Q.MXFP4, Gm.W4A4, h, ex)
    assert y[0, 0] == 2.0
