"""Mixture-of-experts layer over block-scaled FP4 experts, by definition.

Test infrastructure: only tests, the smoke check and the bench's CPU-baseline leg
use this module.

Sources
* "vLLM on the NVIDIA DGX Spark (GB10 / sm_121): A Complete Technical Guide",
  §7.1 (modular fused-MoE architecture): Router -> Quantize-Dispatch ->
  Permute-Experts-Unpermute -> Combine.
* Same guide, §4.3 (b12x): the fused expert does token dispatch, two GEMMs with a
  SwiGLU activation between them, and the top-k-weighted reduction; the BF16
  input is quantized to FP4 inside.
* "GLM-5.3-Flash on vLLM, on GB10": per-expert dequant alpha is
  weight_scale_2 * input_scale; a weight-only checkpoint leaves the activation
  scale at zero, which silently multiplies every routed expert by zero while the
  shared expert still runs.  Here that case is refused (``InputScaleError``); the
  test-only ``buggy=True`` switch reproduces the zeroed behaviour so tests can
  prove the library does not.

Readings where the pages are silent:
* routing: top-k of the fp32 logits, larger first, ties to the lower expert
  index; weights are the softmax over all experts (float64) taken at the chosen
  experts, divided by their sum when ``renormalize`` is set.
* W13 rows [0, I) are the gate projection and rows [I, 2I) the up projection;
  SwiGLU h = SiLU(gate) * up with SiLU(z) = z / (1 + exp(-z)).
* W4A4: the expert input is quantized under the expert's a13_scale (NVFP4) or per
  32-block (MXFP4); the intermediate h is rounded to fp32 and quantized under
  a2_scale (NVFP4) or per 32-block (MXFP4).  W4A16: the expert input is the bf16
  hidden state and h is rounded to bf16 before the down projection.
* the shared expert has the routed experts' shapes and format and weight 1.
* permute order: rows grouped by expert in increasing expert index; inside an
  expert, by the flat index t*k + j (a stable counting sort).
"""
import numpy as np

from . import gemm as Gm
from . import quant as Q


# ----------------------------------------------------------------------------------
# router
# ----------------------------------------------------------------------------------


def topk_softmax(logits, k, renormalize=True):
    """(ids int32 [T, k], weights float64 [T, k]) for fp32 logits [T, E]."""
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        row = logits[t]
        # stable sort on (-logit, index): larger logits first, lower index on ties
        order = np.lexsort((np.arange(E), -row.astype(np.float64)))
        ids[t] = order[:k]
    l64 = logits.astype(np.float64)
    mx = l64.max(axis=1, keepdims=True)
    p = np.exp(l64 - mx)
    p /= p.sum(axis=1, keepdims=True)
    w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return ids, w


# ----------------------------------------------------------------------------------
# dispatch bookkeeping
# ----------------------------------------------------------------------------------


def permute(ids, E):
    """Stable counting sort of the (token, slot) pairs by expert.

    Returns (expert_offsets int32 [E+1], sorted_rows int32 [T*k], inverse int32 [T*k]):
    sorted_rows[p] is the flat index t*k + j of the p-th routed row; inverse is its
    inverse permutation.
    """
    ids = np.asarray(ids, dtype=np.int64)
    flat = ids.reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_rows = np.empty(flat.size, dtype=np.int64)
    fill = offsets[:-1].copy()
    for i, e in enumerate(flat):
        sorted_rows[fill[e]] = i
        fill[e] += 1
    inverse = np.empty_like(sorted_rows)
    inverse[sorted_rows] = np.arange(flat.size)
    return offsets.astype(np.int32), sorted_rows.astype(np.int32), inverse.astype(np.int32)


# ----------------------------------------------------------------------------------
# one expert
# ----------------------------------------------------------------------------------


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def _round_bf16(x):
    """Round float values to bfloat16 (round to nearest even), returned as float64."""
    f = np.asarray(x, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


class Expert:
    """Packed weights of one expert.

    w13_codes [2I, H/2], w13_scales [2I, H/G], w2_codes [H, I/2], w2_scales [H, I/G];
    NVFP4 adds w13_scale_2 / w2_scale_2 (weight) and a13_scale / a2_scale (activation).
    """

    def __init__(self, w13_codes, w13_scales, w2_codes, w2_scales, w13_scale_2=1.0,
                 w2_scale_2=1.0, a13_scale=1.0, a2_scale=1.0):
        self.w13_codes, self.w13_scales = w13_codes, w13_scales
        self.w2_codes, self.w2_scales = w2_codes, w2_scales
        self.w13_scale_2, self.w2_scale_2 = w13_scale_2, w2_scale_2
        self.a13_scale, self.a2_scale = a13_scale, a2_scale


def expert_gu(fmt, mode, x, ex, buggy=False):
    """gate/up projection of rows x [n, H] -> float64 [n, 2I] (gate cols [0, I), up [I, 2I))."""
    x = np.asarray(x, dtype=np.float32)
    if mode == Gm.W4A16:
        return Gm.gemm_w4a16(fmt, x, ex.w13_codes, ex.w13_scales, ex.w13_scale_2)
    if fmt == Q.NVFP4:
        s = ex.a13_scale
        if buggy and float(s) == 0.0:
            # the GLM page's fault: a zero activation scale zeroes alpha
            return Gm.gemm_fused(fmt, x, ex.w13_codes, ex.w13_scales, ex.w13_scale_2, 1.0) * 0.0
        return Gm.gemm_fused(fmt, x, ex.w13_codes, ex.w13_scales, ex.w13_scale_2, s)
    return Gm.gemm_fused(fmt, x, ex.w13_codes, ex.w13_scales)


def swiglu(gu):
    """h = SiLU(gate) * up for gu [n, 2I] (float64)."""
    gu = np.asarray(gu, dtype=np.float64)
    I = gu.shape[1] // 2
    return silu(gu[:, :I]) * gu[:, I:]


def expert_h(fmt, mode, x, ex, buggy=False):
    """gate/up projection and SwiGLU for rows x [n, H] -> h float64 [n, I]."""
    return swiglu(expert_gu(fmt, mode, x, ex, buggy))


def expert_down(fmt, mode, h, ex, buggy=False):
    """Down projection of the intermediate h [n, I] (float64) -> y float64 [n, H]."""
    if mode == Gm.W4A16:
        return Gm.gemm_w4a16(fmt, _round_bf16(h), ex.w2_codes, ex.w2_scales, ex.w2_scale_2)
    h32 = np.asarray(h, dtype=np.float32)        # the intermediate is fp32 before requant
    if fmt == Q.NVFP4:
        s = ex.a2_scale
        if buggy and float(s) == 0.0:
            return Gm.gemm_fused(fmt, h32, ex.w2_codes, ex.w2_scales, ex.w2_scale_2, 1.0) * 0.0
        return Gm.gemm_fused(fmt, h32, ex.w2_codes, ex.w2_scales, ex.w2_scale_2, s)
    return Gm.gemm_fused(fmt, h32, ex.w2_codes, ex.w2_scales)


def expert_forward(fmt, mode, x, ex, buggy=False):
    return expert_down(fmt, mode, expert_h(fmt, mode, x, ex, buggy), ex, buggy)


def check_moe_scales(fmt, mode, experts, shared=None):
    """The refusal rule: NVFP4 W4A4 needs every activation scale finite and positive."""
    if fmt != Q.NVFP4 or mode != Gm.W4A4:
        return
    for e, ex in enumerate(list(experts) + ([shared] if shared is not None else [])):
        Q.check_scale(ex.a13_scale)
        Q.check_scale(ex.a2_scale)


# ----------------------------------------------------------------------------------
# the layer
# ----------------------------------------------------------------------------------


def moe(fmt, mode, hidden, ids, weights, experts, shared=None, buggy=False,
        tokens=None):
    """out[t] = sum_j weights[t, j] * expert_{ids[t, j]}(hidden[t]) (+ shared(hidden[t])).

    hidden: [T, H] bf16 values; ids/weights: [T, k].  Returns float64 [len(tokens), H]
    for the selected token indices (all tokens by default).  Raises
    quant.InputScaleError under the refusal rule unless ``buggy`` is set.
    """
    if not buggy:
        check_moe_scales(fmt, mode, experts, shared)
    hidden = np.asarray(hidden, dtype=np.float32)
    ids = np.asarray(ids)
    weights = np.asarray(weights, dtype=np.float64)
    T, H = hidden.shape
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    out = np.zeros((len(toks), H), dtype=np.float64)
    pos = {int(t): i for i, t in enumerate(toks)}
    k = ids.shape[1]
    # group the selected (token, slot) pairs by expert so each expert runs once
    by_expert = {}
    for t in toks:
        for j in range(k):
            by_expert.setdefault(int(ids[t, j]), []).append((int(t), j))
    for e, pairs in sorted(by_expert.items()):
        rows = np.array([t for t, _ in pairs])
        y = expert_forward(fmt, mode, hidden[rows], experts[e], buggy)
        for r, (t, j) in enumerate(pairs):
            out[pos[t]] += weights[t, j] * y[r]
    if shared is not None:
        out += expert_forward(fmt, mode, hidden[toks], shared, buggy)
    return out
