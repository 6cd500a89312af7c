"""GPU parity of the MoE path (router, dispatch, expert GEMMs, SwiGLU + requant,
combine) against the oracle.

Stages: "vLLM on the NVIDIA DGX Spark (GB10 / sm_121): A Complete Technical Guide",
§7.1 and §4.3; alpha and the zero-activation-scale refusal: "GLM-5.3-Flash on vLLM,
on GB10".

Integer work (routing ids, dispatch order, activation codes) must match exactly.
The intermediate h is quantized from an fp32 value that both sides compute with
different accumulation orders, so a code may differ where the oracle's value sits
within a relative 1e-4 of a rounding decision: such differences are checked to be
exactly that, and their effect on the expert output is added to the tolerance
(computed from the two candidate codes).  Everything else follows the GEMM
tolerance: |err| <= 2e-3 * alpha * ||a_hat|| * ||w_hat_n|| per element, and a
relative Frobenius error <= 1e-3.
"""
import copy

import numpy as np
import pytest
import torch

import block_scaled_fp4_quantize_amd as F
from block_scaled_fp4_quantize_amd import tensors as T
import synth
from oracle import formats as OF
from oracle import gemm as OG
from oracle import moe as OM
from oracle import quant as OQ
from tests.gpu_util import DEV, bf16_ulp, round_bf16, to_dev
from tests.moe_data import MoeProblem

pytestmark = pytest.mark.gpu

E2M1_THR = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
E4M3_MID = (OF.E4M3_TABLE[1:0x7F] + OF.E4M3_TABLE[:0x7E]) / 2
EPS = 1e-4


# ---------------------------------------------------------------------------------
# device side
# ---------------------------------------------------------------------------------


def device_moe(pb, flags=0, a13=None):
    st = pb.stacked()
    dev = {n: to_dev(st[n]) for n in ("w13_codes", "w13_scales", "w2_codes", "w2_scales")}
    shared = None
    if pb.shared is not None:
        sh = pb.shared
        shared = dict(w13_codes=to_dev(sh.w13_codes), w13_scales=to_dev(sh.w13_scales),
                      w2_codes=to_dev(sh.w2_codes), w2_scales=to_dev(sh.w2_scales))
        if pb.fmt == OQ.NVFP4:
            shared.update(w13_scale_2=sh.w13_scale_2, w2_scale_2=sh.w2_scale_2)
            if pb.mode == "w4a4":
                shared.update(a13_scale=sh.a13_scale, a2_scale=sh.a2_scale)
    m = T.Moe(pb.fmt, pb.mode, pb.H, pb.I, pb.E, dev["w13_codes"], dev["w13_scales"],
              dev["w2_codes"], dev["w2_scales"], st.get("w13_scale_2"), st.get("w2_scale_2"),
              st.get("a13_scale") if a13 is None else a13, st.get("a2_scale"), shared=shared,
              flags=flags)
    hidden = to_dev(pb.hidden_bits.view(np.int16)).view(torch.bfloat16)
    ids = to_dev(pb.ids.astype(np.int32))
    w = to_dev(pb.w.astype(np.float32))
    return m, hidden, ids, w, dev


def ws_view(ws, off, count, dtype):
    nbytes = count * torch.tensor([], dtype=dtype).element_size()
    return ws[off:off + nbytes].view(dtype)


def run_gpu(pb, flags=0, a13=None, view_mode=None):
    """Run the layer and fetch every stage's output from the workspace.  view_mode:
    the mode whose intermediates to fetch (the layer's own mode by default; "w4a16"
    for a call that fell back to weight-only)."""
    m, hidden, ids, w, dev = device_moe(pb, flags, a13)
    out = torch.full((pb.T, pb.H), float("nan"), dtype=torch.bfloat16, device=DEV)
    _, st = m(hidden, ids, w, out, check=False)
    torch.cuda.synchronize()
    lay = m.layout(hidden, ids, w, out)
    ws = m._ws
    P = pb.T * pb.k
    R = P + (pb.T if pb.shared is not None else 0)
    G = OQ.GROUP[pb.fmt]
    r = dict(status=st, out=out.float().cpu().numpy().astype(np.float64), layout=lay)
    r["offsets"] = ws_view(ws, lay.expert_offsets, pb.E + 1, torch.int32).cpu().numpy()
    r["sorted_rows"] = ws_view(ws, lay.sorted_rows, P, torch.int32).cpu().numpy()
    r["inverse"] = ws_view(ws, lay.inverse, P, torch.int32).cpu().numpy()
    # gate/up rows exist only for the parts without the fused SwiGLU epilogue
    r["gu"] = ws_view(ws, lay.gu, lay.gu_rows * 2 * pb.I, torch.float32).view(lay.gu_rows, 2 * pb.I)
    r["fused"] = int(lay.swiglu_fused)
    r["y"] = ws_view(ws, lay.y, R * pb.H, torch.float32).view(R, pb.H)
    if (view_mode or pb.mode) == "w4a4":
        r["x_codes"] = ws_view(ws, lay.x_codes, lay.x_rows * pb.H // 2, torch.uint8).view(lay.x_rows, -1)
        r["x_scales"] = ws_view(ws, lay.x_scales, lay.x_rows * pb.H // G, torch.uint8).view(lay.x_rows, -1)
        r["h_codes"] = ws_view(ws, lay.h_codes, R * pb.I // 2, torch.uint8).view(R, -1)
        r["h_scales"] = ws_view(ws, lay.h_scales, R * pb.I // G, torch.uint8).view(R, -1)
    else:
        r["h_bf16"] = ws_view(ws, lay.h_bf16, R * pb.I, torch.bfloat16).view(R, pb.I)
    r["_keep"] = (m, hidden, ids, w, dev)
    return r


# ---------------------------------------------------------------------------------
# validity of a differing requantization code
# ---------------------------------------------------------------------------------


def allowed_diffs(fmt, h32, s):
    """Elements of h (fp32 [n, I]) whose quantization sits within EPS of a decision:
    a whole block when its scale choice is that close, else single elements."""
    n, I = h32.shape
    G = OQ.GROUP[fmt]
    hb = np.abs(h32.astype(np.float64)).reshape(n, I // G, G)
    amax = hb.max(-1)
    if fmt == OQ.NVFP4:
        g = float(np.float32(1.0) / np.float32(s))
        sf = amax * g / 6.0
        near_scale = np.min(np.abs(sf[..., None] - E4M3_MID), axis=-1) <= EPS * np.maximum(sf, 1e-30)
        sc = OF.e4m3_encode_pos((amax.astype(np.float32) * np.float32(g)) / np.float32(6.0))
        sd = OF.E4M3_TABLE[sc]
        r = np.where(sd > 0, g / np.where(sd > 0, sd, 1.0), 0.0)
        y = hb * r[..., None]
    else:
        lg = np.log2(np.maximum(amax, 1e-300))
        near_scale = np.abs(lg - np.round(lg)) <= EPS
        E = OF.mx_scale_exponent(amax)
        y = hb * np.ldexp(1.0, -E)[..., None]
    near_elem = np.min(np.abs(y[..., None] - E2M1_THR), axis=-1) <= EPS * np.maximum(y, 1e-30)
    return (near_elem | near_scale[..., None]).reshape(n, I)


# ---------------------------------------------------------------------------------
# oracle side, per routed row
# ---------------------------------------------------------------------------------


def oracle_rows(pb, toks, e):
    """Oracle intermediates of the rows of tokens `toks`, all routed to expert e (or
    'shared'), by the definition: quantize/dequantize x under a13, gate/up times
    alpha13, SiLU(gate) * up, h rounded to fp32 and quantized under a2, down times
    alpha2.  The weight products go through the expert's base matrix and its row
    permutation (a column permutation of the product: the same float64 sums)."""
    ex = pb.shared if e == "shared" else pb.experts[e]
    b, p13, p2 = pb.expert_hat(e)
    w13_base, w2_base, w2_abs = pb.base_hat(b)
    nv = pb.fmt == OQ.NVFP4
    x = pb.hidden[list(toks)]
    if pb.mode == "w4a4":
        s13 = ex.a13_scale if nv else 1.0
        xc, xs = OQ.quantize_packed(pb.fmt, x, s13)
        x_hat = OQ.dequantize_packed(pb.fmt, xc, xs)
        a13 = OG.alpha(pb.fmt, OG.W4A4, ex.w13_scale_2, s13)
    else:
        xc = xs = None
        x_hat = x.astype(np.float64)
        a13 = OG.alpha(pb.fmt, OG.W4A16, ex.w13_scale_2)
    gu = (a13 * (x_hat @ w13_base.T))[:, p13]
    h = OM.swiglu(gu)
    if pb.mode == "w4a4":
        s2 = ex.a2_scale if nv else 1.0
        h32 = h.astype(np.float32)
        hc, hs = OQ.quantize_packed(pb.fmt, h32, s2)
        h_hat = OQ.dequantize_packed(pb.fmt, hc, hs)
        a2 = OG.alpha(pb.fmt, OG.W4A4, ex.w2_scale_2, s2)
    else:
        h32, hc, hs, s2 = None, None, None, None
        h_hat = round_bf16(h)
        a2 = OG.alpha(pb.fmt, OG.W4A16, ex.w2_scale_2)
    y = (a2 * (h_hat @ w2_base.T))[:, p2]
    n13 = np.linalg.norm(w13_base, axis=1)[p13]
    n2 = np.linalg.norm(w2_base, axis=1)[p2]
    return dict(gu=gu, h=h, h32=h32, hc=hc, hs=hs, s2=s2, h_hat=h_hat, y=y, a2=a2,
                x_hat=x_hat, a13=a13, xc=xc, xs=xs, n13=n13, n2=n2, w2_abs=w2_abs, p2=p2)


def expected_dispatch(ids, E):
    """(offsets, sorted_rows, inverse) the dispatch must produce: the oracle's stable
    counting sort over the slots whose id lies in [0, E); the dropped slots have
    inverse -1 and the sorted positions past the routed count hold -1."""
    flat = np.asarray(ids).reshape(-1)
    valid = (flat >= 0) & (flat < E)
    if valid.all():
        return OM.permute(ids, E)
    vidx = np.nonzero(valid)[0]
    off, rows_c, inv_c = OM.permute(flat[vidx].reshape(-1, 1), E)
    rows = np.full(flat.size, -1, np.int32)
    rows[:vidx.size] = vidx[rows_c]
    inv = np.full(flat.size, -1, np.int32)
    inv[vidx] = inv_c
    return off, rows, inv


def coverage_tokens(pb, n_random, seed):
    """Tokens whose rows reach every touched expert's last (ragged) row block -- the
    token of each expert's last sorted row -- and the last 64 rows of the expert with
    the most rows, plus n_random more drawn at random."""
    off, rows, _ = expected_dispatch(pb.ids, pb.E)
    k = pb.k
    toks = set()
    for e in range(pb.E):
        if off[e + 1] > off[e]:
            toks.add(int(rows[off[e + 1] - 1]) // k)
    hot = int(np.argmax(np.diff(off)))
    for p in range(max(off[hot], off[hot + 1] - 64), off[hot + 1]):
        toks.add(int(rows[p]) // k)
    rng = np.random.default_rng(seed)
    extra = rng.choice(pb.T, min(n_random, pb.T), replace=False)
    toks.update(int(t) for t in extra)
    return np.array(sorted(toks))


def verify(pb, r, tokens=None, max_diff_frac=1e-4, max_diff_abs=0, status=F.FP4_OK):
    """Check every stage for the given tokens (all by default).  At most
    max(max_diff_frac * n, max_diff_abs) of the n intermediate codes checked may
    differ from the oracle's, each only next to a rounding decision."""
    T_, k, E, H, I = pb.T, pb.k, pb.E, pb.H, pb.I
    tokens = np.arange(T_) if tokens is None else np.asarray(tokens)
    G = OQ.GROUP[pb.fmt]
    assert r["status"] == status, F.status_str(r["status"])
    # dispatch bookkeeping: exact
    off, rows, inv = expected_dispatch(pb.ids, E)
    assert np.array_equal(r["offsets"], off)
    assert np.array_equal(r["sorted_rows"], rows)
    assert np.array_equal(r["inverse"], inv)
    P = T_ * k
    # rows to check: (sorted position, token, routing weight), grouped by expert
    work = {}
    for t in tokens:
        for j in range(k):
            e = int(pb.ids[t, j])
            if not 0 <= e < E:
                continue                                 # dropped slot
            work.setdefault(e, []).append((int(inv[t * k + j]), int(t), float(np.float32(pb.w[t, j]))))
    if pb.shared is not None:
        work["shared"] = [(P + int(t), int(t), 1.0) for t in tokens]
    contrib = {int(t): [] for t in tokens}       # per token: (y_ref, bound_vec, allowance_vec, w)
    n_diff = n_total = 0
    gu_all = r["gu"]
    y_all = r["y"]
    for e, items in work.items():
        pos = np.array([p for p, _, _ in items])
        toks = [t for _, t, _ in items]
        o = oracle_rows(pb, toks, e)
        # GEMM1 input codes (W4A4): exact
        if pb.mode == "w4a4":
            xr = np.array(toks) if pb.fmt == OQ.MXFP4 else pos
            assert np.array_equal(r["x_codes"][xr].cpu().numpy(), o["xc"]), f"x codes, expert {e}"
            assert np.array_equal(r["x_scales"][xr].cpu().numpy(), o["xs"]), f"x scales, expert {e}"
        # GEMM1 output (fp32), unless the SwiGLU epilogue was fused into GEMM1: then
        # gate/up never reach memory and the intermediate codes below check it
        fused = bool(r["fused"] & (2 if e == "shared" else 1))
        if not fused:
            routed_rows = 0 if r["fused"] & 1 else P
            grow = pos - P + routed_rows if e == "shared" else pos
            gu = gu_all[grow].cpu().numpy().astype(np.float64)
            b1 = 2e-3 * abs(o["a13"]) * np.outer(np.linalg.norm(o["x_hat"], axis=1), o["n13"])
            assert (np.abs(gu - o["gu"]) <= b1).all(), f"gate/up outside tolerance, expert {e}"
            assert np.linalg.norm(gu - o["gu"]) <= 1e-5 * np.linalg.norm(o["gu"]) + 1e-30
        # intermediate
        if pb.mode == "w4a4":
            gc = OF.unpack_nibbles(r["h_codes"][pos].cpu().numpy())
            gs = r["h_scales"][pos].cpu().numpy()
            oc = OF.unpack_nibbles(o["hc"])
            diff = (gc != oc) | np.repeat(gs != o["hs"], G, axis=1)
            ok = allowed_diffs(pb.fmt, o["h32"], o["s2"])
            assert not (diff & ~ok).any(), f"intermediate codes differ away from a rounding decision, expert {e}"
            n_diff += int(diff.sum())
            n_total += diff.size
            g_hat = OQ.dequantize(pb.fmt, gc, gs)
            dh = np.abs(g_hat - o["h_hat"])
        else:
            g_hat = r["h_bf16"][pos].float().cpu().numpy().astype(np.float64)
            # bf16 rounding of an fp32 value computed in another order: one bf16 ulp
            dh = np.abs(g_hat - o["h_hat"])
            assert (dh <= bf16_ulp(o["h_hat"]) + 1e-30).all(), f"h (bf16), expert {e}"
        allow = abs(o["a2"]) * (dh @ o["w2_abs"].T)[:, o["p2"]]      # [rows, H]
        y = y_all[pos].cpu().numpy().astype(np.float64)
        b2 = 2e-3 * abs(o["a2"]) * np.outer(np.linalg.norm(o["h_hat"], axis=1), o["n2"])
        assert (np.abs(y - o["y"]) <= b2 + allow * (1 + 1e-6) + 1e-30).all(), f"down projection, expert {e}"
        for i, (_, t, wt) in enumerate(items):
            contrib[t].append((o["y"][i], b2[i], allow[i], wt))
    limit = max(max_diff_frac * n_total, max_diff_abs)
    assert n_diff <= limit, f"{n_diff}/{n_total} intermediate codes differ (limit {limit:g})"
    # combine
    zero = np.zeros(H)
    ref_all, bound_all = [], []
    for t in tokens:
        c = contrib[int(t)]
        ref_all.append(sum((wt * yr for yr, _, _, wt in c), zero))
        bound_all.append(sum((wt * (b + a) for _, b, a, wt in c), zero))
    ref_all, bound_all = np.stack(ref_all), np.stack(bound_all)
    ref_c = round_bf16(ref_all)
    got = r["out"][tokens]
    bad = np.abs(got - ref_c) > bound_all + bf16_ulp(ref_c) + 1e-30
    assert not bad.any(), f"out rows {tokens[np.nonzero(bad.any(1))[0]][:8]}"
    den = np.linalg.norm(ref_c)
    if den > 0:
        rel = np.linalg.norm(got - ref_c) / den
        assert rel <= 1e-3, f"relative Frobenius error {rel:.3g}"
    print(f"[moe verify] {pb.fmt} {pb.mode} T={T_} E={E}: {len(tokens)} tokens, "
          f"{n_diff}/{n_total} intermediate codes differ", flush=True)
    return n_diff, n_total, ref_all


# ---------------------------------------------------------------------------------
# tests
# ---------------------------------------------------------------------------------


@pytest.mark.parametrize("T_,E,k", [(64, 128, 8), (5, 100, 3), (300, 256, 8), (7, 8, 8)])
def test_topk_softmax(T_, E, k):
    logits = synth.normal((T_, E), seed=T_, role=synth.LOGITS)
    logits[0, :4] = logits[0, 4]                    # a tie: lower index first
    ids, w = T.topk_softmax(to_dev(logits), k)
    torch.cuda.synchronize()
    rid, rw = OM.topk_softmax(logits, k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.allclose(w.cpu().numpy(), rw, rtol=2e-6, atol=1e-7)
    ids2, w2 = T.topk_softmax(to_dev(logits), k, renormalize=False)
    _, rw2 = OM.topk_softmax(logits, k, renormalize=False)
    assert np.allclose(w2.cpu().numpy(), rw2, rtol=2e-6, atol=1e-7)


def test_topk_zipf_8192():
    logits = synth.zipf_gumbel_logits(8192, 256, 1.1, seed=0)
    ids, w = T.topk_softmax(to_dev(logits), 8)
    torch.cuda.synchronize()
    rid, rw = OM.topk_softmax(logits, 8)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.allclose(w.cpu().numpy(), rw, rtol=2e-6, atol=1e-7)


SMALL = [
    ("nvfp4", "w4a4", dict(T=5, H=64, I=32, E=8, k=2, shared=True)),
    ("mxfp4", "w4a4", dict(T=5, H=64, I=32, E=8, k=2, shared=True)),
    ("nvfp4", "w4a16", dict(T=6, H=128, I=64, E=4, k=2, shared=True)),
    ("mxfp4", "w4a16", dict(T=6, H=128, I=64, E=4, k=2, shared=False)),
    ("nvfp4", "w4a4", dict(T=40, H=256, I=96, E=16, k=4, shared=False)),
    ("mxfp4", "w4a4", dict(T=33, H=256, I=96, E=16, k=4, shared=True)),
    ("nvfp4", "w4a4", dict(T=1, H=64, I=48, E=4, k=1, shared=False)),
    # more NVFP4 experts than one by-value scalar pack holds (4 scalars each, 192
    # experts at most): the scalars take their own launch and the dispatch runs as three
    # kernels even at this token count; and a token count whose activations are too
    # many to quantize inside the one-workgroup dispatch
    ("nvfp4", "w4a4", dict(T=3, H=64, I=32, E=200, k=2, shared=False)),
    ("nvfp4", "w4a4", dict(T=100, H=1024, I=64, E=8, k=2, shared=True)),
    # >= 48 routed rows per expert on average, H and I multiples of 128: the grouped
    # GEMMs run on 128-row tiles, with ragged expert row counts
    ("nvfp4", "w4a4", dict(T=150, H=256, I=128, E=4, k=2, shared=True)),
    ("mxfp4", "w4a4", dict(T=200, H=384, I=256, E=6, k=3, shared=True)),
    # decode token counts with H and I multiples of 128: SwiGLU + requant ride on the
    # streaming gate/up GEMM where it streams anyway (MXFP4 expert tables, the shared
    # expert) or has at most 16 rows
    ("nvfp4", "w4a4", dict(T=8, H=256, I=128, E=8, k=2, shared=True)),
    ("nvfp4", "w4a4", dict(T=60, H=256, I=128, E=8, k=4, shared=False)),
    ("mxfp4", "w4a4", dict(T=40, H=384, I=256, E=16, k=4, shared=True)),
    ("mxfp4", "w4a4", dict(T=1, H=256, I=128, E=8, k=2, shared=False)),
    # W4A16 experts averaging >= 48 rows, H and I multiples of 128: the grouped GEMMs run on
    # the W4A16 tile kernel's 128-row blocks
    ("nvfp4", "w4a16", dict(T=150, H=256, I=128, E=4, k=2, shared=True)),
    ("mxfp4", "w4a16", dict(T=200, H=384, I=256, E=6, k=3, shared=False)),
    # NVFP4 W4A4 with at most 4 tokens and 32 routed slots and no shared expert: the
    # two-launch layer (gate/up with routing and activation quantization; down projection
    # with the weighted combine), incl. its longer-K variants (H > 2048, I > 1024)
    ("nvfp4", "w4a4", dict(T=1, H=256, I=128, E=8, k=2, shared=False)),
    ("nvfp4", "w4a4", dict(T=3, H=384, I=256, E=16, k=8, shared=False)),
    ("nvfp4", "w4a4", dict(T=2, H=128, I=128, E=20, k=16, shared=False)),
    ("nvfp4", "w4a4", dict(T=4, H=256, I=128, E=9, k=8, shared=False)),
    ("nvfp4", "w4a4", dict(T=2, H=4096, I=256, E=4, k=2, shared=False)),
    ("nvfp4", "w4a4", dict(T=1, H=256, I=2048, E=4, k=3, shared=False)),
    # more than 8 experts per token: the combine adds a token's slots in groups of 8,
    # the last one partial
    ("nvfp4", "w4a4", dict(T=7, H=128, I=64, E=24, k=12, shared=True)),
    ("mxfp4", "w4a4", dict(T=5, H=128, I=64, E=32, k=20, shared=False)),
]


@pytest.mark.parametrize("fmt,mode,kw", SMALL)
def test_moe_small(fmt, mode, kw):
    pb = MoeProblem(fmt, mode, seed=kw["T"] + kw["E"], **kw)
    r = run_gpu(pb)
    if mode == "w4a4" and kw["H"] % 128 == 0 and kw["I"] % 128 == 0:
        # 128-row expert blocks or MXFP4 expert tables (tiled or streaming kernels):
        # SwiGLU + requant ride on the routed gate/up GEMM, and on the shared expert's
        if kw["T"] * kw["k"] >= 48 * kw["E"] or fmt == "mxfp4":
            assert r["fused"] & 1, r["fused"]
        if kw["shared"]:
            assert r["fused"] & 2, r["fused"]
    verify(pb, r, max_diff_abs=2)


def test_moe_deterministic():
    pb = MoeProblem("nvfp4", "w4a4", T=20, H=128, I=64, E=8, k=2, seed=3, shared=True)
    a = run_gpu(pb)["out"]
    b = run_gpu(pb)["out"]
    assert np.array_equal(a, b)


def test_zero_activation_scale_rejected_not_zeroed():
    pb = MoeProblem("nvfp4", "w4a4", T=8, H=64, I=32, E=4, k=2, seed=5, shared=True)
    st = pb.stacked()
    a13 = st["a13_scale"].copy()
    a13[2] = 0.0                                  # a weight-only checkpoint's missing scale
    m, hidden, ids, w, dev = device_moe(pb, a13=a13)
    out = torch.full((pb.T, pb.H), 7.0, dtype=torch.bfloat16, device=DEV)
    _, s = m(hidden, ids, w, out, check=False)
    torch.cuda.synchronize()
    assert s == F.FP4_ERR_INPUT_SCALE
    assert (out == 7.0).all()                     # nothing ran
    # with the opt-in flag the layer runs weight-only and says so; every stage then
    # matches the W4A16 oracle to the usual bounds
    r = run_gpu(pb, flags=F.FP4_FLAG_ALLOW_W4A16_FALLBACK, a13=a13, view_mode="w4a16")
    pb16 = copy.copy(pb)
    pb16.mode = "w4a16"
    verify(pb16, r, status=F.FP4_OK_FELL_BACK_W4A16)
    got = r["out"]
    # and it is not the zeroed-experts output of the page's bug
    for ex in pb.experts:
        ex.a13_scale = 0.0
    buggy = OM.moe("nvfp4", "w4a4", pb.hidden, pb.ids, pb.w, pb.experts, pb.shared, buggy=True)
    assert np.linalg.norm(got - buggy) > 0.1 * np.linalg.norm(got)


@pytest.mark.parametrize("fmt,kw", [
    ("nvfp4", dict(T=20, H=128, I=64, E=8, k=4)),      # one-workgroup dispatch, folded quant
    ("nvfp4", dict(T=100, H=1024, I=64, E=8, k=2)),    # one-workgroup dispatch, quant pass
    ("nvfp4", dict(T=200, H=256, I=64, E=16, k=8)),    # three-kernel dispatch, unfused SwiGLU
    ("nvfp4", dict(T=150, H=256, I=128, E=4, k=2)),    # 128-row tiles, fused SwiGLU
    ("mxfp4", dict(T=200, H=256, I=64, E=16, k=8)),
    ("nvfp4", dict(T=20, H=256, I=128, E=8, k=4)),     # streaming fused SwiGLU
    ("mxfp4", dict(T=9, H=384, I=128, E=8, k=2)),
    ("nvfp4", dict(T=6, H=128, I=64, E=16, k=12)),     # two combine groups of slots
    ("nvfp4", dict(T=3, H=256, I=128, E=8, k=4, shared=False)),   # the two-launch small layer
])
def test_moe_dropped_ids(fmt, kw):
    # expert ids outside [0, E) (device data, not checked on the host) drop their slot:
    # it contributes nothing, and the passes that walk every sorted position stay in
    # bounds.  Token 0 has every slot dropped and gets only the shared expert (zero
    # without one).
    kw = dict(kw)
    shared = kw.pop("shared", True)
    pb = MoeProblem(fmt, "w4a4", seed=kw["T"] + 11, shared=shared, **kw)
    rng = np.random.default_rng(12)
    ids = pb.ids.copy()
    drop = rng.random(ids.shape) < 0.2
    ids[drop] = rng.choice(np.array([-1, kw["E"], 1 << 30, -(1 << 31)]), size=int(drop.sum()))
    ids[0, :] = -1
    pb.ids = ids.astype(np.int32)
    r = run_gpu(pb)
    verify(pb, r, max_diff_abs=2)


@pytest.mark.parametrize("T_", [1, 64, 4096])
def test_nvfp4_moe_128_experts(T_):
    # 128 experts, top-8 softmax routing from N(0,1) logits, hidden 2048, gate+up
    # 2048 -> 1536, down 768 -> 2048.  Every token is checked up to T = 64; at T =
    # 4096 the tokens that reach each expert's last row block, the busiest expert's
    # last 64 rows and 64 more at random.
    pb = MoeProblem("nvfp4", "w4a4", T=T_, H=2048, I=768, E=128, k=8, seed=0, n_base=8)
    r = run_gpu(pb)
    toks = None if T_ <= 64 else coverage_tokens(pb, 64, seed=0)
    verify(pb, r, tokens=toks)


@pytest.mark.parametrize("T_", [64, 8192])
def test_mxfp4_moe_256_experts_shared_zipf(T_):
    # 256 experts top-8 + 1 shared, hidden 6144, intermediate 2048, Zipf(1.1) routing.
    # Every token at T = 64; at T = 8192 the tokens that reach each touched expert's
    # last row block, the hottest expert's last 64 rows and 64 more at random.
    pb = MoeProblem("mxfp4", "w4a4", T=T_, H=6144, I=2048, E=256, k=8, seed=0, n_base=4,
                    shared=True, zipf=1.1)
    r = run_gpu(pb)
    toks = None if T_ <= 64 else coverage_tokens(pb, 64, seed=1)
    verify(pb, r, tokens=toks)
