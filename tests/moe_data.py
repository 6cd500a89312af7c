"""Synthetic MoE problems for the tests and the bench.

Experts: ``n_base`` experts are drawn (weights N(0, 0.02)) and quantized by the oracle;
every further expert is a seeded row permutation of one of them (expert e uses base
e % n_base).  Permuting rows of a quantized matrix is the same as quantizing the
row-permuted matrix (quantization is per row), so every expert is a valid quantized
N(0, 0.02) matrix, and no two experts are equal -- a wrong expert index changes the
result.  This keeps the 257-expert layer affordable to generate on the CPU.
"""
import numpy as np

import synth
from oracle import moe as OM
from oracle import quant as OQ


def _perm_rows(a, perm):
    return None if a is None else np.ascontiguousarray(a[perm])


class MoeProblem:
    def __init__(self, fmt, mode, T, H, I, E, k, seed=0, n_base=None, shared=False,
                 zipf=None, calib_tokens=16):
        self.fmt, self.mode, self.T, self.H, self.I, self.E, self.k = fmt, mode, T, H, I, E, k
        n_base = E if n_base is None else min(n_base, E)
        bases = []
        for b in range(n_base + (1 if shared else 0)):
            w13 = synth.normal((2 * I, H), 0.02, seed=seed, role=synth.W13, index=b)
            w2 = synth.normal((H, I), 0.02, seed=seed, role=synth.W2, index=b)
            bases.append((OQ.quantize_weight(fmt, w13), OQ.quantize_weight(fmt, w2)))
        self.experts = []
        # expert e = base e % n_base with its W13 rows permuted by perm13[e] and its W2
        # rows by perm2[e] (identity for the bases themselves); the shared expert is
        # base n_base, unpermuted
        self.bases = bases
        self.base_of, self.perm13, self.perm2 = [], [], []
        for e in range(E):
            (c13, s13, ws13), (c2, s2, ws2) = bases[e % n_base]
            p13, p2 = np.arange(2 * I), np.arange(H)
            if e >= n_base:
                p13 = synth.rows_permutation(2 * I, seed=seed, index=2 * e)
                p2 = synth.rows_permutation(H, seed=seed, index=2 * e + 1)
                c13, s13, c2, s2 = (_perm_rows(c13, p13), _perm_rows(s13, p13),
                                    _perm_rows(c2, p2), _perm_rows(s2, p2))
            self.experts.append(OM.Expert(c13, s13, c2, s2, ws13, ws2))
            self.base_of.append(e % n_base)
            self.perm13.append(p13)
            self.perm2.append(p2)
        self.shared = None
        if shared:
            (c13, s13, ws13), (c2, s2, ws2) = bases[-1]
            self.shared = OM.Expert(c13, s13, c2, s2, ws13, ws2)
        self._hat = {}
        x = synth.normal((T, H), seed=seed, role=synth.HIDDEN)
        self.hidden_bits, self.hidden = synth.bf16_bits(x)
        if zipf is None:
            self.logits = synth.normal((T, E), seed=seed, role=synth.LOGITS)
        else:
            self.logits = synth.zipf_gumbel_logits(T, E, s=zipf, seed=seed)
        self.ids, self.w = OM.topk_softmax(self.logits, k)
        if fmt == OQ.NVFP4 and mode == "w4a4":
            self._calibrate(calib_tokens)

    def _calibrate(self, n):
        """Activation scales: a13 = amax(hidden)/2688 (varied per expert so a wrong
        expert index shows), a2 = amax of the oracle's intermediate on n calibration
        tokens / 2688, also varied per expert."""
        base13 = float(np.abs(self.hidden).max()) / 2688.0
        for e, ex in enumerate(self.experts):
            ex.a13_scale = float(np.float32(base13 * (1.0 + (e % 5) / 8.0)))
        probe = self.experts[: min(4, self.E)]
        hmax = 0.0
        for ex in probe:
            h = OM.expert_h(self.fmt, self.mode, self.hidden[:n], ex)
            hmax = max(hmax, float(np.abs(h).max()))
        base2 = hmax / 2688.0
        for e, ex in enumerate(self.experts):
            ex.a2_scale = float(np.float32(base2 * (1.0 + (e % 3) / 4.0)))
        if self.shared is not None:
            self.shared.a13_scale = float(np.float32(base13))
            h = OM.expert_h(self.fmt, self.mode, self.hidden[:n], self.shared)
            self.shared.a2_scale = float(np.float32(float(np.abs(h).max()) / 2688.0))

    # -- dequantized weights, through the bases ------------------------------------
    def base_hat(self, b):
        """Exact dequantized (w13_hat [2I, H], w2_hat [H, I], |w2_hat|) of base b (the
        shared expert is base n_base), computed once by the oracle's dequantizer."""
        if b not in self._hat:
            (c13, s13, _), (c2, s2, _) = self.bases[b]
            w13 = OQ.dequantize_packed(self.fmt, c13, s13)
            w2 = OQ.dequantize_packed(self.fmt, c2, s2)
            self._hat[b] = (w13, w2, np.abs(w2))
        return self._hat[b]

    def expert_hat(self, e):
        """(base index, perm13, perm2) of expert e, or of the shared expert for e ==
        'shared': expert e's w13_hat is base_hat(b)[0][perm13] and its w2_hat is
        base_hat(b)[1][perm2], so x @ w13_hat.T == (x @ base_w13_hat.T)[:, perm13]."""
        if e == "shared":
            return len(self.bases) - 1, slice(None), slice(None)
        return self.base_of[e], self.perm13[e], self.perm2[e]

    # -- stacked arrays for the device --------------------------------------------
    def stacked(self):
        st = lambda name: np.stack([getattr(ex, name) for ex in self.experts])
        out = {n: st(n) for n in ("w13_codes", "w13_scales", "w2_codes", "w2_scales")}
        if self.fmt == OQ.NVFP4:
            out["w13_scale_2"] = np.array([ex.w13_scale_2 for ex in self.experts], np.float32)
            out["w2_scale_2"] = np.array([ex.w2_scale_2 for ex in self.experts], np.float32)
            if self.mode == "w4a4":
                out["a13_scale"] = np.array([ex.a13_scale for ex in self.experts], np.float32)
                out["a2_scale"] = np.array([ex.a2_scale for ex in self.experts], np.float32)
        return out

    def oracle_out(self, tokens=None):
        return OM.moe(self.fmt, self.mode, self.hidden, self.ids, self.w, self.experts,
                      self.shared, tokens=tokens)
