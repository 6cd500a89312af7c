"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws random numbers and lays them out; it holds none of the
quantization, matmul or routing arithmetic.  Both the CPU oracle and the GPU
library consume what it produces, and neither is imported here.

Every tensor comes from its own PCG64 stream, keyed by (seed, role, index), so a
tensor does not change when another one is added or resized.
"""
import numpy as np

# stream roles
WEIGHT, ACT, OUTLIER, LOGITS, W13, W2, HIDDEN, PERM, MISC = range(1, 10)


def rng(seed, role, index=0):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, role, index])))


def normal(shape, std=1.0, seed=0, role=ACT, index=0):
    """float32 N(0, std^2) samples."""
    g = rng(seed, role, index)
    return (g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def with_outliers(x, frac=0.01, factor=20.0, seed=0, index=0):
    """Multiply exactly round(frac * numel) entries, drawn uniformly without
    replacement, by ``factor`` (applied before any bf16 rounding)."""
    x = np.array(x, dtype=np.float32, copy=True)
    n = int(round(frac * x.size))
    if n:
        g = rng(seed, OUTLIER, index)
        pos = g.choice(x.size, size=n, replace=False)
        flat = x.reshape(-1)
        flat[pos] *= np.float32(factor)
    return x


def bf16_bits(x):
    """Round float32 values to bfloat16 (nearest even) -> (uint16 bits, float32 values).

    Uses torch's own conversion, which rounds to nearest even.
    """
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16).copy()
    vals = t.to(torch.float32).numpy().copy()
    return bits, vals


def zipf_gumbel_logits(T, E, s=1.1, seed=0, index=0):
    """Router logits whose top-k is a draw without replacement from Zipf(s) over a
    seeded permutation of the experts: logit = log p_e + Gumbel(0, 1)."""
    gp = rng(seed, PERM, index)
    perm = gp.permutation(E)
    rank = np.empty(E, dtype=np.int64)
    rank[perm] = np.arange(1, E + 1)
    logp = -s * np.log(rank.astype(np.float64))
    logp -= np.log(np.exp(logp).sum())
    g = rng(seed, LOGITS, index)
    gumbel = g.gumbel(size=(T, E))
    return (logp[None, :] + gumbel).astype(np.float32)


def rows_permutation(n, seed=0, index=0):
    """A seeded permutation of n rows (used to derive distinct experts from a few
    independently drawn ones without drawing every expert in full)."""
    return rng(seed, MISC, index).permutation(n)
