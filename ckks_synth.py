"""Seeded synthetic inputs for the RNS-CKKS rotation hot path.

This module is the only code shared by the CPU oracle side and the GPU side.
It draws random numbers and nothing else: it holds no modular arithmetic, no
NTT, no CRT and no part of the scheme.  Every random quantity the scheme needs
(secret key, error terms, uniform ring elements, slot values, rotation
offsets) is drawn here and handed to whichever side consumes it, so both sides
see the same words.

Streams are numpy PCG64 generators keyed by (seed, tag), where the tag names
the purpose (for instance ``"evk/3"`` or ``"ct/a"``).  The same (seed, tag)
always yields the same numbers, independent of the order in which other
streams are drawn.
"""
from __future__ import annotations

import zlib

import numpy as np

__all__ = [
    "stream",
    "uniform_limbs",
    "top_limbs",
    "ternary_secret",
    "rounded_gaussian",
    "uniform_slots",
    "normal_values",
    "distinct_offsets",
]


def stream(seed: int, tag: str) -> np.random.Generator:
    """Independent generator for one purpose (``tag``) under one seed."""
    key = zlib.crc32(tag.encode("utf-8"))
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), key])))


def uniform_limbs(rng: np.random.Generator, moduli, n: int, lead=()) -> np.ndarray:
    """uint64 array of shape ``lead + (len(moduli), n)``; limb t is uniform in [0, moduli[t])."""
    lead = tuple(lead)
    out = np.empty(lead + (len(moduli), n), dtype=np.uint64)
    for t, m in enumerate(moduli):
        out[..., t, :] = rng.integers(0, int(m), size=lead + (n,), dtype=np.uint64)
    return out


def top_limbs(rng: np.random.Generator, moduli, n: int, lead=(), span: int = 1 << 16) -> np.ndarray:
    """Like uniform_limbs, but every word of limb t lies in [moduli[t] - span, moduli[t]): the top of
    the residue range, where lazy (partially reduced) intermediate values come closest to overflowing."""
    lead = tuple(lead)
    out = np.empty(lead + (len(moduli), n), dtype=np.uint64)
    for t, m in enumerate(moduli):
        out[..., t, :] = np.uint64(int(m) - 1) - rng.integers(0, min(span, int(m)), size=lead + (n,), dtype=np.uint64)
    return out


def ternary_secret(rng: np.random.Generator, n: int, h: int) -> np.ndarray:
    """int8 vector of length n with exactly h entries in {-1, +1} at distinct positions."""
    if not 0 <= h <= n:
        raise ValueError("hamming weight out of range")
    s = np.zeros(n, dtype=np.int8)
    pos = rng.choice(n, size=h, replace=False)
    s[pos] = rng.choice(np.array([-1, 1], dtype=np.int8), size=h)
    return s


def rounded_gaussian(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    """int64 samples round(N(0, sigma^2)); no tail cut (a benchmark sampler, not a secure one)."""
    return np.rint(rng.normal(0.0, sigma, size=shape)).astype(np.int64)


def uniform_slots(rng: np.random.Generator, n: int, complex_values: bool = True, lo=-1.0, hi=1.0) -> np.ndarray:
    """complex128 slot vector; real (and, if requested, imaginary) parts uniform in [lo, hi)."""
    re = rng.uniform(lo, hi, size=n)
    im = rng.uniform(lo, hi, size=n) if complex_values else np.zeros(n)
    return (re + 1j * im).astype(np.complex128)


def normal_values(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    """float64 samples N(0, std^2)."""
    return rng.normal(0.0, std, size=shape)


def distinct_offsets(rng: np.random.Generator, count: int, lo: int, hi: int) -> np.ndarray:
    """``count`` distinct integers drawn uniformly without replacement from [lo, hi]."""
    return (rng.choice(hi - lo + 1, size=count, replace=False) + lo).astype(np.int64)


# ---------------------------------------------------------------------------
# Workload recipes (plain numbers; primes are derived by each side from these)
# ---------------------------------------------------------------------------

CONFIGS = {
    # Tiny single rotation: 2048 complex slots, rotate by 1 and by 7.
    "C1": dict(log_n=12, L=4, q_bits=30, K=1, p_bits=60, dnum=4, h=64, sigma=3.2, scale=2.0 ** 25,
               complex_slots=True, rotations=(1, 7), batch=1),
    # Batched NTT / iNTT: 16 polynomials x 24 limbs of 2^16 words.
    "C2": dict(log_n=16, L=24, q_bits=54, K=0, p_bits=60, dnum=1, npoly=16),
    # HRot throughput: 32 ciphertexts at the top level, each with its own offset and key.
    "C3": dict(log_n=16, L=24, q_bits=54, K=8, p_bits=60, dnum=3, h=192, sigma=3.2, scale=2.0 ** 40,
               complex_slots=False, batch=32, offset_range=(1, 32767)),
    # FFN-style BSGS ct x pt matvec at level 12 (13 primes).
    "C4": dict(log_n=16, L=24, q_bits=54, K=8, p_bits=60, dnum=3, h=192, sigma=3.2, scale=2.0 ** 40,
               level=12, n_in=3, n_out=12, n1=8, n2=8, w_std=0.02, w_rows=768, w_cols=3072),
    # Attention-shaped batch: 48 ct x ct products, relinearise, rescale, rotate-and-sum over 15 offsets.
    "C5": dict(log_n=16, L=24, q_bits=54, K=8, p_bits=60, dnum=3, h=192, sigma=3.2, scale=2.0 ** 40,
               batch=48, tokens=2048, hidden=768, rotsum_steps=15),
    # Attention output A x V with encrypted weights: V as 3 ciphertexts (128 tokens x 768 hidden),
    # 3 outputs, 64 ciphertext diagonals per (output, input) block, BSGS 8 x 8 at level 12.
    "AV": dict(log_n=16, L=24, q_bits=54, K=8, p_bits=60, dnum=3, h=192, sigma=3.2, scale=2.0 ** 40,
               level=12, n_in=3, n_out=3, n1=8, n2=8, tokens=128, hidden=768),
}
