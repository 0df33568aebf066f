"""Seeded random tensors with the value laws of the workloads.

Recipe (all draws from numpy's PCG64 bit generator, seeded per tensor):

* normal fp16 tensor: z ~ N(0, 1) drawn as float32, multiplied by sigma in
  float32, rounded to fp16 (round-to-nearest-even, numpy's cast).
* activation tensor [M][K]: z ~ N(0, 1) float32 per element times a per-channel
  multiplier c_k (float32), rounded to fp16.  c_k is the product of
    - a lognormal magnitude m_k = exp(u_k), u_k ~ N(0, 1), when requested, and
    - 20 on a seeded set of round(0.01 * K) "salient" channels, else 1.
  The salient set mimics the heavy-tailed activation channels that the AWQ
  summary page (fdeinterviews.com, paragraph 2) says carry the most important
  features; 1% is the top of the 0.1%..1% range it quotes.

Rows are drawn in chunks of 4096 so that the biggest tensors (65,536 x 11,008)
never need a float32 copy of the whole matrix.
"""
from __future__ import annotations

import numpy as np

_CHUNK_ROWS = 4096


def rng(seed: int) -> np.random.Generator:
    """A PCG64 generator for one tensor."""
    return np.random.Generator(np.random.PCG64(int(seed)))


def normal_fp16(shape, sigma: float, seed: int) -> np.ndarray:
    """fp16 array with elements fp16(sigma * z), z ~ N(0, 1) drawn in float32."""
    g = rng(seed)
    shape = tuple(int(d) for d in shape)
    out = np.empty(shape, dtype=np.float16)
    flat = out.reshape(-1) if out.size else out
    n = flat.size
    step = _CHUNK_ROWS * 4096
    for start in range(0, n, step):
        stop = min(n, start + step)
        z = g.standard_normal(stop - start, dtype=np.float32)
        z *= np.float32(sigma)
        flat[start:stop] = z.astype(np.float16)
    return out


def outlier_channels(K: int, frac: float, seed: int) -> np.ndarray:
    """Sorted indices of round(frac * K) distinct channels, chosen by a seeded permutation."""
    count = int(round(frac * K))
    if count <= 0:
        return np.zeros(0, dtype=np.int64)
    perm = rng(seed).permutation(K)
    return np.sort(perm[:count]).astype(np.int64)


def lognormal_profile(K: int, seed: int) -> np.ndarray:
    """Per-channel magnitudes m_k = exp(u_k), u_k ~ N(0, 1), as float32."""
    u = rng(seed).standard_normal(K)  # float64
    return np.exp(u).astype(np.float32)


def activations_fp16(
    M: int,
    K: int,
    seed: int,
    outlier_frac: float = 0.01,
    outlier_mult: float = 20.0,
    lognormal: bool = False,
) -> np.ndarray:
    """[M][K] fp16 activations: fp16(z_tk * c_k) with the channel multipliers above.

    Sub-seeds: seed drives z, seed + 7919 the salient set, seed + 104729 the
    lognormal profile, so that changing one law does not reshuffle the others.
    """
    mult = np.ones(K, dtype=np.float32)
    if lognormal:
        mult *= lognormal_profile(K, seed + 104729)
    idx = outlier_channels(K, outlier_frac, seed + 7919)
    mult[idx] *= np.float32(outlier_mult)
    g = rng(seed)
    out = np.empty((M, K), dtype=np.float16)
    for r0 in range(0, M, _CHUNK_ROWS):
        r1 = min(M, r0 + _CHUNK_ROWS)
        z = g.standard_normal((r1 - r0, K), dtype=np.float32)
        z *= mult[None, :]
        out[r0:r1] = z.astype(np.float16)
    return out
