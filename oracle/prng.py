"""Seeded standard normals for the codec (test infrastructure only).

The pages fix that a codec is a deterministic function of (head_dim, bits,
seed) ("omlx turboquant_kv.py", ``_rebuild_codecs``: the rotation and codebook
are rebuilt from those three values alone), but not which generator draws the
Gaussian matrices.  Reading taken: a counter-based SplitMix64 generator
(Steele, Lea & Flood, "Fast splittable pseudorandom number generators",
OOPSLA 2014) feeding the Box-Muller transform (Box & Muller, 1958).

SplitMix64 as a counter-based generator
    state_k = start + (k + 1) * GAMMA            (mod 2**64), k = 0, 1, ...
    z = state_k
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9       (mod 2**64)
    z = (z ^ (z >> 27)) * 0x94D049BB133111EB       (mod 2**64)
    out_k = z ^ (z >> 31)
with GAMMA = 0x9E3779B97F4A7C15.  A stream ``s`` of seed ``seed`` starts at
``start = seed XOR (s * GAMMA mod 2**64)``; stream 0 draws the rotation's
Gaussian matrix, stream 1 the QJL sketch.

Uniforms in (0, 1]:  u_k = ((out_k >> 11) + 1) / 2**53.
Box-Muller on consecutive pairs (u_2i, u_2i+1):
    r = sqrt(-2 ln u_2i),  theta = 2 pi u_2i+1,
    g_2i = r cos(theta),   g_2i+1 = r sin(theta).
Matrices are filled in row-major order.
"""
from __future__ import annotations

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

STREAM_ROTATION = 0
STREAM_SKETCH = 1
STREAM_SPLIT_HIGH = 2   # rotation of the high part of a split codec


def stream_start(seed: int, stream: int) -> int:
    """Starting state of stream ``stream`` of ``seed``."""
    return (int(seed) & MASK64) ^ ((int(stream) * GAMMA) & MASK64)


def splitmix64(start: int, n: int) -> np.ndarray:
    """The first ``n`` SplitMix64 outputs after ``start`` as uint64."""
    k = np.arange(1, n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(start) + k * np.uint64(GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(MIX1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(MIX2)
        z = z ^ (z >> np.uint64(31))
    return z


def splitmix64_scalar(start: int, k: int) -> int:
    """Output ``k`` (0-based) of the stream, in plain Python integers."""
    z = (start + (k + 1) * GAMMA) & MASK64
    z = ((z ^ (z >> 30)) * MIX1) & MASK64
    z = ((z ^ (z >> 27)) * MIX2) & MASK64
    return z ^ (z >> 31)


def uniforms(start: int, n: int) -> np.ndarray:
    """``n`` uniforms in (0, 1] (float64, 53 random bits each)."""
    z = splitmix64(start, n)
    return ((z >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)


def normals(seed: int, stream: int, n: int) -> np.ndarray:
    """``n`` standard normals (n even) of stream ``stream`` of ``seed``."""
    if n % 2:
        raise ValueError("normals are drawn in Box-Muller pairs; n must be even")
    u = uniforms(stream_start(seed, stream), n)
    u1, u2 = u[0::2], u[1::2]
    r = np.sqrt(-2.0 * np.log(u1))
    theta = 2.0 * np.pi * u2
    g = np.empty(n, dtype=np.float64)
    g[0::2] = r * np.cos(theta)
    g[1::2] = r * np.sin(theta)
    return g


def gaussian_matrix(seed: int, stream: int, d: int) -> np.ndarray:
    """A d x d matrix of iid N(0, 1) entries, filled row-major."""
    return normals(seed, stream, d * d).reshape(d, d)
