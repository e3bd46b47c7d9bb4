"""Quantisers and dequantisers (test infrastructure only).

All arithmetic is float64 on the float32 values the state stores.  Inputs
``x`` are arrays [..., d] of float32 values (bf16 inputs are passed as their
exact float32 widening).

MSE state (``TurboQuantMSEState(norms, indices)``, "omlx turboquant_kv.py"):
    n = ||x||_2, u = Pi x / n, idx_j = #{k : u_j > b_k}  (a tie goes to the
    lower cell; n = 0 gives u = 0), stored as the float32 norm and the packed
    indices.  Dequantisation: x~ = n Pi^T c[idx] -- the three decompression
    steps of "lightning-mlx plan.md" (lookup, denormalise, inverse rotation).

Prod state (``TurboQuantProdState(norms, mse_indices, residual_norms,
qjl_signs)``; 3-bit keys are "MSE + QJL" per the commit note of
"turboquant validate_moe_phase2.py"):
    MSE stage at bits-1; rotated residual rho = Pi x - n^ c[idx] (n^ the
    stored norm, so rho = Pi (x - x~_mse)); gamma = ||rho||; z = S rho;
    sign bit_j = [z_j >= 0]; stored gamma as float32 and the sign bits.
    Inner-product estimator (reading: the QJL estimator, unbiased over S):
        <q, x> ~ n^ <Pi q, c[idx]> + gamma^ sqrt(pi/2)/d <S Pi q, sigma>,
    sigma_j = 2 bit_j - 1.

Group state (``quantize_values(v, bits, group_size=32)`` -> data, scales,
zeros; "turboquant validate_moe_phase2.py", Tests 2 and 5):
    per group of 32 consecutive coordinates of the unrotated vector:
    mn = min, mx = max, s = (mx - mn)/(2^b - 1),
    q = clip(rint((v - mn)/s), 0, 2^b - 1) with rint ties-to-even, q = 0 when
    mx = mn; stored float32 scale s and float32 minimum ("zeros") mn.
    Dequantisation: q s^ + mn.

Decision margins: where a float decides an integer the exact (float64) value
is returned with its distance to the decision threshold, so that a float32
implementation can be compared outside a window around the thresholds.
"""
from __future__ import annotations

import math

import numpy as np

from . import packing
from .codec import GROUP_SIZE, MODE_GROUP, MODE_MSE, MODE_PROD, MODE_SPLIT, Codec


def _f32(a) -> np.ndarray:
    """Round to float32 (nearest-even) and return as float64."""
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def mse_quantize(x: np.ndarray, codec: Codec) -> dict:
    """MSE stage.  Returns norm (float32 values), idx, packed words, u and the
    distance of each u_j to its nearest decision boundary."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1))
    y = x @ codec.rot.T                      # y = Pi x, row-vector form
    safe = np.where(n > 0.0, n, 1.0)
    u = np.where((n > 0.0)[..., None], y / safe[..., None], 0.0)
    idx = np.sum(u[..., None] > codec.boundaries, axis=-1)
    margin = np.min(np.abs(u[..., None] - codec.boundaries), axis=-1)
    return {
        "norm": _f32(n),
        "idx": idx,
        "words": packing.pack(idx, codec.mse_bits),
        "u": u,
        "margin": margin,
        "y": y,
    }


def prod_quantize(x: np.ndarray, codec: Codec) -> dict:
    """Prod (MSE at bits-1 + 1-bit QJL of the rotated residual)."""
    assert codec.mode == MODE_PROD
    m = mse_quantize(x, codec)
    rho = m["y"] - m["norm"][..., None] * codec.centroids[m["idx"]]
    gamma = np.sqrt(np.sum(rho * rho, axis=-1))
    z = rho @ codec.sketch.T                 # z = S rho
    bits = (z >= 0.0).astype(np.int64)
    d = codec.head_dim
    safe = np.where(gamma > 0.0, gamma, 1.0)
    zmargin = np.where((gamma > 0.0)[..., None], np.abs(z) / (math.sqrt(d) * safe[..., None]), np.inf)
    m.update({
        "rnorm": _f32(gamma),
        "sign_bits": bits,
        "sign_words": packing.pack(bits, 1),
        "z": z,
        "zmargin": zmargin,
    })
    return m


def group_quantize(v: np.ndarray, bits: int, group_size: int = GROUP_SIZE) -> dict:
    """Asymmetric min-max group quantisation of the unrotated vector."""
    v = np.asarray(v, dtype=np.float64)
    d = v.shape[-1]
    g = v.reshape(v.shape[:-1] + (d // group_size, group_size))
    mn = g.min(axis=-1)
    mx = g.max(axis=-1)
    rng = mx - mn
    top = (1 << bits) - 1
    safe = np.where(rng > 0.0, rng, 1.0)
    t = (g - mn[..., None]) * top / safe[..., None]
    q = np.clip(np.rint(t), 0, top)
    q = np.where((rng > 0.0)[..., None], q, 0.0).astype(np.int64)
    frac = t - np.floor(t)
    margin = np.where((rng > 0.0)[..., None], np.abs(frac - 0.5), np.inf)
    q = q.reshape(v.shape)
    return {
        "q": q,
        "words": packing.pack(q, bits),
        "scale": _f32(rng / top),
        "min": _f32(mn),
        "t": t.reshape(v.shape),
        "margin": margin.reshape(v.shape),
    }


def split_quantize(x: np.ndarray, codec) -> dict:
    """Split codec: the low channels through the low MSE codec, the high
    channels through the high one.  The stored layout is one token record: the
    low part's packed words then the high part's, the low norm ("norm") and
    the high norm ("rnorm"); margins and codes are the two parts' side by
    side."""
    x = np.asarray(x, dtype=np.float64)
    lo = mse_quantize(x[..., :codec.d_lo], codec.low)
    hi = mse_quantize(x[..., codec.d_lo:], codec.high)
    return {
        "low": lo, "high": hi,
        "words": np.concatenate([lo["words"], hi["words"]], axis=-1),
        "norm": lo["norm"], "rnorm": hi["norm"],
        "idx": np.concatenate([lo["idx"], hi["idx"]], axis=-1),
        "margin": np.concatenate([lo["margin"], hi["margin"]], axis=-1),
    }


def quantize(x: np.ndarray, codec: Codec) -> dict:
    if codec.mode == MODE_MSE:
        return mse_quantize(x, codec)
    if codec.mode == MODE_PROD:
        return prod_quantize(x, codec)
    if codec.mode == MODE_SPLIT:
        return split_quantize(x, codec)
    return group_quantize(x, codec.bits)


def qjl_constant(d: int) -> float:
    """sqrt(pi/2)/d, the scale that makes the sign estimator unbiased."""
    return math.sqrt(math.pi / 2.0) / d


def dequantize_mse(norm: np.ndarray, idx: np.ndarray, codec: Codec) -> np.ndarray:
    """x~ = n Pi^T c[idx] (row-vector form: n * (c[idx] @ Pi))."""
    return np.asarray(norm, dtype=np.float64)[..., None] * (codec.centroids[idx] @ codec.rot)


def dequantize_prod(norm, idx, rnorm, sign_bits, codec: Codec) -> np.ndarray:
    """x~ = Pi^T (n c[idx] + gamma sqrt(pi/2)/d S^T sigma)."""
    sigma = 2.0 * np.asarray(sign_bits, dtype=np.float64) - 1.0
    rot_dom = (np.asarray(norm, dtype=np.float64)[..., None] * codec.centroids[idx]
               + qjl_constant(codec.head_dim) * np.asarray(rnorm, dtype=np.float64)[..., None]
               * (sigma @ codec.sketch))
    return rot_dom @ codec.rot


def dequantize_group(q, scale, mn, group_size: int = GROUP_SIZE) -> np.ndarray:
    """q s + mn per group."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    s = np.repeat(np.asarray(scale, dtype=np.float64), group_size, axis=-1)
    m = np.repeat(np.asarray(mn, dtype=np.float64), group_size, axis=-1)
    assert s.shape[-1] == d
    return q * s + m


def dequantize_state(state: dict, codec: Codec) -> np.ndarray:
    """Dequantise a state dict as produced by :func:`quantize` (or one with the
    same keys read back from packed words)."""
    if codec.mode == MODE_MSE:
        return dequantize_mse(state["norm"], state["idx"], codec)
    if codec.mode == MODE_PROD:
        return dequantize_prod(state["norm"], state["idx"], state["rnorm"], state["sign_bits"], codec)
    if codec.mode == MODE_SPLIT:
        lo = dequantize_mse(state["norm"], state["idx"][..., :codec.d_lo], codec.low)
        hi = dequantize_mse(state["rnorm"], state["idx"][..., codec.d_lo:], codec.high)
        return np.concatenate([lo, hi], axis=-1)
    return dequantize_group(state["q"], state["scale"], state["min"])


def state_from_words(codec: Codec, words, norm=None, rnorm=None, sign_words=None,
                     scale=None, mn=None) -> dict:
    """Unpack a stored state (packed words + side data) into a state dict."""
    d = codec.head_dim
    if codec.mode == MODE_GROUP:
        return {"q": packing.unpack(words, codec.bits, d), "scale": scale, "min": mn}
    if codec.mode == MODE_SPLIT:
        w_lo = codec.d_lo * codec.low.bits // 32
        words = np.asarray(words)
        idx = np.concatenate([packing.unpack(words[..., :w_lo], codec.low.bits, codec.d_lo),
                              packing.unpack(words[..., w_lo:], codec.high.bits, codec.d_hi)], axis=-1)
        return {"idx": idx, "norm": norm, "rnorm": rnorm}
    st = {"idx": packing.unpack(words, codec.mse_bits, d), "norm": norm}
    if codec.mode == MODE_PROD:
        st["rnorm"] = rnorm
        st["sign_bits"] = packing.unpack(sign_words, 1, d)
    return st
