"""Decode attention over a compressed KV cache (test infrastructure only).

What is computed ("turboquant validate_moe_phase2.py", Tests 1 and 5: scores
scaled by 1/sqrt(head_dim), softmax over the cached tokens, weights applied to
the values, outputs compared in the original domain; "omlx turboquant_kv.py",
``make_mask``: new tokens see the cache causally):

  For sequence b with attended length N_b, query head h (KV head g = h div G,
  G = Hq / Hkv -- grouped-query attention with contiguous groups) and query
  row i < q_len, the visible tokens are t <= N_b - q_len + i (the q_len new
  tokens were appended before the call and are counted in N_b).
      s_t = scale * score(q, K_t),  p = softmax(s over visible t),
      out = sum_t p_t V~_t  (original domain, float64).
  A row with no visible token outputs zeros.

Two independent evaluations are provided:
  * :func:`decode_attention` -- brute force on dequantised K~ and V~;
  * :func:`decode_attention_rotated` -- scores from the rotated query against
    centroid values (plus the QJL term), values accumulated in the rotated
    domain and rotated back once per row.
They agree to rounding (about 1e-12 relative).  :func:`reference_attention`
is the same softmax attention on unquantised K and V, used for the quality
(cosine-similarity) report.
"""
from __future__ import annotations

import numpy as np

from . import quant
from .codec import MODE_GROUP, MODE_MSE, MODE_PROD, MODE_SPLIT, Codec


def _visible(n_b: int, q_len: int, i: int) -> int:
    """Number of visible tokens for row i (tokens 0 .. count-1)."""
    return max(0, min(n_b, n_b - q_len + i + 1))


def _softmax_weights(s: np.ndarray) -> np.ndarray:
    m = np.max(s)
    e = np.exp(s - m)
    return e / np.sum(e)


def decode_attention(q, k_deq, v_deq, lens, scale: float) -> np.ndarray:
    """Brute force.  q [B, Hq, q_len, d]; k_deq, v_deq [B, Hkv, N, d]."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, q_len, d = q.shape
    Hkv = k_deq.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, q_len, d), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(q_len):
                cnt = _visible(int(lens[b]), q_len, i)
                if cnt == 0:
                    continue
                s = scale * (np.asarray(k_deq[b, g, :cnt], dtype=np.float64) @ q[b, h, i])
                p = _softmax_weights(s)
                out[b, h, i] = p @ np.asarray(v_deq[b, g, :cnt], dtype=np.float64)
    return out


def reference_attention(q, k, v, lens, scale: float) -> np.ndarray:
    """Exact attention on unquantised K and V (float64)."""
    return decode_attention(q, np.asarray(k, dtype=np.float64), np.asarray(v, dtype=np.float64), lens, scale)


def key_scores_rotated(qrow: np.ndarray, kstate: dict, kc: Codec, cnt: int) -> np.ndarray:
    """score(q, K_t) for t < cnt from the rotated query (no K reconstruction)."""
    if kc.mode == MODE_SPLIT:
        # the sum of the two parts' scores, each against its own rotated query
        lo = {"idx": kstate["idx"][..., :kc.d_lo], "norm": kstate["norm"]}
        hi = {"idx": kstate["idx"][..., kc.d_lo:], "norm": kstate["rnorm"]}
        return (key_scores_rotated(qrow[:kc.d_lo], lo, kc.low, cnt) +
                key_scores_rotated(qrow[kc.d_lo:], hi, kc.high, cnt))
    q_rot = kc.rot @ qrow                                  # Pi q
    cv = kc.centroids[kstate["idx"][:cnt]]                 # [cnt, d]
    s = np.asarray(kstate["norm"][:cnt], dtype=np.float64) * (cv @ q_rot)
    if kc.mode == MODE_PROD:
        q_s = kc.sketch @ q_rot                            # S Pi q
        sigma = 2.0 * np.asarray(kstate["sign_bits"][:cnt], dtype=np.float64) - 1.0
        s = s + quant.qjl_constant(kc.head_dim) * np.asarray(kstate["rnorm"][:cnt], dtype=np.float64) * (sigma @ q_s)
    return s


def value_accumulate_rotated(p: np.ndarray, vstate: dict, vc: Codec, cnt: int) -> np.ndarray:
    """sum_t p_t V~_t, accumulated in the rotated domain for MSE values."""
    if vc.mode == MODE_GROUP:
        return p @ quant.dequantize_group(vstate["q"][:cnt], vstate["scale"][:cnt], vstate["min"][:cnt])
    if vc.mode == MODE_SPLIT:
        lo = {"idx": vstate["idx"][..., :vc.d_lo], "norm": vstate["norm"]}
        hi = {"idx": vstate["idx"][..., vc.d_lo:], "norm": vstate["rnorm"]}
        return np.concatenate([value_accumulate_rotated(p, lo, vc.low, cnt),
                               value_accumulate_rotated(p, hi, vc.high, cnt)])
    assert vc.mode == MODE_MSE
    w = p * np.asarray(vstate["norm"][:cnt], dtype=np.float64)
    o_rot = w @ vc.centroids[vstate["idx"][:cnt]]          # rotated domain
    return vc.rot.T @ o_rot                                 # one inverse rotation


def _slice(state: dict, b: int, g: int) -> dict:
    return {k: (v[b, g] if isinstance(v, np.ndarray) and v.ndim >= 2 else v) for k, v in state.items()}


def decode_attention_rotated(q, kstate: dict, kc: Codec, vstate: dict, vc: Codec, lens, scale: float) -> np.ndarray:
    """Rotated-domain evaluation.  States hold arrays shaped [B, Hkv, N, ...]."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, q_len, d = q.shape
    Hkv = (kstate["idx"] if "idx" in kstate else kstate["q"]).shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, q_len, d), dtype=np.float64)
    for b in range(B):
        for g in range(Hkv):
            ks, vs = _slice(kstate, b, g), _slice(vstate, b, g)
            for hh in range(G):
                h = g * G + hh
                for i in range(q_len):
                    cnt = _visible(int(lens[b]), q_len, i)
                    if cnt == 0:
                        continue
                    s = scale * key_scores_rotated(q[b, h, i], ks, kc, cnt)
                    p = _softmax_weights(s)
                    out[b, h, i] = value_accumulate_rotated(p, vs, vc, cnt)
    return out


def dequantize_cache(state: dict, codec: Codec) -> np.ndarray:
    """Dequantise a whole [B, Hkv, N, ...] state to [B, Hkv, N, d]."""
    return quant.dequantize_state(state, codec)
