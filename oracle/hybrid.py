"""Hybrid cache: a recent-token buffer in front of the compressed state (test
infrastructure only).

What the pages show: "turboquant validate_moe_phase2.py", Test 5 builds its
caches with ``buffer_size=128`` and reads scores for every cached token after
``prefill``; the page's commit note names "hybrid decode".  They give no
further semantics.  Reading taken (the plainest one): the most recent tokens
of a sequence stay unquantised in a buffer of ``buffer_size`` tokens; when the
buffer is full, all of its tokens are quantised into the compressed state (at
its written end) and the buffer empties.  A sequence of N tokens therefore
holds tokens 0 .. Nc-1, Nc = floor(N / B) * B, compressed and tokens Nc .. N-1
unquantised, whatever the order of its appends; decode attends over all N
tokens with one softmax (the causal rule for the q_len new tokens is that of
every decode: row i sees t <= N - q_len + i), compressed tokens through their
codes and buffered tokens exactly.
"""
from __future__ import annotations

import numpy as np

from . import attention, quant
from .codec import Codec


def compressed_length(n: int, buffer_size: int) -> int:
    return (int(n) // int(buffer_size)) * int(buffer_size)


def hybrid_decode(q, k, v, lens, buffer_size: int, kc: Codec, vc: Codec, scale: float) -> np.ndarray:
    """Decode attention of a batch of hybrid caches, by brute force.

    q [B, Hq, q_len, d]; k, v [B, Hkv, N, d] every sequence's tokens
    (unquantised inputs); sequence b holds lens[b] of them.  Its first
    compressed_length(lens[b]) tokens are taken quantised and dequantised,
    the rest as they are; then plain softmax attention over the lot."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    kk, vv = k.copy(), v.copy()
    for b, n in enumerate(lens):
        nc = compressed_length(n, buffer_size)
        if nc:
            kk[b, :, :nc] = quant.dequantize_state(quant.quantize(k[b:b + 1, :, :nc], kc), kc)[0]
            vv[b, :, :nc] = quant.dequantize_state(quant.quantize(v[b:b + 1, :, :nc], vc), vc)[0]
    return attention.decode_attention(q, kk, vv, lens, scale)
