"""The packed index layout (test infrastructure only).

The pages fix the packed width: a state of d-dimensional vectors quantised to
b bits stores W = ceil(d*b/32) uint32 words per vector ("omlx
turboquant_kv.py", ``_infer_head_dim``), i.e. a dense packing with no padding
bits.  They do not fix the bit order.  Reading taken (head_dim is a multiple
of 32, so every 32 coordinates own exactly b words):

* b in {1, 2, 4}: an LSB-first stream.  Index j occupies bits
  [b*j, b*j + b) of the stream; stream bit k is bit (k mod 32) of word
  floor(k / 32).  No index straddles two words.
* b = 3: each group of 32 coordinates (j = 32*G + r) owns the three words
  X = 3G, Y = 3G + 1, Z = 3G + 2.  Write r = 4*a + k with byte lane
  k = r mod 4 and quad a = r div 4; every field of coordinate r lives in byte
  k of its word (bits 8k .. 8k+7):

      quad a   field location inside byte k
      0        X bits 0-2
      1        X bits 3-5
      2        X bits 6-7 (index bits 0-1) and Z bit 6 (index bit 2)
      3        Y bits 0-2
      4        Y bits 3-5
      5        Y bits 6-7 (index bits 0-1) and Z bit 7 (index bit 2)
      6        Z bits 0-2
      7        Z bits 3-5

  (Each byte of X, Y and Z then holds fields of four coordinates with the same
  byte lane, so one shift and one mask expose four indices at once.)

The QJL sign words of the Prod state use the b = 1 stream: bit j is
coordinate j.  The functions below follow the table literally, one
coordinate at a time.
"""
from __future__ import annotations

import numpy as np

_QUAD3 = {
    0: [(0, 0, 3, 0)],
    1: [(0, 3, 3, 0)],
    2: [(0, 6, 2, 0), (2, 6, 1, 2)],
    3: [(1, 0, 3, 0)],
    4: [(1, 3, 3, 0)],
    5: [(1, 6, 2, 0), (2, 7, 1, 2)],
    6: [(2, 0, 3, 0)],
    7: [(2, 3, 3, 0)],
}


def words_per_vector(d: int, b: int) -> int:
    """W = ceil(d * b / 32)."""
    return (d * b + 31) // 32


def field_pieces(b: int, j: int):
    """Where the bits of coordinate j's b-bit index live.

    Returns a list of (word, bit, nbits, src) pieces: index bits
    [src, src + nbits) are stored at bits [bit, bit + nbits) of word ``word``.
    """
    if b in (1, 2, 4):
        k = b * j
        return [(k // 32, k % 32, b, 0)]
    if b == 3:
        g, r = divmod(j, 32)
        a, k = divmod(r, 4)
        return [(3 * g + w, 8 * k + bit, n, src) for (w, bit, n, src) in _QUAD3[a]]
    raise ValueError("packed indices use 1..4 bits")


def pack(idx: np.ndarray, b: int) -> np.ndarray:
    """Pack integer indices [..., d] (each < 2**b) into uint32 words [..., W]."""
    idx = np.asarray(idx, dtype=np.int64)
    d = idx.shape[-1]
    if np.any(idx < 0) or np.any(idx >= (1 << b)):
        raise ValueError("index out of range for the bit width")
    out = np.zeros(idx.shape[:-1] + (words_per_vector(d, b),), dtype=np.uint64)
    for j in range(d):
        for (w, bit, n, src) in field_pieces(b, j):
            field = (idx[..., j] >> src) & ((1 << n) - 1)
            out[..., w] |= (field.astype(np.uint64) << np.uint64(bit))
    return out.astype(np.uint32)


def unpack(words: np.ndarray, b: int, d: int) -> np.ndarray:
    """Inverse of :func:`pack`: uint32 words [..., W] -> int64 indices [..., d]."""
    words = np.asarray(words, dtype=np.uint64)
    out = np.zeros(words.shape[:-1] + (d,), dtype=np.int64)
    for j in range(d):
        for (w, bit, n, src) in field_pieces(b, j):
            field = (words[..., w] >> np.uint64(bit)) & np.uint64((1 << n) - 1)
            out[..., j] |= field.astype(np.int64) << src
    return out
