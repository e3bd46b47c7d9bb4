"""Batch bookkeeping on compressed caches (test infrastructure only).

What the pages show ("omlx turboquant_kv.py", ``BatchTurboQuantKVCache``):
batched requests are selected (``filter``), split off (``extract``) and joined
(``extend``, ``merge``) as whole rows of the packed state -- never
re-quantised -- along the batch axis (``_filter_state``,
``_concat_state_batch``); new tokens of each request are written at that
request's written end (``update_and_fetch``; the ``_phys_end`` note: a write
position derived from another row's offset overwrote live tokens after a
filter); only written tokens may be attended (the ``state`` note: capacity
columns exposed after the buffer grew); ``merge`` refuses caches whose codecs
differ in bits or seed.

Reading taken (the plainest one): a batch cache is a list of sequences, and
sequence b's cache is exactly the quantisation of its own token list, in
order, whatever happened to the batch around it.  Every operation below is
the list operation that statement implies, on the stored fields of the state
(packed words and side data):

  filter(keep)          the sequences keep[0], keep[1], ... in that order
  extract(b, s0, n)     tokens s0 .. s0+n-1 of sequence b, as a 1-sequence batch
  extend / merge        the sequences of several batches one after the other;
                        refused (ValueError) unless every codec has the same
                        head_dim, bits, mode and seed
  append(new)           sequence b gets the quantised new tokens after its own
                        last token
  trim(b, n)            sequence b keeps its first n tokens

``padded`` lays a batch out as the arrays [B, H, cap, ...] plus lengths that a
device cache holds; slots past a sequence's length are filled with
``fill`` (they are never attended).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List

import numpy as np

from . import quant
from .codec import MODE_GROUP, MODE_MSE, MODE_PROD, MODE_SPLIT, Codec

# the fields a cache stores per token-head, by mode (packing.pack output and
# float32 side data)
STORED = {
    MODE_MSE: ("words", "norm"),
    MODE_PROD: ("words", "norm", "rnorm", "sign_words"),
    MODE_GROUP: ("words", "scale", "min"),
    MODE_SPLIT: ("words", "norm", "rnorm"),
}


def stored(state: dict, codec: Codec) -> dict:
    """The stored fields of a state from :func:`oracle.quant.quantize`."""
    return {k: np.asarray(state[k]) for k in STORED[codec.mode]}


@dataclass
class Batch:
    """One compressed cache (K or V) of a batch: ``seqs[b]`` maps every
    stored field to an array [H, n_b, ...]."""
    codec: Codec
    seqs: List[dict] = field(default_factory=list)

    @property
    def lens(self) -> np.ndarray:
        return np.array([s["words"].shape[1] for s in self.seqs], dtype=np.int64)


def from_inputs(xs, codec: Codec) -> Batch:
    """Quantise each sequence's tokens (arrays [H, n_b, d])."""
    return Batch(codec, [stored({k: v[0] if isinstance(v, np.ndarray) else v
                                 for k, v in quant.quantize(np.asarray(x, dtype=np.float64)[None], codec).items()},
                                codec) for x in xs])


def filter_rows(batch: Batch, keep) -> Batch:
    return Batch(batch.codec, [batch.seqs[i] for i in keep])


def extract(batch: Batch, b: int, start: int, count: int) -> Batch:
    s = batch.seqs[b]
    if start < 0 or count < 0 or start + count > s["words"].shape[1]:
        raise ValueError("token range outside the sequence")
    return Batch(batch.codec, [{k: v[:, start:start + count] for k, v in s.items()}])


def _same_codec(a: Codec, b: Codec) -> bool:
    return (a.head_dim, a.bits, a.mode, a.seed) == (b.head_dim, b.bits, b.mode, b.seed)   # split: bits is the width


def merge(*batches: Batch) -> Batch:
    """extend and merge: the sequences of every batch in order."""
    first = batches[0].codec
    for bt in batches[1:]:
        if not _same_codec(first, bt.codec):
            raise ValueError("caches quantised with different head_dim, bits, mode or seed cannot be merged")
    return Batch(first, [s for bt in batches for s in bt.seqs])


def append(batch: Batch, new_tokens) -> Batch:
    """new_tokens[b]: array [H, t_b, d] of sequence b's new tokens."""
    fresh = from_inputs(new_tokens, batch.codec)
    return Batch(batch.codec, [{k: np.concatenate([s[k], t[k]], axis=1) for k in s}
                               for s, t in zip(batch.seqs, fresh.seqs)])


def trim(batch: Batch, b: int, n: int) -> Batch:
    seqs = list(batch.seqs)
    seqs[b] = {k: v[:, :n] for k, v in seqs[b].items()}
    return Batch(batch.codec, seqs)


def padded(batch: Batch, cap: int, fill=0):
    """Arrays [B, H, cap, ...] of every stored field (slots past a sequence's
    length set to ``fill``) and the lengths."""
    out = {}
    for k in STORED[batch.codec.mode]:
        ref = batch.seqs[0][k]
        a = np.full((len(batch.seqs), ref.shape[0], cap) + ref.shape[2:], fill, dtype=ref.dtype)
        for b, s in enumerate(batch.seqs):
            a[b, :, :s[k].shape[1]] = s[k]
        out[k] = a
    return out, batch.lens


def unpacked(arrays: dict, codec: Codec) -> dict:
    """A padded state in the form the oracle's decode reads (unpacked codes)."""
    if codec.mode == MODE_SPLIT:
        return quant.state_from_words(codec, arrays["words"], norm=arrays["norm"], rnorm=arrays["rnorm"])
    if codec.mode == MODE_GROUP:
        return quant.state_from_words(codec, arrays["words"], scale=arrays["scale"], mn=arrays["min"])
    return quant.state_from_words(codec, arrays["words"], norm=arrays["norm"], rnorm=arrays.get("rnorm"),
                                  sign_words=arrays.get("sign_words"))
