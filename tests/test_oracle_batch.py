"""Pins for the oracle's batch bookkeeping (CPU only): the list operations
against what they must mean for attention -- every sequence's decode depends
on its own tokens only."""
import math

import numpy as np
import pytest

from oracle import attention, batch, codec, quant


def _inputs(rng, lens, H=2, d=64):
    return [rng.standard_normal((H, n, d)) * 0.02 for n in lens]


def _decode(kb, vb, q, cap):
    ka, lens = batch.padded(kb, cap)
    va, _ = batch.padded(vb, cap)
    return attention.decode_attention_rotated(q, batch.unpacked(ka, kb.codec), kb.codec, batch.unpacked(va, vb.codec),
                                              vb.codec, lens, 1 / math.sqrt(kb.codec.head_dim))


@pytest.fixture
def setup():
    rng = np.random.default_rng(0)
    kc, vc = codec.make_codec(64, 3, 0, codec.MODE_PROD), codec.make_codec(64, 2, 1, codec.MODE_MSE)
    lens = [9, 30, 1, 17]
    xs_k, xs_v = _inputs(rng, lens), _inputs(rng, lens)
    q = rng.standard_normal((4, 4, 1, 64)) * 0.5
    return rng, kc, vc, lens, xs_k, xs_v, q


def test_filter_and_merge_select_and_join_rows(setup):
    rng, kc, vc, lens, xs_k, xs_v, q = setup
    K, V = batch.from_inputs(xs_k, kc), batch.from_inputs(xs_v, vc)
    full = _decode(K, V, q, 32)
    keep = [3, 1]
    part = _decode(batch.filter_rows(K, keep), batch.filter_rows(V, keep), q[keep], 32)
    assert np.array_equal(part, full[keep])            # rows are independent: identical floats
    # extract every row and merge them back: the original batch
    rows = [batch.extract(K, b, 0, n) for b, n in enumerate(lens)]
    back = batch.merge(*rows)
    assert all(np.array_equal(a[k], b[k]) for a, b in zip(back.seqs, K.seqs) for k in a)
    # a filtered batch quantises exactly like a batch built from those inputs
    direct = batch.from_inputs([xs_k[i] for i in keep], kc)
    assert all(np.array_equal(a[k], b[k]) for a, b in zip(direct.seqs, batch.filter_rows(K, keep).seqs) for k in a)


def test_append_after_filter_lands_at_each_rows_own_end(setup):
    """The regression the pages record: after a filter, the write position of
    a row must be that row's own end, not an offset taken from another row."""
    rng, kc, vc, lens, xs_k, xs_v, q = setup
    K = batch.from_inputs(xs_k, kc)
    keep = [3, 0]
    new = [rng.standard_normal((2, 2, 64)) * 0.02 for _ in keep]
    after = batch.append(batch.filter_rows(K, keep), new)
    # the same as quantising each surviving sequence's whole token list
    truth = batch.from_inputs([np.concatenate([xs_k[i], t], axis=1) for i, t in zip(keep, new)], kc)
    for a, b in zip(after.seqs, truth.seqs):
        for k in a:
            assert np.array_equal(a[k], b[k])
    assert list(after.lens) == [lens[3] + 2, lens[0] + 2]


def test_capacity_slots_are_never_attended(setup):
    rng, kc, vc, lens, xs_k, xs_v, q = setup
    K, V = batch.from_inputs(xs_k, kc), batch.from_inputs(xs_v, vc)
    ka, ln = batch.padded(K, 40, fill=0)
    kg, _ = batch.padded(K, 40, fill=0)
    for k in kg:       # garbage in every slot past each length
        for b, n in enumerate(ln):
            kg[k][b, :, n:] = (rng.integers(0, 2**31, kg[k][b, :, n:].shape) if kg[k].dtype.kind in "ui"
                               else rng.standard_normal(kg[k][b, :, n:].shape) * 1e3)
    va, _ = batch.padded(V, 40)
    sc = 1 / math.sqrt(64)
    a = attention.decode_attention_rotated(q, batch.unpacked(ka, kc), kc, batch.unpacked(va, vc), vc, ln, sc)
    b = attention.decode_attention_rotated(q, batch.unpacked(kg, kc), kc, batch.unpacked(va, vc), vc, ln, sc)
    assert np.array_equal(a, b)


def test_trim_and_short_rows(setup):
    """Trimming is a length change; a 1-token row next to long ones decodes its
    own token (no left-padded row attends to nothing)."""
    rng, kc, vc, lens, xs_k, xs_v, q = setup
    K, V = batch.from_inputs(xs_k, kc), batch.from_inputs(xs_v, vc)
    t = batch.trim(K, 1, 5)
    assert list(t.lens) == [9, 5, 1, 17]
    out = _decode(K, V, q, 32)
    vdeq = quant.dequantize_state(batch.unpacked({k: v[None] for k, v in V.seqs[2].items()}, vc), vc)[0]
    assert np.allclose(out[2, 2:4, 0], vdeq[1, 0][None], rtol=0, atol=1e-15)   # N = 1: the value itself


def test_merge_refuses_codecs_of_different_bits_or_seed(setup):
    rng, kc, vc, lens, xs_k, xs_v, q = setup
    K = batch.from_inputs(xs_k[:1], kc)
    other_seed = batch.from_inputs(xs_k[:1], codec.make_codec(64, 3, 5, codec.MODE_PROD))
    other_bits = batch.from_inputs(xs_k[:1], codec.make_codec(64, 4, 0, codec.MODE_PROD))
    for other in (other_seed, other_bits):
        with pytest.raises(ValueError):
            batch.merge(K, other)
    assert len(batch.merge(K, K).seqs) == 2
