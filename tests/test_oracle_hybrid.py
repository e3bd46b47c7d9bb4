"""Pins for the oracle's hybrid cache (CPU only): with nothing compressed it
is textbook attention on the unquantised K and V; with an empty buffer it is
the compressed cache's decode; tokens move from the buffer to the compressed
state in whole buffers."""
import math

import numpy as np
import pytest

from oracle import attention, codec, hybrid, quant


@pytest.fixture
def data():
    rng = np.random.default_rng(2)
    B, Hkv, Hq, N, d = 3, 2, 4, 70, 64
    k = rng.standard_normal((B, Hkv, N, d)) * 0.02
    v = rng.standard_normal((B, Hkv, N, d)) * 0.02
    q = rng.standard_normal((B, Hq, 2, d)) * 0.7
    kc, vc = codec.make_codec(d, 3, 0, codec.MODE_PROD), codec.make_codec(d, 2, 1, codec.MODE_MSE)
    return k, v, q, kc, vc, 1 / math.sqrt(d)


def test_compressed_length_moves_whole_buffers():
    assert [hybrid.compressed_length(n, 16) for n in (0, 1, 15, 16, 17, 31, 32, 33)] == [0, 0, 0, 16, 16, 16, 32, 32]


def test_nothing_compressed_is_exact_attention(data):
    k, v, q, kc, vc, sc = data
    lens = [70, 5, 33]
    got = hybrid.hybrid_decode(q, k, v, lens, 128, kc, vc, sc)     # every N < buffer size
    # textbook softmax attention, written out here independently
    want = np.zeros_like(got)
    for b in range(3):
        for h in range(4):
            for i in range(2):
                cnt = lens[b] - 2 + i + 1
                s = (k[b, h // 2, :cnt] @ q[b, h, i]) * sc
                p = np.exp(s - s.max())
                want[b, h, i] = (p / p.sum()) @ v[b, h // 2, :cnt]
    assert np.allclose(got, want, rtol=1e-12, atol=1e-15)


def test_empty_buffer_is_the_compressed_decode(data):
    k, v, q, kc, vc, sc = data
    lens = [64, 32, 48]                                              # multiples of 16: nothing buffered
    got = hybrid.hybrid_decode(q, k, v, lens, 16, kc, vc, sc)
    ks, vs = quant.quantize(k, kc), quant.quantize(v, vc)
    want = attention.decode_attention_rotated(q, ks, kc, vs, vc, np.array(lens), sc)
    assert np.abs(got - want).max() <= 1e-12 * np.abs(want).max()


def test_buffered_tokens_are_exact_and_compressed_ones_quantised(data):
    """Changing a buffered token's value changes the output exactly as exact
    attention would; changing a compressed token changes it only through its
    quantised value."""
    k, v, q, kc, vc, sc = data
    lens = [40, 40, 40]
    base = hybrid.hybrid_decode(q, k, v, lens, 16, kc, vc, sc)      # 32 compressed, 8 buffered
    v2 = v.copy()
    v2[:, :, 35] += 0.01                                             # a buffered token
    moved = hybrid.hybrid_decode(q, k, v2, lens, 16, kc, vc, sc)
    kk = k.copy()
    ks = quant.dequantize_state(quant.quantize(k[:, :, :32], kc), kc)
    vq = quant.dequantize_state(quant.quantize(v[:, :, :32], vc), vc)
    kk[:, :, :32] = ks
    vv = v2.copy()
    vv[:, :, :32] = vq
    assert np.allclose(moved, attention.decode_attention(q, kk, vv, lens, sc), rtol=1e-12, atol=1e-15)
    assert not np.allclose(moved, base)
