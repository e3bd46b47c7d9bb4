"""Pins for the oracle's decode attention (CPU only)."""
import math

import numpy as np
import pytest

from oracle import attention, codec, quant


def _random_cache(rng, B, Hkv, N, d, kc, vc):
    k = (rng.standard_normal((B, Hkv, N, d)) * 0.02).astype(np.float32)
    v = (rng.standard_normal((B, Hkv, N, d)) * 0.02).astype(np.float32)
    return k, v, quant.quantize(k, kc), quant.quantize(v, vc)


CASES = [
    # (d, kbits, kmode, vbits, vmode, Hq, Hkv, q_len)
    (32, 3, codec.MODE_MSE, 3, codec.MODE_MSE, 2, 1, 1),
    (64, 3, codec.MODE_PROD, 4, codec.MODE_MSE, 8, 2, 1),
    (128, 3, codec.MODE_PROD, 2, codec.MODE_GROUP, 4, 1, 1),
    (128, 3, codec.MODE_MSE, 3, codec.MODE_MSE, 4, 2, 2),
    (256, 3, codec.MODE_PROD, 2, codec.MODE_GROUP, 2, 1, 2),
]


@pytest.mark.parametrize("case", CASES)
def test_bruteforce_equals_rotated_domain(case):
    d, kb, km, vb, vm, Hq, Hkv, q_len = case
    rng = np.random.default_rng(d + kb)
    kc = codec.make_codec(d, kb, 0, km)
    vc = codec.make_codec(d, vb, 1, vm)
    B, N = 2, 40
    k, v, ks, vs = _random_cache(rng, B, Hkv, N, d, kc, vc)
    q = rng.standard_normal((B, Hq, q_len, d)) * 0.5
    lens = np.array([N, 17])
    scale = 1 / math.sqrt(d)
    a = attention.decode_attention(q, quant.dequantize_state(ks, kc), quant.dequantize_state(vs, vc), lens, scale)
    b = attention.decode_attention_rotated(q, ks, kc, vs, vc, lens, scale)
    assert np.abs(a - b).max() <= 1e-12 * np.abs(a).max()


def test_special_cases():
    rng = np.random.default_rng(1)
    d = 64
    kc = codec.make_codec(d, 3, 0, codec.MODE_MSE)
    vc = codec.make_codec(d, 3, 1, codec.MODE_MSE)
    k, v, ks, vs = _random_cache(rng, 1, 1, 30, d, kc, vc)
    kd, vd = quant.dequantize_state(ks, kc), quant.dequantize_state(vs, vc)
    q = rng.standard_normal((1, 1, 1, d))
    # one visible token: the output is that token's value
    out = attention.decode_attention(q, kd, vd, np.array([1]), 0.1)
    assert np.allclose(out[0, 0, 0], vd[0, 0, 0], rtol=0, atol=1e-15)
    # q = 0: uniform weights, the output is the mean value
    out = attention.decode_attention(np.zeros_like(q), kd, vd, np.array([30]), 0.1)
    assert np.allclose(out[0, 0, 0], vd[0, 0].mean(0), rtol=1e-12, atol=1e-16)
    # empty cache: zeros
    out = attention.decode_attention(q, kd, vd, np.array([0]), 0.1)
    assert np.all(out == 0)
    # permutation of the tokens does not change a q_len = 1 output
    perm = rng.permutation(30)
    a = attention.decode_attention(q, kd, vd, np.array([30]), 0.1)
    b = attention.decode_attention(q, kd[:, :, perm], vd[:, :, perm], np.array([30]), 0.1)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-16)


def test_causal_rows_for_two_new_tokens():
    rng = np.random.default_rng(2)
    d, N = 32, 12
    k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    q = rng.standard_normal((1, 1, 2, d))
    out = attention.reference_attention(q, k, v, np.array([N]), 0.3)
    # row 0 sees tokens 0..N-2 (the second new token is in the future), row 1 sees all
    for i, cnt in ((0, N - 1), (1, N)):
        s = 0.3 * (k[0, 0, :cnt] @ q[0, 0, i])
        p = np.exp(s - s.max())
        p /= p.sum()
        assert np.allclose(out[0, 0, i], p @ v[0, 0, :cnt], rtol=1e-13, atol=0)


def test_gqa_mapping_contiguous_groups():
    rng = np.random.default_rng(3)
    d, N = 32, 9
    k = rng.standard_normal((1, 2, N, d))
    v = rng.standard_normal((1, 2, N, d))
    q = rng.standard_normal((1, 4, 1, d))
    out = attention.reference_attention(q, k, v, np.array([N]), 0.2)
    for h in range(4):
        single = attention.reference_attention(q[:, h:h + 1], k[:, h // 2:h // 2 + 1], v[:, h // 2:h // 2 + 1], np.array([N]), 0.2)
        assert np.allclose(out[:, h], single[:, 0], rtol=1e-14, atol=0)


def test_quality_improves_with_bits():
    rng = np.random.default_rng(4)
    d, N = 128, 256
    k = (rng.standard_normal((1, 1, N, d))).astype(np.float32)
    v = (rng.standard_normal((1, 1, N, d))).astype(np.float32)
    q = rng.standard_normal((1, 1, 1, d)) * 2
    ref = attention.reference_attention(q, k, v, np.array([N]), 1 / math.sqrt(d))[0, 0, 0]
    cos = []
    for bits in (2, 3, 4):
        kc = codec.make_codec(d, bits, 0, codec.MODE_MSE)
        vc = codec.make_codec(d, bits, 1, codec.MODE_MSE)
        out = attention.decode_attention(q, quant.dequantize_state(quant.quantize(k, kc), kc),
                                         quant.dequantize_state(quant.quantize(v, vc), vc),
                                         np.array([N]), 1 / math.sqrt(d))[0, 0, 0]
        cos.append(out @ ref / np.linalg.norm(out) / np.linalg.norm(ref))
    assert cos[0] < cos[1] < cos[2] < 1.0


# the (head_dim, key bits, key mode, value bits, value mode) of the five workloads
WORKLOAD_CODECS = [
    (128, 3, codec.MODE_MSE, 3, codec.MODE_MSE),
    (128, 3, codec.MODE_PROD, 4, codec.MODE_MSE),
    (256, 3, codec.MODE_PROD, 2, codec.MODE_GROUP),
]


@pytest.mark.parametrize("case", WORKLOAD_CODECS)
def test_codebook_grid_cost_on_attention_quality(case):
    """The stored (2^-E grid) codebook against the unrounded float64 Lloyd-Max
    solution, both through the same oracle: attention quality, as the cosine
    similarity to exact attention on the unquantised K and V (the metric of
    "turboquant validate_moe_phase2.py", Test 1), moves by less than 1e-4 on
    average and 5e-4 on any row.  (Codes of coordinates between the two
    codebooks' boundaries differ, so individual outputs differ by up to a few
    1e-3; the quality figure does not.)"""
    import dataclasses
    d, kb, km, vb, vm = case
    rng = np.random.default_rng(1)
    B, Hkv, G, N = 1, 2, 8, 1024
    k = rng.standard_normal((B, Hkv, N, d)) * 0.02
    v = rng.standard_normal((B, Hkv, N, d)) * 0.02
    q = rng.standard_normal((B, Hkv * G, 1, d)) * 0.6
    kc, vc = codec.make_codec(d, kb, 0, km), codec.make_codec(d, vb, 1, vm)

    def unrounded(cb):
        if cb.mode == codec.MODE_GROUP:
            return cb
        s = cb.solution
        return dataclasses.replace(cb, centroids=s, boundaries=0.5 * (s[:-1] + s[1:]))

    lens, sc = np.array([N]), 1 / math.sqrt(d)
    ref = attention.reference_attention(q, k, v, lens, sc)

    def quality(kcb, vcb):
        o = attention.decode_attention_rotated(q, quant.quantize(k, kcb), kcb, quant.quantize(v, vcb), vcb, lens, sc)
        return np.sum(o * ref, -1) / (np.linalg.norm(o, axis=-1) * np.linalg.norm(ref, axis=-1))

    stored, exact = quality(kc, vc), quality(unrounded(kc), unrounded(vc))
    assert stored.mean() > 0.9
    assert abs(stored.mean() - exact.mean()) < 1e-4
    assert np.abs(stored - exact).max() < 5e-4
