"""Pins for the oracle's fractional bit-widths and split codecs (CPU only).

The rebuild rule is the pages' ("omlx turboquant_kv.py", _rebuild_codecs:
fractional = not within 1e-6 of an integer; keys floor, values ceil); the
split codec's packed width is checked against the pages' width formula
ceil(head_dim * bits / 32) (_infer_head_dim) taken at the fractional width,
its distortion against the parts' Lloyd-Max distortions computed by
independent quadrature, and its decode against brute force."""
import math

import numpy as np
import pytest
from scipy import integrate

from oracle import attention, codec, prng, quant


@pytest.mark.parametrize("bits,want", [(3.5, (3, 4)), (2.5, (2, 3)), (3.0, (3, 3)), (3.0000004, (3, 3)),
                                       (2.9999996, (3, 3)), (3.2, (3, 4)), (4, (4, 4))])
def test_kv_rebuild_rule(bits, want):
    assert codec.kv_bits(bits) == want
    k, v = codec.kv_codecs(128, bits, 9)
    assert (k.bits, v.bits) == want and k.mode == v.mode == codec.MODE_MSE
    assert (k.seed, v.seed) == (9, 10)


@pytest.mark.parametrize("d,bits,want", [(128, 3.5, (64, 64, 3, 4)), (128, 3.25, (96, 32, 3, 4)),
                                         (128, 2.75, (32, 96, 2, 3)), (256, 2.5, (128, 128, 2, 3)),
                                         (64, 1.5, (32, 32, 1, 2))])
def test_split_shape_and_packed_width(d, bits, want):
    assert codec.split_shape(d, bits) == want
    sc = codec.make_split_codec(d, bits, 0)
    x = np.random.default_rng(1).standard_normal((3, d))
    st = quant.quantize(x, sc)
    # the pages' width formula at the fractional width: ceil(d * bits / 32)
    assert st["words"].shape[-1] == math.ceil(d * bits / 32)


@pytest.mark.parametrize("d,bits", [(128, 3.1), (128, 4.5), (128, 0.5), (32, 2.5), (128, 3.0)])
def test_split_refuses_what_it_cannot_build(d, bits):
    with pytest.raises(ValueError):
        codec.make_split_codec(d, bits, 0)


def test_split_parts_are_independent_orthogonal_rotations():
    sc = codec.make_split_codec(128, 3.5, 4)
    lo, hi = sc.low.rot, sc.high.rot
    for r in (lo, hi):
        assert np.abs(r.T @ r - np.eye(64)).max() < 1e-5
    assert not np.allclose(lo, hi)                        # streams 0 and 2 of one seed
    assert np.array_equal(hi, codec.rotation(64, 4, prng.STREAM_SPLIT_HIGH).astype(np.float32).astype(np.float64))


def _part_distortion(d, bits):
    """d D_b(d) of the stored codebook by adaptive quadrature."""
    cb = codec.make_codec(d, bits, 0, codec.MODE_MSE)
    f = lambda y: codec.coordinate_density(d, y)
    edges = np.concatenate(([-1.0], cb.boundaries, [1.0]))
    tot = sum(integrate.quad(lambda y, c=c: (y - c) ** 2 * f(y), lo, hi, epsabs=0, epsrel=1e-11, limit=200)[0]
              for c, lo, hi in zip(cb.centroids, edges[:-1], edges[1:]))
    return d * tot


@pytest.mark.parametrize("d,bits", [(128, 3.5), (128, 3.25), (256, 2.5)])
def test_split_distortion_is_the_parts_distortion(d, bits):
    """For Gaussian x the parts are independent Gaussian vectors and each part's
    expected relative error is exactly its d_p D(d_p) (the norm-and-direction
    identity of the MSE quantiser), so
        E ||x - x~||^2 = sigma^2 (d_lo * dD_lo + d_hi * dD_hi)."""
    sc = codec.make_split_codec(d, bits, 2)
    n = 20000
    x = np.random.default_rng(3).standard_normal((n, d))
    err = np.sum((quant.dequantize_state(quant.quantize(x, sc), sc) - x) ** 2, axis=-1)
    want = sc.d_lo * _part_distortion(sc.d_lo, sc.low.bits) + sc.d_hi * _part_distortion(sc.d_hi, sc.high.bits)
    se = err.std() / math.sqrt(n)
    assert abs(err.mean() - want) < 4 * se


@pytest.mark.parametrize("kspec,vspec", [("split", "split"), ("split", "mse"), ("mse", "split"), ("prod", "split")])
def test_split_decode_bruteforce_equals_rotated(kspec, vspec):
    rng = np.random.default_rng(5)
    d, B, Hkv, Hq, q_len, N = 128, 2, 2, 4, 2, 40
    make = {"split": lambda s: codec.make_split_codec(d, 2.5, s), "mse": lambda s: codec.make_codec(d, 3, s, 0),
            "prod": lambda s: codec.make_codec(d, 3, s, 1)}
    kc, vc = make[kspec](0), make[vspec](1)
    k = rng.standard_normal((B, Hkv, N, d)) * 0.02
    v = rng.standard_normal((B, Hkv, N, d)) * 0.02
    q = rng.standard_normal((B, Hq, q_len, d)) * 0.5
    ks, vs = quant.quantize(k, kc), quant.quantize(v, vc)
    lens = np.array([N, 17])
    sc = 1 / math.sqrt(d)
    a = attention.decode_attention(q, quant.dequantize_state(ks, kc), quant.dequantize_state(vs, vc), lens, sc)
    b = attention.decode_attention_rotated(q, ks, kc, vs, vc, lens, sc)
    assert np.abs(a - b).max() <= 1e-12 * np.abs(a).max()
    # and the stored words unpack back to the same codes
    st = quant.state_from_words(kc, ks["words"], norm=ks["norm"], rnorm=ks.get("rnorm"),
                                sign_words=ks.get("sign_words"))
    assert np.array_equal(st["idx"], ks["idx"])
