"""Pins for the oracle's packing and quantisers (CPU only)."""
import math
import os

import numpy as np
import pytest
from scipy import integrate

from oracle import codec, packing, quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "packing_examples.txt")


def _golden_cases():
    cases = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        head, rule, words = [s.strip() for s in line.split("|")]
        b, d = (int(v) for v in head.split())
        cases.append((b, d, rule, [int(w, 16) for w in words.split()]))
    return cases


def _indices(rule, b, d):
    if rule == "mod8":
        return np.arange(d) % 8
    if rule == "mod4":
        return np.arange(d) % 4
    if rule == "all7":
        return np.full(d, 7)
    if rule == "even1":
        return (np.arange(d) % 2 == 0).astype(np.int64)
    if rule.startswith("one:"):
        j, v = rule[4:].split("=")
        idx = np.zeros(d, dtype=np.int64)
        idx[int(j)] = int(v)
        return idx
    raise ValueError(rule)


@pytest.mark.parametrize("b,d,rule,want", _golden_cases())
def test_packing_hand_derived_examples(b, d, rule, want):
    idx = _indices(rule, b, d)
    words = packing.pack(idx[None], b)[0]
    assert [int(w) for w in words] == want
    assert np.array_equal(packing.unpack(words[None], b, d)[0], idx)


@pytest.mark.parametrize("b", [1, 2, 3, 4])
@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_packing_round_trip_and_width(b, d):
    rng = np.random.default_rng(b * 1000 + d)
    idx = rng.integers(0, 1 << b, size=(5, d))
    words = packing.pack(idx, b)
    assert words.shape == (5, math.ceil(d * b / 32))      # W = ceil(d*b/32)
    assert np.array_equal(packing.unpack(words, b, d), idx)


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_packing_uses_every_bit_once(b):
    d = 64
    seen = np.zeros((d * b) // 32 * 32, dtype=int)
    for j in range(d):
        for (w, bit, n, src) in packing.field_pieces(b, j):
            seen[w * 32 + bit: w * 32 + bit + n] += 1
    assert np.all(seen == 1)


def _distortion(d, cb):
    """Per-coordinate MSE sum_k int_cell (y - c_k)^2 f_d(y) dy by quadrature."""
    edges = np.concatenate(([-1.0], cb.boundaries, [1.0]))
    tot = 0.0
    for k, ck in enumerate(cb.centroids):
        tot += integrate.quad(lambda y: (y - ck) ** 2 * codec.coordinate_density(d, y),
                              edges[k], edges[k + 1], epsabs=0, epsrel=1e-12, limit=200)[0]
    return tot


@pytest.mark.parametrize("d,bits", [(64, 2), (64, 3), (128, 3), (32, 4)])
def test_mse_quantizer_distortion_matches_density(d, bits):
    cb = codec.make_codec(d, bits, 5, codec.MODE_MSE)
    rng = np.random.default_rng(17)
    n = 20000
    x = rng.standard_normal((n, d)).astype(np.float32)
    st = quant.mse_quantize(x, cb)
    xt = quant.dequantize_mse(st["norm"], st["idx"], cb)
    nrm = np.linalg.norm(x.astype(np.float64), axis=1)
    err = np.sum((x / nrm[:, None] - xt / st["norm"][:, None]) ** 2, axis=1)
    dd = d * _distortion(d, cb)
    se = err.std() / math.sqrt(n)
    assert abs(err.mean() - dd) < 4 * se
    # centroid condition -> <u, u~> has mean 1 - d D (multiplicative shrink)
    inner = np.sum((x / nrm[:, None]) * (xt / st["norm"][:, None]), axis=1)
    assert abs(inner.mean() - (1 - dd)) < 4 * inner.std() / math.sqrt(n)
    # known value of d*D for (128, 3) (derived when the build was planned)
    if (d, bits) == (128, 3):
        assert abs(dd - 0.033966) < 2e-5


def test_mse_zero_vector_and_ties():
    cb = codec.make_codec(32, 3, 1, codec.MODE_MSE)
    st = quant.mse_quantize(np.zeros((1, 32), dtype=np.float32), cb)
    assert st["norm"][0] == 0.0
    assert np.all(st["idx"] == cb.levels // 2 - 1)
    # a coordinate exactly on a boundary goes to the lower cell
    u = np.array(cb.boundaries)
    assert np.all(np.sum(u[:, None] > cb.boundaries, axis=-1) == np.arange(len(u)))


def test_prod_zero_vector():
    cb = codec.make_codec(32, 3, 1, codec.MODE_PROD)
    st = quant.prod_quantize(np.zeros((1, 32), dtype=np.float32), cb)
    assert st["rnorm"][0] == 0.0 and np.all(st["sign_bits"] == 1)


def test_qjl_estimator_is_unbiased_over_seeds():
    d, bits, seeds = 32, 3, 4096
    rng = np.random.default_rng(0)
    x = rng.standard_normal(d).astype(np.float32)
    q = rng.standard_normal(d)
    cb0 = codec.make_codec(d, bits, 0, codec.MODE_PROD)
    est = np.empty(seeds)
    mse_only = np.empty(seeds)
    self_prod = np.empty(seeds)
    self_mse = np.empty(seeds)
    for s in range(seeds):
        cb = codec.Codec(d, bits, s, codec.MODE_PROD, bits - 1,
                         codec.rotation(d, s).astype(np.float32).astype(np.float64),
                         cb0.centroids, cb0.boundaries,
                         codec.sketch(d, s).astype(np.float32).astype(np.float64), cb0.grid_exp, None)
        st = quant.prod_quantize(x[None], cb)
        xt = quant.dequantize_prod(st["norm"], st["idx"], st["rnorm"], st["sign_bits"], cb)[0]
        xm = quant.dequantize_mse(st["norm"], st["idx"], cb)[0]
        est[s] = q @ xt
        mse_only[s] = q @ xm
        self_prod[s] = x @ xt
        self_mse[s] = x @ xm
    truth = float(q @ x.astype(np.float64))
    assert abs(est.mean() - truth) < 4 * est.std() / math.sqrt(seeds)
    # with q = x the MSE-only estimate is low by about d*D_{b-1}; Prod is not
    xx = float(x.astype(np.float64) @ x)
    assert abs(self_prod.mean() - xx) < 4 * self_prod.std() / math.sqrt(seeds)
    assert self_mse.mean() < xx * (1 - 0.05)


def test_group_quantization_properties():
    rng = np.random.default_rng(3)
    for bits in (2, 4):
        top = (1 << bits) - 1
        v = rng.standard_normal((50, 64)).astype(np.float32)
        st = quant.group_quantize(v, bits)
        rec = quant.dequantize_group(st["q"], st["scale"], st["min"])
        s = np.repeat(st["scale"], 32, axis=-1)
        assert np.all(np.abs(rec - v) <= s / 2 * (1 + 1e-6) + 1e-12)
        assert np.all(st["q"] >= 0) and np.all(st["q"] <= top)
        # group min and max are hit exactly
        g = v.reshape(50, 2, 32).astype(np.float64)
        assert np.array_equal(st["min"], g.min(-1))
        # values already on the grid {mn + k s} reconstruct exactly
        mn, sc = 0.25, 0.125
        k = rng.integers(0, top + 1, size=(1, 32))
        k[0, 0], k[0, 1] = 0, top
        vg = (mn + k * sc).astype(np.float32)
        st2 = quant.group_quantize(vg, bits)
        assert np.array_equal(quant.dequantize_group(st2["q"], st2["scale"], st2["min"]), vg.astype(np.float64))
    # a constant group reconstructs exactly with q = 0
    c = np.full((1, 32), 0.7, dtype=np.float32)
    st = quant.group_quantize(c, 2)
    assert np.all(st["q"] == 0) and st["scale"][0, 0] == 0.0
    assert np.array_equal(quant.dequantize_group(st["q"], st["scale"], st["min"]), c.astype(np.float64))
    # a half-way value rounds to even: (mn, mx) = (0, 3), v = 0.5 -> t = 0.5 -> 0; v = 1.5 -> 2
    v = np.zeros((1, 32), dtype=np.float32)
    v[0, 1], v[0, 2], v[0, 3] = 3.0, 0.5, 1.5
    st = quant.group_quantize(v, 2)
    assert st["q"][0, 2] == 0 and st["q"][0, 3] == 2
