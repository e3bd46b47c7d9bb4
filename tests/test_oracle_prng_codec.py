"""Pins for the oracle's generator and codec (CPU only).

Each pin checks the oracle against something other than itself: published
SplitMix64 outputs, distributional facts of the Box-Muller normals, the
defining property of the QR factorisation, the Lloyd-Max optimality
conditions evaluated by independent quadrature, a closed form at one bit, and
Max's (1960) Gaussian quantiser table in the large-d limit.
"""
import math

import numpy as np
import pytest
from scipy import integrate, special, stats

from oracle import codec, prng


def test_splitmix64_published_outputs():
    # First outputs of SplitMix64 started at state 0 (the reference outputs
    # of Steele-Lea-Flood's generator as distributed with Vigna's splitmix64.c).
    want = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F, 0xF88BB8A8724C81EC]
    got = [int(v) for v in prng.splitmix64(0, 4)]
    assert got == want


def test_stream_start_and_uniform_range():
    assert prng.stream_start(5, 0) == 5
    assert prng.stream_start(5, 1) == 5 ^ prng.GAMMA
    u = prng.uniforms(123, 200000)
    assert u.min() > 0.0 and u.max() <= 1.0
    # uniform on (0, 1]: mean 1/2, variance 1/12 within 5 standard errors
    n = u.size
    assert abs(u.mean() - 0.5) < 5 * math.sqrt(1 / 12 / n)
    assert stats.kstest(u, "uniform").pvalue > 1e-4


def test_box_muller_normals_are_standard_normal():
    g = prng.normals(7, 0, 400000)
    n = g.size
    assert abs(g.mean()) < 5 / math.sqrt(n)
    assert abs(g.var() - 1.0) < 5 * math.sqrt(2 / n)
    assert abs(stats.kurtosis(g, fisher=False) - 3.0) < 5 * math.sqrt(24 / n)
    assert stats.kstest(g, "norm").pvalue > 1e-4
    # cos and sin outputs of one pair are uncorrelated
    assert abs(np.corrcoef(g[0::2], g[1::2])[0, 1]) < 5 / math.sqrt(n / 2)


@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_rotation_is_the_positive_diagonal_qr_factor(d):
    g = prng.gaussian_matrix(3, prng.STREAM_ROTATION, d)
    pi = codec.rotation(d, 3)
    # Pi is orthogonal and R = Pi^T G is upper triangular with a positive diagonal
    assert np.abs(pi.T @ pi - np.eye(d)).max() < 1e-12
    r = pi.T @ g
    assert np.abs(np.tril(r, -1)).max() < 1e-10
    assert np.all(np.diag(r) > 0)
    # float32 storage keeps it orthogonal to the stated 1e-5
    p32 = pi.astype(np.float32).astype(np.float64)
    assert np.abs(p32.T @ p32 - np.eye(d)).max() < 1e-5


def test_codec_is_deterministic_in_its_parameters():
    a = codec.make_codec(64, 3, 11, codec.MODE_PROD)
    b = codec.make_codec(64, 3, 11, codec.MODE_PROD)
    c = codec.make_codec(64, 3, 12, codec.MODE_PROD)
    assert a.rot.tobytes() == b.rot.tobytes()
    assert a.sketch.tobytes() == b.sketch.tobytes()
    assert a.centroids.tobytes() == b.centroids.tobytes()
    assert a.rot.tobytes() != c.rot.tobytes()
    # the sketch is a different stream from the rotation's Gaussian
    g0 = prng.gaussian_matrix(11, 0, 64)
    assert not np.allclose(a.sketch, g0.astype(np.float32))


def _cond_mean_quad(d, lo, hi):
    f = lambda y: codec.coordinate_density(d, y)
    mass = integrate.quad(f, lo, hi, epsabs=0, epsrel=1e-13, limit=200)[0]
    mom = integrate.quad(lambda y: y * f(y), lo, hi, epsabs=0, epsrel=1e-13, limit=200)[0]
    return mom / mass


@pytest.mark.parametrize("d,bits", [(32, 2), (64, 3), (128, 1), (128, 2), (128, 3), (128, 4), (256, 2), (256, 3)])
def test_lloyd_max_optimality_by_quadrature(d, bits):
    c = codec.lloyd_max_solve(d, bits)
    levels = 1 << bits
    assert c.shape == (levels,)
    assert np.all(np.diff(c) > 0)
    assert np.all(c == -c[::-1])                       # exact odd symmetry
    t = 0.5 * (c[:-1] + c[1:])
    edges = np.concatenate(([-1.0], t, [1.0]))
    for k in range(levels):
        cm = _cond_mean_quad(d, edges[k], edges[k + 1])
        assert abs(cm - c[k]) < 1e-12 * max(1.0, abs(c[k]) * 10)


@pytest.mark.parametrize("d", [32, 128, 256])
def test_one_bit_closed_form(d):
    # E[Y | Y > 0] = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2))
    want = math.exp(math.lgamma(d / 2) - math.lgamma((d + 1) / 2)) / math.sqrt(math.pi)
    c = codec.lloyd_max_solve(d, 1)
    assert abs(c[1] - want) < 1e-14
    if d == 128:
        assert abs(c[1] - 0.0706615727) < 1e-10
    if d == 256:
        assert abs(c[1] - 0.0499165077) < 1e-10


# Max (1960), "Quantizing for minimum distortion", optimum levels for N(0, 1)
MAX_1960 = {
    1: [0.7979],
    2: [0.4528, 1.510],
    3: [0.2451, 0.7560, 1.344, 2.152],
    4: [0.1284, 0.3881, 0.6568, 0.9424, 1.256, 1.618, 2.069, 2.733],
}


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_large_d_limit_is_gaussian_lloyd_max(bits):
    d = 1 << 16
    c = codec.lloyd_max_solve(d, bits)
    upper = c[len(c) // 2:] * math.sqrt(d)
    assert np.allclose(upper, MAX_1960[bits], atol=2e-3)


@pytest.mark.parametrize("d,bits", [(128, 3), (128, 4), (256, 2), (32, 1)])
def test_stored_codebook_grid(d, bits):
    cb = codec.make_codec(d, bits, 0, codec.MODE_MSE)
    e = cb.grid_exp
    units = cb.centroids * 2.0 ** e
    assert np.all(units == np.rint(units))
    assert np.abs(units).max() <= codec.GRID_MAX
    assert np.abs(units).max() * 2 > codec.GRID_MAX      # E is the largest such
    assert np.all(np.abs(cb.centroids - cb.solution) <= 2.0 ** (-e - 1))
    assert np.all(cb.boundaries == 0.5 * (cb.centroids[:-1] + cb.centroids[1:]))
    assert cb.boundaries[len(cb.boundaries) // 2] == 0.0
    assert np.all(cb.centroids.astype(np.float32).astype(np.float64) == cb.centroids)


def _stored_cells(d, c, bnd):
    """Distortion sum_k int_cell_k (y - c_k)^2 f_d(y) dy and the largest
    |E[Y | cell_k] - c_k|, cells bounded by ``bnd``, by adaptive quadrature
    (independent of the closed forms the solver uses)."""
    f = lambda y: codec.coordinate_density(d, y)
    edges = np.concatenate(([-1.0], bnd, [1.0]))
    dist, resid = 0.0, 0.0
    for k in range(len(c)):
        lo, hi = edges[k], edges[k + 1]
        q = lambda g: integrate.quad(g, lo, hi, epsabs=0, epsrel=1e-12, limit=200)[0]
        dist += q(lambda y: (y - c[k]) ** 2 * f(y))
        resid = max(resid, abs(q(lambda y: y * f(y)) / q(f) - c[k]))
    return dist, resid


# every (head_dim, index bits) a workload or a test of this repository uses
GRID_COST_CASES = [(128, 1), (128, 2), (128, 3), (128, 4), (256, 1), (256, 2), (256, 3), (256, 4),
                   (32, 1), (32, 2), (32, 4), (64, 2), (64, 3), (64, 4), (96, 3), (96, 4), (160, 1),
                   (192, 1), (192, 2), (224, 4)]


@pytest.mark.parametrize("d,bits", GRID_COST_CASES)
def test_stored_codebook_distortion_cost(d, bits):
    """Cost of storing the centroids on the 2^-E grid, pinned by the
    mathematics of the Lloyd-Max conditions rather than by the solver.

    Moving centroid k of an optimal quantiser by delta_k with its cell fixed
    adds exactly P(cell_k) delta_k^2 to the distortion (the centroid is the
    cell's conditional mean), and re-drawing the cells at the new midpoints
    can only lower it (nearest-neighbour cells are optimal for given
    centroids).  With |delta_k| <= 2^-(E+1) the stored codebook's per-vector
    distortion d D therefore exceeds the optimum by at most d 2^-(2E+2).
    Each stored centroid also stays within half a grid unit of the
    conditional mean of its own (stored) cell."""
    cb = codec.make_codec(d, bits, 0, codec.MODE_MSE)
    e = cb.grid_exp
    sol = cb.solution
    d_opt, r_opt = _stored_cells(d, sol, 0.5 * (sol[:-1] + sol[1:]))
    d_sto, r_sto = _stored_cells(d, cb.centroids, cb.boundaries)
    assert r_opt < 1e-11                                  # the solution is a fixed point
    excess = d * (d_sto - d_opt)
    assert -1e-12 <= excess <= d * 2.0 ** (-2 * e - 2)
    assert excess <= 1e-6 * d * d_opt                     # relative cost below one part in 10^6
    assert r_sto <= 2.0 ** (-e - 1)


def test_survey_derived_values():
    # sqrt(d) * c for d = 128, 3 bits (derived independently with scipy when
    # the build was planned; 5 decimals)
    c = codec.lloyd_max_solve(128, 3)
    assert np.allclose(c[4:] * math.sqrt(128), [0.24442, 0.75333, 1.33660, 2.13147], atol=1e-5)


def test_unsupported_parameters_raise():
    with pytest.raises(ValueError):
        codec.make_codec(100, 3, 0, codec.MODE_MSE)
    with pytest.raises(ValueError):
        codec.make_codec(128, 1, 0, codec.MODE_PROD)
    with pytest.raises(ValueError):
        codec.make_codec(128, 5, 0, codec.MODE_MSE)
