"""Codec construction: rotation, Lloyd-Max codebook, QJL sketch (test infrastructure only).

What the pages fix
------------------
* A codec is a deterministic function of (head_dim, bits, seed); the K codec
  uses seed s and the V codec seed s + 1 ("omlx turboquant_kv.py",
  ``_rebuild_codecs``).
* Each head vector is rotated by a seeded random orthogonal matrix before
  scalar quantisation, and decompression is "unpack + Lloyd-Max codebook
  lookup, denormalise, inverse rotation" ("lightning-mlx plan.md", the
  section on the current TurboQuant codec).
* The Prod key quantiser carries a d x d rotation Pi and a d x d QJL matrix
  S, 4 bytes per entry each ("turboquant validate_moe_phase2.py", Test 2's
  per-layer Pi + S overhead).

Readings taken where the pages are silent
-----------------------------------------
* Rotation: Householder QR of a seeded Gaussian matrix G = Q R (numpy's
  LAPACK QR), Pi = Q diag(sign(R_ii)) so that the factorisation is the unique
  one with a positive diagonal; applied as y = Pi x; stored as float32.
* Codebook: the Lloyd-Max quantiser (Lloyd 1957/1982, Max 1960) for the exact
  density of one coordinate of a uniformly random unit vector in R^d,
      f_d(y) = (1 - y^2)^((d-3)/2) / B(1/2, (d-1)/2)  on [-1, 1],
  i.e. Y = 2 B - 1 with B ~ Beta((d-1)/2, (d-1)/2).  Lloyd iteration:
  boundaries are midpoints of neighbouring centroids, centroids are the
  conditional means of their cells.  The cell mass is a regularised
  incomplete beta function (scipy); the first moment has the closed form
      int_lo^hi y f_d(y) dy = [(1-lo^2)^a - (1-hi^2)^a] / (2 a B(1/2, a)),
  a = (d-1)/2.  The solution is made exactly odd-symmetric and then stored on
  the dyadic grid 2^-E, E the largest integer with max|c| 2^E <= 16256 (about
  14 significant bits; every stored value is an exact float32 and an exact
  15-bit integer multiple of 2^-E).  Boundaries are the exact midpoints of
  the stored centroids.  The grid is a storage format of the codec (each
  stored centroid is 256 hi + lo grid units with 8-bit pieces); the
  unrounded float64 solution is kept in ``Codec.solution`` so that the cost
  of the grid can be checked against it: with |stored - solution| <= 2^-(E+1)
  the per-vector distortion d D grows by at most d 2^-(2E+2) (the centroid
  condition makes the first-order term vanish).
* QJL sketch: S has iid N(0, 1) entries (stream 1 of the codec seed) and acts
  on the rotated residual; stored as float32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np
from scipy import special

from . import prng

MODE_MSE = 0
MODE_PROD = 1
MODE_GROUP = 2
MODE_SPLIT = 3

GRID_MAX = 16256  # 127 * 128: largest stored centroid magnitude in grid units
GROUP_SIZE = 32


def coordinate_density(d: int, y):
    """f_d(y): density of one coordinate of a uniform unit vector in R^d."""
    a = (d - 1) / 2.0
    y = np.asarray(y, dtype=np.float64)
    return np.exp((a - 1.0) * np.log1p(-y * y) - special.betaln(0.5, a))


def _cell_mass(d: int, lo: np.ndarray, hi: np.ndarray) -> np.ndarray:
    """P(lo < Y <= hi) for Y ~ f_d, via the regularised incomplete beta."""
    a = (d - 1) / 2.0
    # Upper tail by symmetry, P(Y > y) = I_{(1-y)/2}(a, a), avoids cancellation.
    upper_lo = special.betainc(a, a, (1.0 - lo) / 2.0)
    upper_hi = special.betainc(a, a, (1.0 - hi) / 2.0)
    return upper_lo - upper_hi


def _cell_first_moment(d: int, lo: np.ndarray, hi: np.ndarray) -> np.ndarray:
    """int_lo^hi y f_d(y) dy in closed form."""
    a = (d - 1) / 2.0
    norm = math.exp(-special.betaln(0.5, a))
    with np.errstate(divide="ignore"):
        p_lo = np.exp(a * np.log1p(-lo * lo))
        p_hi = np.exp(a * np.log1p(-hi * hi))
    return norm * (p_lo - p_hi) / (2.0 * a)


def lloyd_max_step(d: int, c: np.ndarray) -> np.ndarray:
    """One Lloyd iteration: midpoint boundaries, then conditional means."""
    t = 0.5 * (c[:-1] + c[1:])
    lo = np.concatenate(([-1.0], t))
    hi = np.concatenate((t, [1.0]))
    return _cell_first_moment(d, lo, hi) / _cell_mass(d, lo, hi)


def lloyd_max_solve(d: int, bits: int, tol: float = 1e-14, max_iter: int = 20000) -> np.ndarray:
    """The float64 Lloyd-Max centroids (ascending) of f_d with 2**bits levels.

    Iterates until no centroid moves by more than ``tol`` (the map's own
    rounding noise is a few 1e-15), starting from levels spread uniformly
    over +-2.5/sqrt(d)."""
    levels = 1 << bits
    c = (2.0 * np.arange(levels) + 1.0 - levels) / levels * (2.5 / math.sqrt(d))
    for _ in range(max_iter):
        nxt = lloyd_max_step(d, c)
        step = np.max(np.abs(nxt - c))
        c = nxt
        if step <= tol:
            break
    # exact odd symmetry c_k = -c_{L-1-k}
    return 0.5 * (c - c[::-1])


def grid_exponent(c: np.ndarray) -> int:
    """Largest E with max|c| * 2**E <= GRID_MAX."""
    m = float(np.max(np.abs(c)))
    e = int(math.floor(math.log2(GRID_MAX / m)))
    while m * 2.0 ** (e + 1) <= GRID_MAX:
        e += 1
    while m * 2.0 ** e > GRID_MAX:
        e -= 1
    return e


def store_codebook(c: np.ndarray):
    """Round the solution onto the dyadic grid; return (centroids, boundaries, E)."""
    e = grid_exponent(c)
    units = np.rint(c * 2.0 ** e)
    cs = units * 2.0 ** -e
    bnd = 0.5 * (cs[:-1] + cs[1:])
    assert np.all(cs.astype(np.float32).astype(np.float64) == cs)
    assert np.all(bnd.astype(np.float32).astype(np.float64) == bnd)
    return cs, bnd, e


def rotation(d: int, seed: int, stream: int = prng.STREAM_ROTATION) -> np.ndarray:
    """Pi (float64): QR of the seed's Gaussian (stream 0 unless stated) with
    positive diag(R)."""
    g = prng.gaussian_matrix(seed, stream, d)
    q, r = np.linalg.qr(g)
    sgn = np.where(np.diag(r) < 0.0, -1.0, 1.0)
    return q * sgn[None, :]


def sketch(d: int, seed: int) -> np.ndarray:
    """S (float64): iid N(0, 1) from the seed's stream 1."""
    return prng.gaussian_matrix(seed, prng.STREAM_SKETCH, d)


@dataclass
class Codec:
    head_dim: int
    bits: int
    seed: int
    mode: int
    mse_bits: int                 # bits of the packed index stream
    rot: Optional[np.ndarray]     # Pi as stored (float32 values, float64 dtype)
    centroids: Optional[np.ndarray]
    boundaries: Optional[np.ndarray]
    sketch: Optional[np.ndarray]  # S as stored (float32 values, float64 dtype)
    grid_exp: Optional[int]
    solution: Optional[np.ndarray]  # unrounded float64 Lloyd-Max solution

    @property
    def levels(self) -> int:
        return 1 << self.mse_bits


def make_codec(head_dim: int, bits: int, seed: int, mode: int, rot_stream: int = prng.STREAM_ROTATION) -> Codec:
    """Build a codec.  Prod spends bits-1 on the MSE stage and 1 on QJL signs
    ("omlx turboquant_kv.py", ``_infer_head_dim``: the Prod state's packed
    width uses bits - 1); group mode has no rotation or codebook."""
    d = int(head_dim)
    if d <= 0 or d % 32 or d > 256:
        raise ValueError("head_dim must be a positive multiple of 32, at most 256")
    if mode == MODE_GROUP:
        if bits not in (1, 2, 3, 4):
            raise ValueError("group mode supports 1..4 bits")
        return Codec(d, bits, seed, mode, bits, None, None, None, None, None, None)
    mse_bits = bits - 1 if mode == MODE_PROD else bits
    if mode not in (MODE_MSE, MODE_PROD) or not 1 <= mse_bits <= 4:
        raise ValueError("unsupported (bits, mode)")
    sol = lloyd_max_solve(d, mse_bits)
    cs, bnd, e = store_codebook(sol)
    rot = rotation(d, seed, rot_stream).astype(np.float32).astype(np.float64)
    sk = None
    if mode == MODE_PROD:
        sk = sketch(d, seed).astype(np.float32).astype(np.float64)
    return Codec(d, bits, seed, mode, mse_bits, rot, cs, bnd, sk, e, sol)


# ---- fractional bit-widths ---------------------------------------------------
#
# "omlx turboquant_kv.py", _rebuild_codecs: a bit-width is fractional when it
# is not within 1e-6 of an integer; then the key codec takes floor(bits) and
# the value codec ceil(bits) (both MSE, key on seed s, value on s + 1);
# otherwise both take bits.  The same page's state helpers carry a
# TurboQuantSplitState(low, high): two sub-states filtered and concatenated
# together along the batch axis.  Reading taken for it (the plainest one the
# rest supports): a split codec of fractional width b quantises the first
# d_lo channels of a head vector with a floor(b)-bit MSE codec ("low") and the
# last d_hi channels with a ceil(b)-bit one ("high"), each an independent
# TurboQuant instance of its own dimension (own rotation, norm and Lloyd-Max
# codebook), d_hi = round((b - floor b) d / 32) * 32 so that both parts are
# whole 32-coordinate groups; the mean width is b whenever (b - floor b) d is
# a multiple of 32 (2.5, 3.5, 3.25 and 3.75 bits at d = 128).  The low part's
# rotation is stream 0 of the seed, the high part's stream 2.


def is_fractional(bits: float) -> bool:
    return not math.isclose(bits, round(bits), abs_tol=1e-6)


def kv_bits(bits: float):
    """(key bits, value bits) of the codec rebuild rule."""
    if is_fractional(bits):
        return int(math.floor(bits)), int(math.ceil(bits))
    return int(round(bits)), int(round(bits))


def kv_codecs(head_dim: int, bits: float, seed: int):
    """The key and value MSE codecs a cache of width ``bits`` rebuilds."""
    kb, vb = kv_bits(bits)
    return make_codec(head_dim, kb, seed, MODE_MSE), make_codec(head_dim, vb, seed + 1, MODE_MSE)


@dataclass
class SplitCodec:
    head_dim: int
    bits: float
    seed: int
    low: Codec      # channels 0 .. d_lo - 1, floor(bits)
    high: Codec     # channels d_lo .. d - 1, ceil(bits)
    mode: int = MODE_SPLIT

    @property
    def d_lo(self) -> int:
        return self.low.head_dim

    @property
    def d_hi(self) -> int:
        return self.high.head_dim


def split_shape(head_dim: int, bits: float):
    """(d_lo, d_hi, low bits, high bits) of a split codec."""
    if not is_fractional(bits):
        raise ValueError("a split codec needs a fractional bit-width")
    lo, hi = int(math.floor(bits)), int(math.ceil(bits))
    d_hi = int(round((bits - lo) * head_dim / 32.0)) * 32
    if lo < 1 or hi > 4 or not 32 <= d_hi <= head_dim - 32:
        raise ValueError("unsupported split: each part needs 32..head_dim-32 channels and 1..4 bits")
    return head_dim - d_hi, d_hi, lo, hi


def make_split_codec(head_dim: int, bits: float, seed: int) -> SplitCodec:
    d = int(head_dim)
    if d <= 0 or d % 32 or d > 256:
        raise ValueError("head_dim must be a positive multiple of 32, at most 256")
    d_lo, d_hi, lo, hi = split_shape(d, bits)
    return SplitCodec(d, float(bits), seed, make_codec(d_lo, lo, seed, MODE_MSE),
                      make_codec(d_hi, hi, seed, MODE_MSE, rot_stream=prng.STREAM_SPLIT_HIGH))
