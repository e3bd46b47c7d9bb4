"""Helpers for the GPU tests: moving oracle states into device caches and
reading device caches back (plumbing only)."""
from __future__ import annotations

import numpy as np

WINDOW = 1e-6  # decision window on the unit-vector coordinate / sign / group grid


def to_device_f(a, bf16: bool, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    return t.to(torch.bfloat16) if bf16 else t


def words_i32(words) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(words, dtype=np.uint32)).view(np.int32)


def upload_state(cache, state: dict, mode: int, n: int) -> None:
    """Write an oracle state (arrays [B, H, n, ...]) into cache slots 0..n-1."""
    import torch
    dev = cache.idx.device
    cache.idx[:, :, :n] = torch.from_numpy(words_i32(state["words"])).to(dev)
    if mode in (0, 1):
        cache.norm[:, :, :n] = torch.from_numpy(np.asarray(state["norm"], dtype=np.float32)).to(dev)
    if mode == 1:
        cache.rnorm[:, :, :n] = torch.from_numpy(np.asarray(state["rnorm"], dtype=np.float32)).to(dev)
        cache.sign[:, :, :n] = torch.from_numpy(words_i32(state["sign_words"])).to(dev)
    if mode == 2:
        cache.scale[:, :, :n] = torch.from_numpy(np.asarray(state["scale"], dtype=np.float32)).to(dev)
        cache.gmin[:, :, :n] = torch.from_numpy(np.asarray(state["min"], dtype=np.float32)).to(dev)


def download(cache) -> dict:
    out = {}
    for k, v in cache.arrays().items():
        a = v.cpu().numpy()
        out[k] = a.view(np.uint32) if a.dtype == np.int32 else a
    return out


def rel_l2_rows(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Relative L2 error of a against b per last-axis row (0 where both are 0)."""
    num = np.linalg.norm(a - b, axis=-1)
    den = np.linalg.norm(b, axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


def expected_window(codec, n_vectors: int) -> float:
    """Expected number of decision values within WINDOW of their threshold for
    n_vectors isotropic inputs: rotated coordinates follow the coordinate
    density f_d near each codebook boundary; a QJL sign's z / gamma is N(0, 1)
    (its window is |z| / (sqrt(d) gamma) < WINDOW); a group code's fractional
    part is uniform (window |frac - 1/2| < WINDOW (2^b - 1)).  Used to bound
    the window counts the parity tests report."""
    import math
    from oracle import codec as ocodec
    d = codec.head_dim
    if codec.mode == ocodec.MODE_GROUP:
        top = (1 << codec.bits) - 1
        return n_vectors * d * 2.0 * WINDOW * top
    per = 2.0 * WINDOW * float(np.sum(ocodec.coordinate_density(d, codec.boundaries)))
    lam = n_vectors * d * per
    if codec.mode == ocodec.MODE_PROD:
        lam += n_vectors * d * 2.0 * WINDOW * math.sqrt(d) / math.sqrt(2.0 * math.pi)
    return lam


def window_ceiling(lam: float) -> float:
    """A count a Poisson(lam) variable exceeds with negligible probability
    (lam + 6 sqrt(lam) + 6), with 50% slack for inputs that are only close to
    isotropic (bf16 rounding, outlier channels)."""
    import math
    return 1.5 * (lam + 6.0 * math.sqrt(lam) + 6.0)
