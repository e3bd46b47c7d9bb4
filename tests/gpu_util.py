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
