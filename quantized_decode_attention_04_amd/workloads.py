"""Seeded synthetic inputs shaped like the pages' workloads.

Only random draws and input rounding live here -- none of the method's
arithmetic -- so that the tests, the bench and the oracle's baseline timing can
share the same inputs.

Recipe (the pages' own synthetic data, "turboquant validate_moe_phase2.py",
Tests 1-5: N(0, 1) * 0.02 keys, values and queries):
  * streams: ``numpy.random.default_rng([seed, layer, stream])`` draws
    float32 ``standard_normal`` in C order [B, H, N, d], times 0.02;
    stream 0 = K, 1 = V, 2 = q, 3 = new K, 4 = new V;
  * bf16 inputs are rounded to nearest-even bf16 values (kept as float32
    arrays holding exactly representable values);
  * per-channel outliers: per (layer, KV head), round(4% of d) channels chosen
    without replacement and scaled by U[1, 8], separately for K and V
    (stream 10 + 2*head for K, 11 + 2*head for V);
  * ragged lengths: ``default_rng(0).integers(1024, 65536, 32, endpoint=True)``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

STD = np.float32(0.02)
STREAM_K, STREAM_V, STREAM_Q, STREAM_KNEW, STREAM_VNEW = 0, 1, 2, 3, 4


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns
    float32 values that bfloat16 represents exactly."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    out = r.astype(np.uint32).view(np.float32)
    return np.where(np.isnan(a), a, out)


def normal(seed: int, layer: int, stream: int, shape, bf16: bool) -> np.ndarray:
    x = np.random.default_rng([seed, layer, stream]).standard_normal(shape, dtype=np.float32) * STD
    return round_bf16(x) if bf16 else x


def outlier_scales(seed: int, layer: int, heads: int, d: int, which: int, frac: float = 0.04) -> np.ndarray:
    """[heads, d] per-channel multipliers: 1 except round(frac*d) channels per
    head drawn without replacement with a U[1, 8] scale."""
    k = int(round(frac * d))
    s = np.ones((heads, d), dtype=np.float32)
    for h in range(heads):
        rng = np.random.default_rng([seed, layer, 10 + 2 * h + which])
        ch = rng.choice(d, size=k, replace=False)
        s[h, ch] = rng.uniform(1.0, 8.0, size=k).astype(np.float32)
    return s


def ragged_lengths(n: int = 32, lo: int = 1024, hi: int = 65536, seed: int = 0) -> np.ndarray:
    return np.random.default_rng(seed).integers(lo, hi, n, endpoint=True)


@dataclass
class Workload:
    name: str
    batch: int
    hkv: int
    hq: int
    d: int
    n: int                      # cached tokens (max over the batch)
    q_len: int
    kbits: int
    kmode: int                  # 0 MSE, 1 Prod
    vbits: int
    vmode: int                  # 0 MSE, 2 group
    bf16: bool
    layers: int = 1
    outliers: bool = False
    lengths: Optional[List[int]] = None
    append: int = 0             # tokens appended per sequence per step
    prefill: int = 0            # bulk prefill tokens per head
    extra: dict = field(default_factory=dict)

    def lens(self) -> np.ndarray:
        if self.lengths is not None:
            return np.asarray(self.lengths, dtype=np.int64)
        return np.full(self.batch, self.n, dtype=np.int64)


def configs() -> dict:
    """The five workloads (sizes from the pages' shapes, see module doc)."""
    lens5 = ragged_lengths().tolist()
    return {
        "single_head_d128_n4096_mse3": Workload("single_head_d128_n4096_mse3", 1, 1, 1, 128, 4096, 1, 3, 0, 3, 0, False),
        "gqa8_d128_n32k_prod3_mse4": Workload("gqa8_d128_n32k_prod3_mse4", 1, 8, 64, 128, 32768, 1, 3, 1, 4, 0, True),
        "moe_d256_n131k_prod3_group2": Workload("moe_d256_n131k_prod3_group2", 1, 2, 16, 256, 131072, 1, 3, 1, 2, 2, True),
        "l64_d128_n256k_mse3_mtp2": Workload("l64_d128_n256k_mse3_mtp2", 1, 8, 64, 128, 262144, 2, 3, 0, 3, 0, True,
                                             layers=64, outliers=True, append=2),
        "ragged32_d128_prod3_mse4": Workload("ragged32_d128_prod3_mse4", 32, 8, 64, 128, max(lens5), 1, 3, 1, 4, 0, True,
                                             lengths=lens5, append=1, prefill=8192),
    }


def kv_tensors(w: Workload, layer: int, seed: int = 0, n: Optional[int] = None):
    """K and V [B, Hkv, n, d] float32 values (bf16-rounded for bf16 workloads)."""
    n = w.n if n is None else n
    shape = (w.batch, w.hkv, n, w.d)
    k = np.random.default_rng([seed, layer, STREAM_K]).standard_normal(shape, dtype=np.float32) * STD
    v = np.random.default_rng([seed, layer, STREAM_V]).standard_normal(shape, dtype=np.float32) * STD
    if w.outliers:
        k *= outlier_scales(seed, layer, w.hkv, w.d, 0)[None, :, None, :]
        v *= outlier_scales(seed, layer, w.hkv, w.d, 1)[None, :, None, :]
    if w.bf16:
        k, v = round_bf16(k), round_bf16(v)
    return k, v


def queries(w: Workload, layer: int, seed: int = 0) -> np.ndarray:
    return normal(seed, layer, STREAM_Q, (w.batch, w.hq, w.q_len, w.d), w.bf16)


def device_normal(shape, seed: int, layer: int, stream: int, bf16: bool, device="cuda", scales=None):
    """Seeded N(0, 1) * 0.02 drawn on the device with torch's Philox generator
    (used where host generation of gigabytes would dominate set-up time);
    ``scales`` ([heads, d]) applies the per-channel outlier multipliers to a
    [B, heads, n, d] tensor.  Returns float32 or bfloat16 (round to nearest
    even)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(((seed * 1000003 + layer) * 1009 + stream) & 0x7FFFFFFFFFFFFFFF)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * float(STD)
    if scales is not None:
        x *= torch.from_numpy(scales).to(device)[None, :, None, :]
    return x.to(torch.bfloat16) if bf16 else x
