"""GPU parity for the hybrid cache (recent-token rings in front of the
compressed caches; "turboquant validate_moe_phase2.py", Test 5's buffer_size
and the commit note's hybrid decode, read as in oracle.hybrid): step by step
through ring flushes, with sequences in different phases, the compressed
caches hold the oracle's quantisation of each sequence's first
floor(N/B)*B tokens (window-free inputs: bit-exact words, norms to 1e-6), the
rings hold the rest bit for bit, and hybrid decode matches the oracle's
hybrid decode to relative L2 1e-4 per row."""
import dataclasses
import math
import sys

import numpy as np
import pytest

from oracle import codec as ocodec
from oracle import hybrid as ohybrid
from oracle import quant as oquant
from tests.gpu_util import WINDOW, download, rel_l2_rows, to_device_f

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


import quantized_decode_attention_04_amd as tq  # noqa: E402
from quantized_decode_attention_04_amd.workloads import round_bf16  # noqa: E402


def _window_free_tokens(rng, shape, codecs):
    """bf16 tokens N(0, 0.02^2) none of whose decision values (under any of
    ``codecs``) is inside the window, so that GPU and oracle codes agree."""
    x = round_bf16(rng.standard_normal(shape).astype(np.float32) * np.float32(0.02))
    for _ in range(60):
        bad = np.zeros(shape[:-1], dtype=bool)
        for oc in codecs:
            st = oquant.quantize(x.astype(np.float64), oc)
            m = st["margin"] < WINDOW * (((1 << oc.bits) - 1) if oc.mode == 2 else 1)
            if oc.mode == 1:
                m = m | (st["zmargin"] < WINDOW)
            bad |= m.any(-1)
        if not bad.any():
            return x
        x = x.copy()
        x[bad] = round_bf16(rng.standard_normal((int(bad.sum()), shape[-1])).astype(np.float32) * np.float32(0.02))
    raise RuntimeError("no window-free draw")


def _row_view(c, b):
    sl = lambda t: None if t is None else t[b:b + 1]
    return dataclasses.replace(c, batch=1, idx=sl(c.idx), norm=sl(c.norm), rnorm=sl(c.rnorm), sign=sl(c.sign),
                               scale=sl(c.scale), gmin=sl(c.gmin))


CASES = [
    # name, d, (kbits, kmode), (vbits, vmode), Hkv, Hq, ring
    ("mse3_mse3_int8_path", 128, (3, 0), (3, 0), 2, 16, 16),
    ("prod3_mse4_bf16_path", 128, (3, 1), (4, 0), 2, 16, 16),
    ("d256_prod3_group2_general_path", 256, (3, 1), (2, 2), 1, 4, 32),
    # split caches of 2.5 bits (mode 3): the fp32 matrix-core split kernel
    ("split25_split25_split_path", 128, (2.5, 3), (2.5, 3), 2, 16, 16),
]


def _codecs(spec, d, seed):
    """(bits, mode) -> (oracle codec, device codec); mode 3 is a split codec
    of fractional width bits."""
    bits, mode = spec
    if mode == 3:
        return ocodec.make_split_codec(d, bits, seed), tq.tq_codec_create_split(d, bits, seed)
    return ocodec.make_codec(d, bits, seed, mode), tq.tq_codec_create(d, bits, seed, mode)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_hybrid_steps_through_flushes(case):
    name, d, kspec, vspec, Hkv, Hq, ring = case
    print(f"hybrid {name}", flush=True)
    sys.stdout.flush()
    rng = np.random.default_rng(23)
    B, q_len, n_new, steps = 3, 2, 2, 6
    start = [5, ring - 1, 2 * ring - 2]
    final = [s + steps * n_new for s in start]
    cap = max(final)
    (okc, gk), (ovc, gv) = _codecs(kspec, d, 0), _codecs(vspec, d, 1)
    k = _window_free_tokens(rng, (B, Hkv, cap, d), [okc])
    v = _window_free_tokens(rng, (B, Hkv, cap, d), [ovc])
    K, V = tq.allocate_cache(gk, B, Hkv, cap), tq.allocate_cache(gv, B, Hkv, cap)
    kr, vr = tq.allocate_ring(B, Hkv, ring, d), tq.allocate_ring(B, Hkv, ring, d)
    kd, vd = to_device_f(k, True), to_device_f(v, True)
    # prefill each sequence: its whole rings compressed, the rest in its ring
    for b, n in enumerate(start):
        nc = ohybrid.compressed_length(n, ring)
        if nc:
            tq.tq_quantize_append_kv(gk, gv, kd[b:b + 1, :, :nc], vd[b:b + 1, :, :nc], _row_view(K, b),
                                     _row_view(V, b), torch.zeros(1, dtype=torch.int32, device="cuda"), nc)
        kr[b, :, :n - nc] = kd[b, :, nc:n]
        vr[b, :, :n - nc] = vd[b, :, nc:n]
    lens = list(start)
    scale = 1 / math.sqrt(d)
    ws = torch.zeros(tq.tq_hybrid_decode_workspace_size(gk, gv, B, Hq, Hkv, q_len, cap, ring), dtype=torch.uint8,
                     device="cuda")
    for step in range(steps):
        lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
        nk = torch.stack([kd[b, :, lens[b]:lens[b] + n_new] for b in range(B)])
        nv = torch.stack([vd[b, :, lens[b]:lens[b] + n_new] for b in range(B)])
        tq.tq_hybrid_append(gk, gv, nk, nv, K, V, kr, vr, lt, max(lens) + n_new)
        lens = [n + n_new for n in lens]
        torch.cuda.synchronize()
        # state: compressed part against the oracle's quantisation, ring exact
        gks, gvs = download(K), download(V)
        krh, vrh = kr.float().cpu().numpy(), vr.float().cpu().numpy()
        for b, n in enumerate(lens):
            nc = ohybrid.compressed_length(n, ring)
            for got, x, oc in ((gks, k, okc), (gvs, v, ovc)):
                if nc:
                    st = oquant.quantize(x[b:b + 1, :, :nc].astype(np.float64), oc)
                    assert np.array_equal(got["idx"][b, :, :nc], st["words"][0]), f"{name} step {step} row {b}"
                    if oc.mode != 2:
                        np.testing.assert_allclose(got["norm"][b, :, :nc], st["norm"][0], rtol=1e-6, atol=0)
                    if oc.mode == 3:
                        np.testing.assert_allclose(got["rnorm"][b, :, :nc], st["rnorm"][0], rtol=1e-6, atol=0)
            assert np.array_equal(krh[b, :, :n - nc], k[b, :, nc:n]), f"{name} step {step}: key ring of row {b}"
            assert np.array_equal(vrh[b, :, :n - nc], v[b, :, nc:n]), f"{name} step {step}: value ring of row {b}"
        # decode: every row over its compressed tokens and its ring
        q = round_bf16(rng.standard_normal((B, Hq, q_len, d)).astype(np.float32) * np.float32(1.0))
        out = torch.zeros((B, Hq, q_len, d), dtype=torch.float32, device="cuda")
        tq.tq_hybrid_decode_attention(gk, gv, to_device_f(q, True), K, V, kr, vr,
                                      torch.tensor(lens, dtype=torch.int32, device="cuda"), cap, scale, out, ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        want = ohybrid.hybrid_decode(q.astype(np.float64), k, v, lens, ring, okc, ovc, scale)
        err = rel_l2_rows(got, want)
        print(f"  step {step}: lens {lens}, max row rel L2 {err.max():.2e}", flush=True)
        assert err.max() <= 1e-4, f"{name} step {step}"


def test_hybrid_with_nothing_compressed_is_exact_attention():
    """Every sequence shorter than its ring: decode is exact softmax attention
    over the unquantised tokens (oracle.hybrid reduces to it), and the
    compressed caches are never touched."""
    print("hybrid, nothing compressed", flush=True)
    rng = np.random.default_rng(3)
    d, B, Hkv, Hq, ring = 128, 2, 2, 8, 64
    lens = [40, 7]
    gk, gv = tq.tq_codec_create(d, 3, 0, 0), tq.tq_codec_create(d, 3, 1, 0)
    okc, ovc = ocodec.make_codec(d, 3, 0, 0), ocodec.make_codec(d, 3, 1, 0)
    k = round_bf16(rng.standard_normal((B, Hkv, 64, d)).astype(np.float32) * np.float32(0.02))
    v = round_bf16(rng.standard_normal((B, Hkv, 64, d)).astype(np.float32) * np.float32(0.02))
    K, V = tq.allocate_cache(gk, B, Hkv, 8), tq.allocate_cache(gv, B, Hkv, 8)
    kr, vr = tq.allocate_ring(B, Hkv, ring, d), tq.allocate_ring(B, Hkv, ring, d)
    # fill the rings through the append path, one token at a time
    kd, vd = to_device_f(k, True), to_device_f(v, True)
    for t in range(max(lens)):
        lt = torch.tensor([min(t, n) for n in lens], dtype=torch.int32, device="cuda")
        tq.tq_hybrid_append(gk, gv, kd[:, :, t:t + 1].contiguous(), vd[:, :, t:t + 1].contiguous(), K, V, kr, vr,
                            lt, t + 1)
    torch.cuda.synchronize()
    assert not download(K)["idx"].any() and not download(V)["idx"].any()
    q = round_bf16(rng.standard_normal((B, Hq, 1, d)).astype(np.float32) * np.float32(0.5))
    out = torch.zeros((B, Hq, 1, d), dtype=torch.float32, device="cuda")
    ws = torch.zeros(tq.tq_hybrid_decode_workspace_size(gk, gv, B, Hq, Hkv, 1, 63, ring), dtype=torch.uint8,
                     device="cuda")
    tq.tq_hybrid_decode_attention(gk, gv, to_device_f(q, True), K, V, kr, vr,
                                  torch.tensor(lens, dtype=torch.int32, device="cuda"), 63, 1 / math.sqrt(d), out, ws)
    torch.cuda.synchronize()
    want = ohybrid.hybrid_decode(q.astype(np.float64), k, v, lens, ring, okc, ovc, 1 / math.sqrt(d))
    assert rel_l2_rows(out.cpu().numpy().astype(np.float64), want).max() <= 1e-4
