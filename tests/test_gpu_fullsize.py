"""GPU parity at the full benchmark sizes, on sampled outputs.

Each case builds one layer of a benchmark workload at its real size on the
device, in the launch configuration bench.py times (bulk 65536-token appends,
then one decode call over every KV head, and one prefill call of 64 new
tokens per sequence):

* one sampled KV head's whole history is taken from the device *inputs*
  (seeded synthetic K and V, before quantisation) and quantised by the
  oracle; the GPU's state for that head must match it bit for bit outside
  the decision window (norms to 1e-6 relative);
* the oracle's state for that head is then written over the GPU's, the decode
  runs over all heads, and the sampled head's output rows must match the
  oracle's decode of its own state to relative L2 1e-4, and so must sampled
  rows of the prefill call (the first and last positions of the 64).

No oracle input comes from the HIP path: the oracle sees the generated
inputs only, and the GPU decodes the oracle's state.
"""
import math
import sys

import numpy as np
import pytest

from oracle import attention as oatt
from oracle import codec as ocodec
from oracle import packing
from oracle import quant as oquant
from tests.gpu_util import WINDOW, download, expected_window, rel_l2_rows, window_ceiling, words_i32

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


import quantized_decode_attention_04_amd as tq  # noqa: E402
from quantized_decode_attention_04_amd import workloads as wl  # noqa: E402

CHUNK = 65536


def _put_head(cache, state, mode, b, g, n):
    """Write an oracle state of one head ([1, 1, n, ...]) into cache[b, g, :n]."""
    dev = cache.idx.device
    cache.idx[b, g, :n] = torch.from_numpy(words_i32(state["words"][0, 0])).to(dev)
    if mode in (0, 1):
        cache.norm[b, g, :n] = torch.from_numpy(np.asarray(state["norm"][0, 0], dtype=np.float32)).to(dev)
    if mode == 1:
        cache.rnorm[b, g, :n] = torch.from_numpy(np.asarray(state["rnorm"][0, 0], dtype=np.float32)).to(dev)
        cache.sign[b, g, :n] = torch.from_numpy(words_i32(state["sign_words"][0, 0])).to(dev)
    if mode == 2:
        cache.scale[b, g, :n] = torch.from_numpy(np.asarray(state["scale"][0, 0], dtype=np.float32)).to(dev)
        cache.gmin[b, g, :n] = torch.from_numpy(np.asarray(state["min"][0, 0], dtype=np.float32)).to(dev)


def _check_state(got, ora, codec, tag):
    """GPU state of one head against the oracle's, outside the window."""
    mode, d = codec.mode, codec.head_dim
    if mode == 2:
        top = (1 << codec.bits) - 1
        q = packing.unpack(got["idx"], codec.bits, d)
        inwin = ora["margin"][0, 0] < WINDOW * top
        bad = (q != ora["q"][0, 0]) & ~inwin
        assert not bad.any(), f"{tag}: {int(bad.sum())} group codes differ outside the window"
        np.testing.assert_allclose(got["scale"], ora["scale"][0, 0], rtol=1e-6, atol=0)
        np.testing.assert_array_equal(got["gmin"], ora["min"][0, 0].astype(np.float32))
        return int(inwin.sum())
    idx = packing.unpack(got["idx"], codec.mse_bits, d)
    inwin = ora["margin"][0, 0] < WINDOW
    bad = (idx != ora["idx"][0, 0]) & ~inwin
    assert not bad.any(), f"{tag}: {int(bad.sum())} indices differ outside the window"
    np.testing.assert_allclose(got["norm"], ora["norm"][0, 0], rtol=1e-6, atol=0)
    nwin = int(inwin.sum())
    if mode == 1:
        ok = (idx == ora["idx"][0, 0]).all(-1)
        s = packing.unpack(got["sign"], 1, d)
        zwin = ora["zmargin"][0, 0] < WINDOW
        bad = (s != ora["sign_bits"][0, 0]) & ~zwin & ok[:, None]
        assert not bad.any(), f"{tag}: {int(bad.sum())} QJL signs differ outside the window"
        np.testing.assert_allclose(got["rnorm"][ok], ora["rnorm"][0, 0][ok], rtol=1e-6, atol=0)
        nwin += int((zwin & ok[:, None]).sum())
    return nwin


# workload, sampled (sequence, KV head), layer (the 64-layer workload is
# checked on its first, middle and last layer: their inputs and outlier
# channels differ)
CASES = [
    ("l64_d128_n256k_mse3_mtp2", 0, 5, 0),
    ("l64_d128_n256k_mse3_mtp2", 0, 2, 31),
    ("l64_d128_n256k_mse3_mtp2", 0, 7, 63),
    ("gqa8_d128_n32k_prod3_mse4", 0, 3, 0),
    ("moe_d256_n131k_prod3_group2", 0, 1, 0),
    ("ragged32_d128_prod3_mse4", None, 6, 0),   # None: the longest sequence
]

# floors of the mean cos-sim to unquantised attention (the oracle gives about
# 0.98, 0.996, 0.93 and 0.996 for these codec pairs on N(0, 0.02^2) inputs)
QUALITY_FLOOR = {
    "l64_d128_n256k_mse3_mtp2": 0.95,
    "gqa8_d128_n32k_prod3_mse4": 0.98,
    "moe_d256_n131k_prod3_group2": 0.90,
    "ragged32_d128_prod3_mse4": 0.98,
}


@pytest.mark.parametrize("name,b,g,layer", CASES, ids=[f"{c[0]}-layer{c[3]}" for c in CASES])
def test_full_size_layer_sampled_head(name, b, g, layer):
    w = wl.configs()[name]
    dev = torch.device("cuda")
    lens = w.lens()
    B, Hkv, Hq, d, qlen = w.batch, w.hkv, w.hq, w.d, w.q_len
    max_len = int(lens.max())
    if b is None:
        b = int(np.argmax(lens))
    n_b = int(lens[b])
    tag = f"{name} layer={layer} b={b} g={g} len={n_b}"
    _say(f"full size {tag}")
    gk = tq.tq_codec_create(d, w.kbits, 0, w.kmode)
    gv = tq.tq_codec_create(d, w.vbits, 1, w.vmode)
    kc = ocodec.make_codec(d, w.kbits, 0, w.kmode)
    vc = ocodec.make_codec(d, w.vbits, 1, w.vmode)
    K = tq.allocate_cache(gk, B, Hkv, max_len, dev)
    V = tq.allocate_cache(gv, B, Hkv, max_len, dev)
    ksc = wl.outlier_scales(0, layer, Hkv, d, 0) if w.outliers else None
    vsc = wl.outlier_scales(0, layer, Hkv, d, 1) if w.outliers else None
    # every position of every sequence gets a token (positions past a ragged
    # sequence's length are never attended), in bulk appends like bench.py
    k_head, v_head = [], []
    for s0 in range(0, max_len, CHUNK):
        n = min(CHUNK, max_len - s0)
        pos = torch.full((B,), s0, dtype=torch.int32, device=dev)
        kx = wl.device_normal((B, Hkv, n, d), 0, layer, 100 + s0 // CHUNK, w.bf16, dev, ksc)
        vx = wl.device_normal((B, Hkv, n, d), 0, layer, 200000 + s0 // CHUNK, w.bf16, dev, vsc)
        tq.tq_quantize_append_kv(gk, gv, kx, vx, K, V, pos, s0 + n)
        k_head.append(kx[b, g].float().cpu().numpy())
        v_head.append(vx[b, g].float().cpu().numpy())
        del kx, vx
    torch.cuda.synchronize()
    kh = np.concatenate(k_head)[:n_b][None, None].astype(np.float64)
    vh = np.concatenate(v_head)[:n_b][None, None].astype(np.float64)
    ks = oquant.quantize(kh, kc)
    vs = oquant.quantize(vh, vc)
    sl = slice(0, n_b)
    gotk = {k: a[b, g, sl] for k, a in download(K).items()}
    gotv = {k: a[b, g, sl] for k, a in download(V).items()}
    wk = _check_state(gotk, ks, kc, tag + " keys")
    wv = _check_state(gotv, vs, vc, tag + " values")
    lk, lv = expected_window(kc, n_b), expected_window(vc, n_b)
    _say(f"  state matches; window coordinates K {wk} (expected {lk:.0f}), V {wv} (expected {lv:.0f})"
         f" of {n_b * d} each")
    # (group codes of bf16 values have exact half-way ties the continuous
    # model does not count: no bound for them)
    assert wk <= window_ceiling(lk) and (vc.mode == ocodec.MODE_GROUP or wv <= window_ceiling(lv))

    _put_head(K, ks, w.kmode, b, g, n_b)
    _put_head(V, vs, w.vmode, b, g, n_b)
    q = wl.device_normal((B, Hq, qlen, d), 0, layer, wl.STREAM_Q, w.bf16, dev)
    out = torch.zeros((B, Hq, qlen, d), dtype=torch.float32, device=dev)
    ws = tq.allocate_workspace(gk, gv, B, Hq, Hkv, qlen, max_len, dev)
    ld = torch.tensor(lens, dtype=torch.int32, device=dev)
    scale = 1.0 / math.sqrt(d)
    tq.tq_decode_attention(gk, gv, q, K, V, ld, max_len, scale, out, ws)
    torch.cuda.synchronize()
    G = Hq // Hkv
    got = out[b, g * G:(g + 1) * G].cpu().numpy().astype(np.float64)[None]
    qh = q[b, g * G:(g + 1) * G].float().cpu().numpy().astype(np.float64)[None]
    want = oatt.decode_attention_rotated(qh, ks, kc, vs, vc, np.array([n_b]), scale)
    err = rel_l2_rows(got, want)
    _say(f"  decode max row rel L2 {err.max():.3e} over {err.size} rows")
    assert err.max() <= 1e-4
    # quality: cos-sim of the GPU output to exact attention on the unquantised
    # inputs of the sampled head ("turboquant validate_moe_phase2.py", Test 1)
    ref = oatt.reference_attention(qh, kh, vh, np.array([n_b]), scale)
    cos = np.sum(got * ref, -1) / (np.linalg.norm(got, axis=-1) * np.linalg.norm(ref, axis=-1))
    _say(f"  cos-sim to unquantised attention: mean {cos.mean():.6f} min {cos.min():.6f}")
    assert cos.mean() >= QUALITY_FLOOR[name]

    # prefill at the bench's size: 64 new tokens of every sequence (the last
    # 64 cached positions, causal among themselves) over the same cache, every
    # row of every KV head in one call; the sampled head's first and last four
    # positions of its first and last query head against the oracle.  A slice
    # of rows i0 .. i0+3 goes to the oracle as a 4-row call over the first
    # n_b - 64 + i0 + 4 tokens, which gives its rows the same visible tokens.
    pq = 64
    qp = wl.device_normal((B, Hq, pq, d), 0, 0, 902, w.bf16, dev)
    outp = torch.zeros((B, Hq, pq, d), dtype=torch.float32, device=dev)
    wsp = tq.allocate_prefill_workspace(gk, gv, B, Hq, Hkv, pq, max_len, dev)
    tq.tq_prefill_attention(gk, gv, qp, K, V, ld, max_len, scale, outp, wsp)
    torch.cuda.synchronize()
    heads = [g * G, g * G + G - 1]
    for i0 in (0, pq - 4):
        gotp = outp[b, heads, i0:i0 + 4].cpu().numpy().astype(np.float64)[None]
        qs_ = qp[b, heads, i0:i0 + 4].float().cpu().numpy().astype(np.float64)[None]
        wantp = oatt.decode_attention_rotated(qs_, ks, kc, vs, vc, np.array([n_b - pq + i0 + 4]), scale)
        errp = rel_l2_rows(gotp, wantp)
        _say(f"  prefill rows {i0}..{i0 + 3} of query heads {heads}: max row rel L2 {errp.max():.3e}")
        assert errp.max() <= 1e-4
