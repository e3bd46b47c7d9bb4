"""C ABI of libtq.so on the host: exports, codec tables against the oracle,
state sizes, and argument validation (no device work is started)."""
import ctypes
import math
import os
import re
import subprocess

import numpy as np
import pytest

import quantized_decode_attention_04_amd as tq
from quantized_decode_attention_04_amd import _binding
from oracle import codec as ocodec
from oracle import packing

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "tq.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 10
    out = subprocess.run(["nm", "-D", "--defined-only", tq.lib_path()], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (tq_[a-z_]+)$", out, flags=re.M))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = ctypes.CDLL(tq.lib_path())
    for n in names:
        getattr(lib, n)
    assert set(_binding.EXPORTED) == set(names)


CODECS = [(32, 1, 3, 0), (64, 4, 9, 0), (96, 2, 4, 0), (128, 3, 0, 0), (128, 4, 1, 0), (128, 3, 0, 1),
          (256, 3, 0, 1), (256, 2, 7, 0), (160, 5, 2, 1), (224, 3, 5, 0)]


@pytest.mark.parametrize("d,bits,seed,mode", CODECS)
def test_codec_tables_match_oracle(d, bits, seed, mode):
    c = tq.tq_codec_create(d, bits, seed, mode)
    t = tq.tq_codec_export(c)
    o = ocodec.make_codec(d, bits, seed, mode)
    # the two builders share no code; float64 results agree to rounding, so
    # the float32 tables agree to one float32 ulp at most
    assert np.abs(t["rot"] - o.rot).max() <= 1e-6
    assert np.array_equal(t["centroids"], o.centroids.astype(np.float32))
    assert np.array_equal(t["boundaries"], o.boundaries.astype(np.float32))
    if mode == ocodec.MODE_PROD:
        assert np.abs(t["sketch"] - o.sketch).max() <= 1e-6 * max(1.0, np.abs(o.sketch).max())
    assert c.info["grid_exp"] == o.grid_exp
    r = t["rot"].astype(np.float64)
    assert np.abs(r.T @ r - np.eye(d)).max() < 1e-5


@pytest.mark.parametrize("d,bits,seed", [(128, 3.5, 0), (128, 2.25, 7), (256, 2.5, 3), (96, 1.5, 1)])
def test_split_codec_tables_match_oracle(d, bits, seed):
    """Each part of a split codec is the oracle's MSE codec of that part (the
    high part's rotation from stream 2 of the seed); the split codec exports
    the block-diagonal rotation."""
    c = tq.tq_codec_create_split(d, bits, seed)
    o = ocodec.make_split_codec(d, bits, seed)
    assert c.info["mode"] == tq.TQ_MODE_SPLIT and c.info["split_high_dim"] == o.d_hi
    assert c.info["idx_words"] == o.d_lo * o.low.bits // 32 + o.d_hi * o.high.bits // 32
    assert c.info["bytes_per_token"] == 4 * c.info["idx_words"] + 8
    for which, oc in ((0, o.low), (1, o.high)):
        part = tq.tq_codec_part(c, which)
        t = tq.tq_codec_export(part)
        assert part.info["head_dim"] == oc.head_dim and part.info["bits"] == oc.bits
        assert np.abs(t["rot"] - oc.rot).max() <= 1e-6
        assert np.array_equal(t["centroids"], oc.centroids.astype(np.float32))
        assert np.array_equal(t["boundaries"], oc.boundaries.astype(np.float32))
    whole = tq.tq_codec_export(c)["rot"]
    assert np.array_equal(whole[:o.d_lo, :o.d_lo], tq.tq_codec_export(tq.tq_codec_part(c, 0))["rot"])
    assert np.array_equal(whole[o.d_lo:, o.d_lo:], tq.tq_codec_export(tq.tq_codec_part(c, 1))["rot"])
    assert not whole[:o.d_lo, o.d_lo:].any() and not whole[o.d_lo:, :o.d_lo].any()


@pytest.mark.parametrize("bits", [3.5, 2.5, 3.0, 2.9999995, 3.25])
def test_kv_codec_pair_follows_the_rebuild_rule(bits):
    k, v = tq.tq_codec_create_kv(128, bits, 11)
    ok, ov = ocodec.kv_codecs(128, bits, 11)
    for g, o in ((k, ok), (v, ov)):
        assert (g.info["bits"], g.info["mode"], g.info["seed"]) == (o.bits, ocodec.MODE_MSE, o.seed)
        assert np.array_equal(tq.tq_codec_export(g)["centroids"], o.centroids.astype(np.float32))


def test_codec_is_rebuilt_identically():
    a = tq.tq_codec_export(tq.tq_codec_create(128, 3, 42, 1))
    b = tq.tq_codec_export(tq.tq_codec_create(128, 3, 42, 1))
    c = tq.tq_codec_export(tq.tq_codec_create(128, 3, 43, 1))
    for k in a:
        assert a[k].tobytes() == b[k].tobytes()
    assert a["rot"].tobytes() != c["rot"].tobytes()


@pytest.mark.parametrize("d,bits,mode,want", [
    (128, 3, 0, 52),      # 12 words + norm
    (128, 3, 1, 56),      # 8 words + 4 sign words + norm + residual norm
    (128, 4, 0, 68),      # 16 words + norm
    (256, 3, 1, 104),     # 16 + 8 sign words + 2 norms
    (256, 2, 2, 128),     # 16 words + 8 scales + 8 minima
])
def test_state_sizes(d, bits, mode, want):
    c = tq.tq_codec_create(d, bits, 0, mode)
    info = c.info
    assert info["bytes_per_token"] == want
    mse_bits = bits - 1 if mode == 1 else bits
    assert info["idx_words"] == packing.words_per_vector(d, mse_bits) == math.ceil(d * mse_bits / 32)
    assert info["sign_words"] == (d // 32 if mode == 1 else 0)
    assert info["groups"] == (d // 32 if mode == 2 else 0)


def test_create_rejects_bad_parameters():
    for args in [(100, 3, 0, 0), (0, 3, 0, 0), (288, 3, 0, 0), (128, 0, 0, 0), (128, 5, 0, 0),
                 (128, 1, 0, 1), (128, 6, 0, 1), (128, 5, 0, 2), (128, 3, 0, 7)]:
        with pytest.raises(tq.TQError) as e:
            tq.tq_codec_create(*args)
        assert e.value.status == 2, args
    lib = _binding._lib
    assert lib.tq_codec_create(128, 3, 0, 0, None) == 1
    assert lib.tq_codec_get_info(None, None) == 1
    assert lib.tq_codec_export(None, None, None, None, None) == 1
    lib.tq_codec_destroy(None)   # no-op


@pytest.fixture
def no_gpu():
    import torch
    if torch.cuda.is_available():
        # every call below is refused on the host before a launch, but the
        # pointers are placeholders: if a check ever regressed, a GPU host
        # would launch a kernel on them, so these run where no GPU is present
        # (the CPU suite, every time)
        pytest.skip("argument-validation tests pass placeholder pointers; they run on hosts without a GPU")


def test_decode_shape_validation():
    kc = tq.tq_codec_create(128, 3, 0, tq.TQ_MODE_MSE)
    vc = tq.tq_codec_create(128, 4, 1, tq.TQ_MODE_MSE)
    vg = tq.tq_codec_create(128, 2, 1, tq.TQ_MODE_GROUP)
    v64 = tq.tq_codec_create(64, 3, 1, tq.TQ_MODE_MSE)
    kp = tq.tq_codec_create(128, 3, 0, tq.TQ_MODE_PROD)
    ws = lambda *a: tq.tq_decode_workspace_size(*a)
    assert ws(kc, vc, 1, 64, 8, 2, 262144) > 0
    assert ws(kp, vg, 2, 16, 2, 1, 1000) > ws(kc, vg, 2, 16, 2, 1, 1000)   # Prod adds S q
    for args, status in [
        ((vg, vc, 1, 8, 8, 1, 10), 2),       # group keys unsupported
        ((kc, kp, 1, 8, 8, 1, 10), 2),       # Prod values unsupported
        ((kc, v64, 1, 8, 8, 1, 10), 3),      # head_dim mismatch
        ((kc, vc, 1, 12, 8, 1, 10), 1),      # hq not a multiple of hkv
        ((kc, vc, 1, 8, 8, 0, 10), 1),       # q_len 0
        ((kc, vc, 1, 8, 8, 1, 0), 1),        # max_len 0
        ((kc, vc, 1, 68, 2, 1, 10), 2),      # 34 rows per KV head
    ]:
        with pytest.raises(tq.TQError) as e:
            ws(*args)
        assert e.value.status == status, args


def test_prefill_workspace_is_one_row_block():
    """Prefill takes any q_len and plans its workspace for one launch of rows,
    which the launches reuse: a decode block (16 rows up to head_dim 128, 8
    above), or on the shared-tile kernels above that up to 1024 rows (the
    rotated queries and every chunk's partial of each row)."""
    kc = tq.tq_codec_create(128, 3, 0, tq.TQ_MODE_MSE)
    vc = tq.tq_codec_create(128, 3, 1, tq.TQ_MODE_MSE)
    kp = tq.tq_codec_create(256, 3, 0, tq.TQ_MODE_PROD)
    vg = tq.tq_codec_create(256, 2, 1, tq.TQ_MODE_GROUP)
    pre, dec = tq.tq_prefill_workspace_size, tq.tq_decode_workspace_size
    assert pre(kc, vc, 1, 8, 1, 2, 5000) == dec(kc, vc, 1, 8, 1, 2, 5000)      # 16 rows: one block
    many = pre(kc, vc, 1, 8, 1, 512, 5000)                                    # 4096 rows: 1024-row launches
    assert many == pre(kc, vc, 1, 8, 1, 128, 5000)                            # 1024 rows
    assert many >= 1024 * 128 * 4 * 2                                         # q_rot + at least one chunk
    assert pre(kc, vc, 1, 8, 1, 5, 5000) < many                               # 40 rows
    assert pre(kp, vg, 1, 2, 1, 4, 5000) == dec(kp, vg, 1, 8, 1, 1, 5000)      # d 256, 8 rows: one block
    big = pre(kp, vg, 1, 2, 1, 300, 5000)                                     # 600 rows: shared tiles
    assert big >= 600 * 256 * 4 * 3                                           # q_rot, S q_rot, one chunk
    with pytest.raises(tq.TQError) as e:
        dec(kc, vc, 1, 8, 1, 3, 5000)                                         # 24 rows: not a decode step
    assert e.value.status == 2
    with pytest.raises(tq.TQError) as e:
        pre(kc, vc, 1, 8, 1, 0, 5000)
    assert e.value.status == 1


def _fake_cache(batch, heads, cap, mode):
    fake = 0x1000
    c = _binding._Cache(fake, fake, fake, fake, fake, fake, batch, heads, cap)
    if mode == 2:
        c.norm = None
    return c


def test_decode_and_append_argument_errors(no_gpu):
    lib = _binding._lib
    kc = tq.tq_codec_create(128, 3, 0, tq.TQ_MODE_MSE)
    vc = tq.tq_codec_create(128, 3, 1, tq.TQ_MODE_MSE)
    P = ctypes.c_void_p(0x1000)
    k, v = _fake_cache(1, 8, 100, 0), _fake_cache(1, 8, 100, 0)
    need = tq.tq_decode_workspace_size(kc, vc, 1, 64, 8, 1, 100)

    def dec(kcache=k, vcache=v, max_len=100, ws_bytes=need, q=P, scale=0.1, batch=1):
        return lib.tq_decode_attention(kc.handle, vc.handle, q, 1, batch, 64, 8, 1, ctypes.byref(kcache),
                                       ctypes.byref(vcache), P, max_len, ctypes.c_float(scale), P, P, ws_bytes, None)

    assert dec(q=None) == 1
    assert dec(scale=float("nan")) == 1
    assert dec(ws_bytes=need - 1) == 5
    assert dec(max_len=101) == 4
    # longest supported sequence: 2^26 tokens (int32 accumulator and merge bounds)
    huge = _fake_cache(1, 8, (1 << 26) + 1, 0)
    assert dec(kcache=huge, vcache=huge, max_len=(1 << 26) + 1) == 2
    assert "max_len above" in tq.tq_last_error()
    assert dec(vcache=_fake_cache(1, 8, 99, 0), max_len=50) == 3
    assert dec(kcache=_fake_cache(1, 4, 100, 0)) == 3
    bad = _fake_cache(1, 8, 100, 0)
    bad.norm = None
    assert dec(kcache=bad) == 1
    # append
    strides = (ctypes.c_int64 * 4)(8 * 2 * 128, 2 * 128, 128, 1)
    app = lambda cache, x=P, n=2, st=strides, dt=1, end=100: lib.tq_quantize_append(
        kc.handle, x, dt, 1, 8, n, st, ctypes.byref(cache), P, end, None)
    assert app(k, x=None) == 1
    assert app(k, dt=5) == 1
    assert app(k, n=-1) == 1
    assert app(_fake_cache(2, 8, 100, 0)) == 3
    assert app(k, st=(ctypes.c_int64 * 4)(0, 0, 0, 2)) == 1
    assert "coordinate stride" in tq.tq_last_error()
    # the written end after the append is bounded on the host: past the
    # capacity is CAPACITY, below n_new is INVALID_ARG
    assert app(k, end=101) == 4
    assert "capacity" in tq.tq_last_error()
    assert app(k, end=1) == 1
    assert app(k, n=0, end=0) == 0             # nothing to do
    appkv = lambda end: lib.tq_quantize_append_kv(kc.handle, kc.handle, P, P, 1, 1, 8, 2, strides, strides,
                                                   ctypes.byref(k), ctypes.byref(_fake_cache(1, 8, 50, 0)), P, end,
                                                   None)
    assert appkv(51) == 4                      # past the smaller (value) cache
    assert appkv(1) == 1


def test_cache_gather_argument_errors(no_gpu):
    """Record copies are refused before any launch when the codecs differ (the
    pages' merge guard on bits and seed), heads differ, an index or range is
    out of bounds, or too many destination sequences are asked for."""
    lib = _binding._lib
    kc = tq.tq_codec_create(128, 3, 0, tq.TQ_MODE_MSE)
    other_seed = tq.tq_codec_create(128, 3, 5, tq.TQ_MODE_MSE)
    other_bits = tq.tq_codec_create(128, 4, 0, tq.TQ_MODE_MSE)
    src, dst = _fake_cache(3, 2, 100, 0), _fake_cache(2, 2, 50, 0)

    def gather(sc=kc, s=src, dc=kc, d=dst, sb=(2, 0), st=(0, 0), n=(40, 50)):
        m = d.batch
        arr = lambda xs: (ctypes.c_int32 * m)(*xs)
        return lib.tq_cache_gather(sc.handle, ctypes.byref(s), dc.handle, ctypes.byref(d), arr(sb), arr(st), arr(n),
                                   None)

    assert gather(dc=other_seed) == 3
    assert gather(dc=other_bits) == 3
    assert gather(d=_fake_cache(2, 4, 50, 0)) == 3            # head counts differ
    assert gather(sb=(3, 0)) == 1                             # source sequence out of range
    assert gather(st=(-1, 0)) == 1
    assert gather(st=(70, 0)) == 4                            # 70 + 40 > source cap 100
    assert gather(n=(40, 51)) == 4                            # above destination cap 50
    assert gather(sb=(-1, -1)) == 0                           # nothing to copy: no launch
    big = _fake_cache(257, 2, 50, 0)
    assert gather(d=big, sb=[-1] * 257, st=[0] * 257, n=[0] * 257) == 2
    bad = _fake_cache(3, 2, 100, 0)
    bad.idx = None
    assert gather(s=bad) == 1


def test_decode_read_reference_argument_errors(no_gpu):
    """The decode-pattern read reference refuses other codecs, mismatched
    caches and lengths outside 1..cap before any launch."""
    lib = _binding._lib
    kc = tq.tq_codec_create(128, 3, 0, tq.TQ_MODE_MSE)
    vc = tq.tq_codec_create(128, 3, 1, tq.TQ_MODE_MSE)
    k4 = tq.tq_codec_create(128, 4, 0, tq.TQ_MODE_MSE)
    P = ctypes.c_void_p(0x1000)
    k, v = _fake_cache(1, 8, 100, 0), _fake_cache(1, 8, 100, 0)

    def rd(kcodec=kc, kcache=k, vcache=v, max_len=100, sink=P, words=1, batch=1, heads=8):
        return lib.tq_decode_read_reference(kcodec.handle, vc.handle, batch, heads, ctypes.byref(kcache),
                                            ctypes.byref(vcache), P, max_len, sink, words, None)

    assert rd(sink=None) == 1
    assert rd(words=0) == 1
    assert rd(kcodec=k4) == 2
    assert "3-bit MSE" in tq.tq_last_error()
    assert rd(heads=4) == 3
    assert rd(vcache=_fake_cache(1, 8, 99, 0), max_len=50) == 3
    assert rd(max_len=101) == 4
    assert rd(max_len=0) == 4
    bad = _fake_cache(1, 8, 100, 0)
    bad.idx = None
    assert rd(kcache=bad) == 1


def test_hybrid_argument_errors(no_gpu):
    """The hybrid entry points refuse NULL or misaligned rings, a bad ring
    dtype or size and a short workspace on the host, before any launch."""
    lib = _binding._lib
    kc = tq.tq_codec_create(128, 3, 0, tq.TQ_MODE_MSE)
    vc = tq.tq_codec_create(128, 3, 1, tq.TQ_MODE_MSE)
    P = ctypes.c_void_p(0x1000)
    k, v = _fake_cache(1, 8, 256, 0), _fake_cache(1, 8, 256, 0)
    need = tq.tq_hybrid_decode_workspace_size(kc, vc, 1, 64, 8, 1, 256, 128)

    def dec(kbuf=P, vbuf=P, dtype=tq.TQ_BF16, buf=128, ws_bytes=need):
        return lib.tq_hybrid_decode_attention(kc.handle, vc.handle, P, tq.TQ_BF16, 1, 64, 8, 1, ctypes.byref(k),
                                              ctypes.byref(v), kbuf, vbuf, dtype, buf, P, 256, ctypes.c_float(0.1),
                                              P, P, ws_bytes, None)

    strides = (ctypes.c_int64 * 4)(8 * 128, 128, 128, 1)

    def app(kbuf=P, vbuf=P, buf=128, n_new=1):
        return lib.tq_hybrid_append(kc.handle, vc.handle, P, P, tq.TQ_BF16, 1, 8, n_new, strides, strides,
                                    ctypes.byref(k), ctypes.byref(v), kbuf, vbuf, buf, P, 200, None)

    for call in (dec, app):
        assert call(kbuf=None) == 1
        assert call(vbuf=ctypes.c_void_p(0x1008)) == 1
        assert "16-byte aligned" in tq.tq_last_error()
        assert call(buf=0) == 1
    assert dec(dtype=7) == 1
    assert dec(ws_bytes=need - 1) == 5  # TQ_ERR_WORKSPACE
    assert app(n_new=129) == 2  # TQ_ERR_UNSUPPORTED
