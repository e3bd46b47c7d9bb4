"""The decode entry point that allocates nothing (tq_decode_attention_noalloc,
for callers that cannot allocate device memory) against tq_decode_attention
with a caller workspace: the same kernels and plan, so the outputs must be
identical, on two calls in a row -- the second with a smaller input, so that
it reads a library scratch array that still holds the first call's partials."""
import ctypes
import math
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


import quantized_decode_attention_04_amd as tq  # noqa: E402
from quantized_decode_attention_04_amd import _binding  # noqa: E402
from quantized_decode_attention_04_amd import workloads as wl  # noqa: E402


def _case(kc, vc, B, hkv, hq, q_len, n, seed):
    dev = torch.device("cuda")
    K, V = tq.allocate_cache(kc, B, hkv, n, dev), tq.allocate_cache(vc, B, hkv, n, dev)
    pos = torch.zeros(B, dtype=torch.int32, device=dev)
    tq.tq_quantize_append_kv(kc, vc, wl.device_normal((B, hkv, n, 128), seed, 0, 1, True, dev),
                             wl.device_normal((B, hkv, n, 128), seed, 0, 2, True, dev), K, V, pos, n)
    q = wl.device_normal((B, hq, q_len, 128), seed, 0, 3, True, dev)
    lens = torch.full((B,), n, dtype=torch.int32, device=dev)
    return K, V, q, lens


@pytest.mark.parametrize("kmode", [tq.TQ_MODE_MSE, tq.TQ_MODE_PROD], ids=["int8_path", "general_path"])
def test_noalloc_decode_matches_workspace_decode_twice(kmode):
    print(f"no-alloc decode, key mode {kmode}", flush=True)
    sys.stdout.flush()
    kc = tq.tq_codec_create(128, 3, 0, kmode)
    vc = tq.tq_codec_create(128, 3, 1, tq.TQ_MODE_MSE)
    tq.tq_codec_upload(kc)
    tq.tq_codec_upload(vc)
    scale = 1.0 / math.sqrt(128)
    # a larger call, then a smaller one (fewer heads, tokens and rows)
    for (B, hkv, hq, q_len, n, seed) in ((1, 8, 64, 2, 40000, 1), (2, 2, 8, 1, 3000, 2)):
        K, V, q, lens = _case(kc, vc, B, hkv, hq, q_len, n, seed)
        want = torch.zeros((B, hq, q_len, 128), dtype=torch.float32, device="cuda")
        ws = tq.allocate_workspace(kc, vc, B, hq, hkv, q_len, n)
        tq.tq_decode_attention(kc, vc, q, K, V, lens, n, scale, want, ws)
        got = torch.full((B, hq, q_len, 128), float("nan"), dtype=torch.float32, device="cuda")
        tq.tq_decode_attention_noalloc(kc, vc, q, K, V, lens, n, scale, got)
        torch.cuda.synchronize()
        g, w_ = got.cpu().numpy(), want.cpu().numpy()
        assert np.isfinite(g).all()
        err = np.linalg.norm(g - w_, axis=-1) / np.linalg.norm(w_, axis=-1)
        assert err.max() <= 1e-4
        assert np.array_equal(g, w_)           # same kernels, same plan: identical


def test_noalloc_refusals():
    """Refused on the host before any launch: a codec whose tables are not on
    the device yet (uploading would allocate), and sizes whose partials exceed
    the library's 64 MiB scratch array."""
    kc = tq.tq_codec_create(128, 3, 0, tq.TQ_MODE_MSE)
    vc = tq.tq_codec_create(128, 3, 1, tq.TQ_MODE_MSE)
    dev = torch.device("cuda")
    K, V = tq.allocate_cache(kc, 1, 2, 512, dev), tq.allocate_cache(vc, 1, 2, 512, dev)
    q = torch.zeros((1, 16, 1, 128), dtype=torch.bfloat16, device=dev)
    lens = torch.full((1,), 512, dtype=torch.int32, device=dev)
    out = torch.zeros((1, 16, 1, 128), dtype=torch.float32, device=dev)
    with pytest.raises(tq.TQError) as e:
        tq.tq_decode_attention_noalloc(kc, vc, q, K, V, lens, 512, 0.1, out)  # tables never uploaded
    assert e.value.status == 1 and "tq_codec_upload" in str(e.value)
    tq.tq_codec_upload(kc)
    tq.tq_codec_upload(vc)
    # 4096 sequences x 64 KV heads x 8 rows at 65536 tokens: far above 64 MiB of
    # partials; refused by size before the caches are looked at
    need = tq.tq_decode_workspace_size(kc, vc, 4096, 512, 64, 1, 65536)
    assert need > 64 << 20
    fake = _binding._Cache(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 4096, 64, 65536)
    st = _binding._lib.tq_decode_attention_noalloc(kc.handle, vc.handle, ctypes.c_void_p(0x1000), 1, 4096, 512, 64, 1,
                                                   ctypes.byref(fake), ctypes.byref(fake), ctypes.c_void_p(0x1000),
                                                   65536, ctypes.c_float(0.1), ctypes.c_void_p(0x1000), None)
    assert st == 5 and "scratch" in tq.tq_last_error()
