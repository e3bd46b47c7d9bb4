"""The append + decode calls captured in a HIP graph give the eager results on
every replay, with eager work and synchronisations between the replays."""
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
from quantized_decode_attention_04_amd import workloads as wl  # noqa: E402


@pytest.mark.parametrize("kspec,vspec,n", [((3, 0), (3, 0), 6000), ((3, 1), (4, 0), 3000)],
                         ids=["mse3_mse3_fast_path", "prod3_mse4_general_path"])
def test_graph_replays_match_eager(kspec, vspec, n):
    print(f"graph replay k={kspec} v={vspec} n={n}", flush=True)
    sys.stdout.flush()
    dev = torch.device("cuda")
    B, hkv, hq, d, qlen = 1, 8, 64, 128, 2
    gk = tq.tq_codec_create(d, kspec[0], 0, kspec[1])
    gv = tq.tq_codec_create(d, vspec[0], 1, vspec[1])
    layers = []
    for l in range(2):
        K = tq.allocate_cache(gk, B, hkv, n, dev)
        V = tq.allocate_cache(gv, B, hkv, n, dev)
        pos0 = torch.zeros(B, dtype=torch.int32, device=dev)
        kx = wl.device_normal((B, hkv, n - qlen, d), 3, l, 100, True, dev)
        vx = wl.device_normal((B, hkv, n - qlen, d), 3, l, 101, True, dev)
        tq.tq_quantize_append_kv(gk, gv, kx, vx, K, V, pos0, n - qlen)
        kn = wl.device_normal((B, hkv, qlen, d), 3, l, 102, True, dev)
        vn = wl.device_normal((B, hkv, qlen, d), 3, l, 103, True, dev)
        q = wl.device_normal((B, hq, qlen, d), 3, l, 104, True, dev)
        layers.append((K, V, kn, vn, q))
    pos = torch.full((B,), n - qlen, dtype=torch.int32, device=dev)
    lens = torch.full((B,), n, dtype=torch.int32, device=dev)
    ws = tq.allocate_workspace(gk, gv, B, hq, hkv, qlen, n, dev)
    scale = 1.0 / math.sqrt(d)
    outs = [torch.zeros((B, hq, qlen, d), dtype=torch.float32, device=dev) for _ in layers]

    def run(l):
        K, V, kn, vn, q = layers[l]
        tq.tq_quantize_append_kv(gk, gv, kn, vn, K, V, pos, n)
        tq.tq_decode_attention(gk, gv, q, K, V, lens, n, scale, outs[l], ws)

    # eager reference (warms the codec tables before capture)
    run(0)
    run(1)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=cap):
        run(0)
        run(1)
    for rep in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for l in range(2):
            assert torch.equal(outs[l], ref[l]), f"replay {rep} layer {l} differs from the eager result"
        # eager work between replays on the same buffers
        run(1)
        torch.cuda.synchronize()
        assert torch.equal(outs[1], ref[1])
    assert np.isfinite(ref[0].cpu().numpy()).all()


def test_decode_read_reference_runs_and_refuses_other_codecs():
    """The measurement kernel behind bench.py's decode_read_reference reads a
    ragged batch's state without error (its one possible write stays inside
    the sink) and refuses codecs the int8 decode kernel does not take."""
    print("decode read reference", flush=True)
    dev = torch.device("cuda")
    B, hkv, d, cap = 3, 2, 128, 5000
    kc = tq.tq_codec_create(d, 3, 0, tq.TQ_MODE_MSE)
    vc = tq.tq_codec_create(d, 3, 1, tq.TQ_MODE_MSE)
    K = tq.allocate_cache(kc, B, hkv, cap, dev)
    V = tq.allocate_cache(vc, B, hkv, cap, dev)
    pos0 = torch.zeros(B, dtype=torch.int32, device=dev)
    kx = wl.device_normal((B, hkv, cap, d), 5, 0, 100, True, dev)
    vx = wl.device_normal((B, hkv, cap, d), 5, 0, 101, True, dev)
    tq.tq_quantize_append_kv(kc, vc, kx, vx, K, V, pos0, cap)
    lens = torch.tensor([5000, 0, 777], dtype=torch.int32, device=dev)
    sink = torch.zeros(7, dtype=torch.int32, device=dev)
    tq.tq_decode_read_reference(kc, vc, K, V, lens, cap, sink)
    torch.cuda.synchronize()
    k4 = tq.tq_codec_create(d, 4, 0, tq.TQ_MODE_MSE)
    K4 = tq.allocate_cache(k4, B, hkv, cap, dev)
    with pytest.raises(tq.TQError, match="3-bit MSE"):
        tq.tq_decode_read_reference(k4, vc, K4, V, lens, cap, sink)
