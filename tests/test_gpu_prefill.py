"""GPU parity of prefill attention over the compressed cache: q_len new tokens
(up to the whole sequence) attend to the cache and causally to each other,
the query rows of each KV head being processed in blocks.  The GPU decodes the
oracle's packed state, and its output is compared with the oracle's decode of
that state (relative L2 per row <= 1e-4)."""
import math
import sys
import zlib

import numpy as np
import pytest

from oracle import attention as oatt
from oracle import codec as ocodec
from oracle import quant as oquant
from tests.gpu_util import rel_l2_rows, to_device_f, upload_state

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


import quantized_decode_attention_04_amd as tq  # noqa: E402
from quantized_decode_attention_04_amd.workloads import round_bf16  # noqa: E402

# name, d, (kbits, kmode), (vbits, vmode), B, Hkv, Hq, q_len, lens, cap, bf16, query std
CASES = [
    # matrix-core path: 8 * 5 = 40 rows per KV head -> blocks of 16, 16, 8
    ("fast_g8_q5", 128, (3, 0), (3, 0), 2, 2, 16, 5, [700, 1234], 1300, True, 0.02),
    # every token is new: row i sees tokens 0..i (200 rows, 13 blocks)
    ("fast_self_attention_q100", 128, (3, 0), (3, 0), 1, 1, 2, 100, [100], 128, False, 1.0),
    # sharp softmax over 33 rows (blocks 16, 16, 1)
    ("fast_sharp_q33", 128, (3, 0), (3, 0), 1, 1, 1, 33, [600], 640, False, 200.0),
    # a sequence shorter than q_len: its first rows see no token
    ("fast_short_sequence", 128, (3, 0), (3, 0), 2, 1, 4, 8, [5, 300], 320, True, 0.02),
    # 512 rows per KV head (four 128-row workgroups) over a ragged batch of
    # several chunks of 64-token tiles
    ("fast_512_rows_ragged", 128, (3, 0), (3, 0), 2, 2, 16, 32, [5000, 2100], 5000, True, 0.02),
    # 1100 rows: two launches (1024 + 76 rows), the second's row groups partly empty
    ("fast_1100_rows_two_launches", 128, (3, 0), (3, 0), 1, 1, 4, 275, [300], 320, False, 1.0),
    # general path: Prod keys, 4-bit values, 36 rows
    ("general_prod3_mse4_q9", 128, (3, 1), (4, 0), 2, 2, 8, 9, [513, 77], 600, True, 0.02),
    # shared-tile kernel of the bf16 / int8 codecs (head_dim 128): 256 rows per
    # KV head (two 128-row workgroups) over a ragged batch of several chunks
    ("bf16_prod3_mse4_256_rows_ragged", 128, (3, 1), (4, 0), 2, 2, 16, 16, [5000, 2100], 5000, True, 0.02),
    # group values, MSE keys of 2 bits, 40 rows (one workgroup, its last 88 rows empty)
    ("bf16_mse2_group2_q5", 128, (2, 0), (2, 2), 1, 2, 16, 5, [1500], 1536, True, 0.02),
    # 1-bit key codes with QJL signs, 1-bit values, a sharp softmax over 33 rows
    ("bf16_prod2_mse1_sharp_q33", 128, (2, 1), (1, 0), 1, 1, 1, 33, [777], 800, False, 200.0),
    # 2-bit values; every token new (row i sees tokens 0..i), 130 rows
    ("bf16_prod3_mse2_self_attention_q130", 128, (3, 1), (2, 0), 1, 1, 1, 130, [130], 160, False, 1.0),
    # 1100 rows: two launches (1024 + 76 rows)
    ("bf16_prod3_mse4_1100_rows_two_launches", 128, (3, 1), (4, 0), 1, 1, 4, 275, [300], 320, False, 1.0),
    # the same kernel at head_dim 256 (64-row workgroups over 32-token tiles):
    # Prod keys and group values, 14 rows (one workgroup, its last 50 rows empty)
    ("bf16_d256_prod3_group2_q7", 256, (3, 1), (2, 2), 1, 1, 2, 7, [300], 320, True, 0.02),
    # 192 rows per KV head (three workgroups) over a ragged batch of several chunks
    ("bf16_d256_prod3_group2_192_rows_ragged", 256, (3, 1), (2, 2), 2, 2, 16, 24, [3000, 1100], 3000, True, 0.02),
    # MSE keys of 2 bits, 4-bit values, 80 rows
    ("bf16_d256_mse2_mse4_q40", 256, (2, 0), (4, 0), 1, 1, 2, 40, [900], 960, False, 1.0),
    # 1-bit key codes with QJL signs, 1-bit values, a sharp softmax over 33 rows
    ("bf16_d256_prod2_mse1_sharp_q33", 256, (2, 1), (1, 0), 1, 1, 1, 33, [700], 704, False, 200.0),
    # 2-bit values; every token new, 70 rows
    ("bf16_d256_prod3_mse2_self_attention_q70", 256, (3, 1), (2, 0), 1, 1, 1, 70, [70], 96, False, 1.0),
    # 1100 rows: two launches (1024 + 76 rows)
    ("bf16_d256_prod3_group2_1100_rows_two_launches", 256, (3, 1), (2, 2), 1, 1, 4, 275, [300], 320, False, 1.0),
    # 3-bit key codes (byte-lane layout) on the shared-tile kernel: the 3.5-bit
    # cache (3-bit keys, 4-bit values), 160 rows; 4-bit Prod keys with group
    # values at head_dim 256, 80 rows
    ("bf16_mse3_mse4_q20", 128, (3, 0), (4, 0), 1, 2, 16, 20, [900], 960, True, 0.02),
    ("bf16_d256_prod4_group2_q40", 256, (4, 1), (2, 2), 1, 1, 2, 40, [700], 768, True, 0.02),
    # 3-bit values (byte-lane groups) on the shared-tile kernel: Prod keys, 160
    # rows; the 2.5-bit cache (2-bit keys, 3-bit values) over a ragged batch of
    # several chunks, 256 rows per KV head; 3-bit keys and values at head_dim
    # 256, 80 rows
    ("bf16_prod3_mse3_q20", 128, (3, 1), (3, 0), 1, 1, 8, 20, [700], 768, True, 0.02),
    ("bf16_mse2_mse3_256_rows_ragged", 128, (2, 0), (3, 0), 2, 2, 16, 16, [4100, 1900], 4100, True, 0.02),
    ("bf16_d256_mse3_mse3_q40", 256, (3, 0), (3, 0), 1, 1, 2, 40, [900], 960, False, 1.0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prefill_parity_on_oracle_state(case):
    name, d, kspec, vspec, B, Hkv, Hq, q_len, lens, cap, bf16, qstd = case
    print(f"prefill {name}", flush=True)
    sys.stdout.flush()
    N = max(lens)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    k = rng.standard_normal((B, Hkv, N, d)).astype(np.float32) * np.float32(0.02)
    v = rng.standard_normal((B, Hkv, N, d)).astype(np.float32) * np.float32(0.02)
    q = rng.standard_normal((B, Hq, q_len, d)).astype(np.float32) * np.float32(qstd)
    if bf16:
        k, v, q = round_bf16(k), round_bf16(v), round_bf16(q)
    kc = ocodec.make_codec(d, kspec[0], 0, kspec[1])
    vc = ocodec.make_codec(d, vspec[0], 1, vspec[1])
    ks, vs = oquant.quantize(k.astype(np.float64), kc), oquant.quantize(v.astype(np.float64), vc)
    gk = tq.tq_codec_create(d, kspec[0], 0, kspec[1])
    gv = tq.tq_codec_create(d, vspec[0], 1, vspec[1])
    kcache, vcache = tq.allocate_cache(gk, B, Hkv, cap), tq.allocate_cache(gv, B, Hkv, cap)
    upload_state(kcache, ks, kspec[1], N)
    upload_state(vcache, vs, vspec[1], N)
    out = torch.zeros((B, Hq, q_len, d), dtype=torch.float32, device="cuda")
    ws = tq.allocate_prefill_workspace(gk, gv, B, Hq, Hkv, q_len, N)
    ld = torch.tensor(lens, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(d)
    tq.tq_prefill_attention(gk, gv, to_device_f(q, bf16), kcache, vcache, ld, N, scale, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    want = oatt.decode_attention_rotated(q.astype(np.float64), ks, kc, vs, vc, np.array(lens), scale)
    seen = np.array([[lens[b] - q_len + i + 1 > 0 for i in range(q_len)] for b in range(B)])
    err = rel_l2_rows(got[seen[:, None, :].repeat(Hq, 1)][None, None],
                      want[seen[:, None, :].repeat(Hq, 1)][None, None])
    print(f"  max row rel L2 {err.max():.3e} over {int(seen.sum()) * Hq} rows", flush=True)
    assert err.max() <= 1e-4
    assert np.all(got[~seen[:, None, :].repeat(Hq, 1)] == 0), "rows that see no token must be zero"


def test_prefill_matches_decode_for_a_decode_step():
    """With q_len 2 and 8 query heads per KV head (16 rows) prefill is one
    block: it writes exactly what tq_decode_attention writes."""
    d, B, Hkv, Hq, q_len, N = 128, 1, 2, 16, 2, 2000
    rng = np.random.default_rng(3)
    k = round_bf16(rng.standard_normal((B, Hkv, N, d)).astype(np.float32) * np.float32(0.02))
    v = round_bf16(rng.standard_normal((B, Hkv, N, d)).astype(np.float32) * np.float32(0.02))
    q = round_bf16(rng.standard_normal((B, Hq, q_len, d)).astype(np.float32) * np.float32(0.02))
    gk, gv = tq.tq_codec_create(d, 3, 0, 0), tq.tq_codec_create(d, 3, 1, 0)
    K, V = tq.allocate_cache(gk, B, Hkv, N), tq.allocate_cache(gv, B, Hkv, N)
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")
    tq.tq_quantize_append_kv(gk, gv, to_device_f(k, True), to_device_f(v, True), K, V, pos, N)
    ld = torch.tensor([N], dtype=torch.int32, device="cuda")
    qd = to_device_f(q, True)
    o1 = torch.zeros((B, Hq, q_len, d), dtype=torch.float32, device="cuda")
    o2 = torch.zeros_like(o1)
    tq.tq_decode_attention(gk, gv, qd, K, V, ld, N, 1 / math.sqrt(d), o1, tq.allocate_workspace(gk, gv, B, Hq, Hkv, q_len, N))
    tq.tq_prefill_attention(gk, gv, qd, K, V, ld, N, 1 / math.sqrt(d), o2,
                            tq.allocate_prefill_workspace(gk, gv, B, Hq, Hkv, q_len, N))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
