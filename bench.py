#!/usr/bin/env python3
"""Compressed-KV decode attention throughput on one MI355X.

A step is one pass of the whole hot path over every layer of the workload:
for each layer, quantise-on-append of the q_len new K and V tokens per
sequence in one launch (the MTP-verify tokens of the 256k workload), then decode attention
of the layer's queries over the compressed cache.  Inputs and compressed
caches are resident in HBM before timing starts.  The timed steps replay the
whole step as one HIP graph (--no-graph: eager launches); the decode-call
time behind roofline.achieved comes from HIP events around every call of an
eager pass over the same layers.

Default workload: 64 layers x 8 KV / 64 query heads, head_dim 128, 262144
cached tokens, q_len 2, K and V 3-bit MSE, bf16 inputs with per-channel
outliers (13.96 GB of compressed state read per step).

Prints one JSON line (see the repository's design notes for every field).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="l64_d128_n256k_mse3_mtp2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager steps instead of a HIP graph of the step")
    ap.add_argument("--cpu-sample-tokens", type=int, default=16384,
                    help="cached tokens of the oracle's baseline layer (0: the workload's whole layer, which takes "
                         "minutes of untimed oracle quantisation first)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--layers", type=int, default=0, help="override the number of layer buffers")
    ap.add_argument("--all-layers-call", action="store_true",
                    help="also time one tq_decode_attention over every layer at once (a labelled upper bound, kept "
                         "out of the default run so that its dispatches do not mix with the per-layer calls in "
                         "kernel traces)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB mebibytes three times (the reference "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


def copy_calibration(mib: int) -> None:
    """A plain float32 device-to-device copy of known size: its FETCH_SIZE and
    WRITE_SIZE readings per dispatch give the factor by which those counters
    over- or under-count HBM bytes."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "read_bytes_per_copy": n * 4, "write_bytes_per_copy": n * 4,
                      "copies": 3}), flush=True)


def cpu_baseline(w, sample_tokens: int, seconds: float) -> dict:
    """The oracle doing what one GPU step does for one layer, on the same
    workload shape: layer 0, every KV head, ``sample_tokens`` cached tokens (the
    whole 262,144-token layer of the 256k workload by default; quantised once,
    untimed).  Each timed step quantises the q_len new K and V tokens of every
    head and runs the oracle's decode over the compressed cache (dequantise all
    tokens, float64 softmax attention).  Steps repeat until ``seconds`` have
    passed.  Rate = attended token positions / time (a step of the workload
    touches ``layers`` such layers, so the per-step rate is the same)."""
    from oracle import attention as oatt
    from oracle import codec as ocodec
    from oracle import quant as oquant
    from quantized_decode_attention_04_amd import workloads as wl

    cores = len(os.sched_getaffinity(0))
    n = min(sample_tokens, w.n) if sample_tokens > 0 else w.n
    g = w.hq // w.hkv
    kc = ocodec.make_codec(w.d, w.kbits, 0, w.kmode)
    vc = ocodec.make_codec(w.d, w.vbits, 1, w.vmode)
    hist = n - w.q_len
    ks, vs, knew, vnew = [], [], [], []
    for hh in range(w.hkv):   # one head at a time: the float64 copies of a whole layer would not fit
        sub = wl.Workload(w.name, 1, 1, g, w.d, n, w.q_len, w.kbits, w.kmode, w.vbits, w.vmode, w.bf16,
                          outliers=w.outliers)
        k, v = wl.kv_tensors(sub, 100 + hh)                  # [1, 1, n, d]
        ks.append(oquant.quantize(k[:, :, :hist].astype(np.float64), kc))
        vs.append(oquant.quantize(v[:, :, :hist].astype(np.float64), vc))
        for st in (ks[-1], vs[-1]):
            for key in ("u", "y", "margin", "z", "zmargin", "t"):
                st.pop(key, None)
        knew.append(k[:, :, hist:].astype(np.float64))
        vnew.append(v[:, :, hist:].astype(np.float64))
    q = wl.normal(0, 0, wl.STREAM_Q, (1, w.hq, w.q_len, w.d), w.bf16).astype(np.float64)
    scale = 1.0 / math.sqrt(w.d)
    lens = np.array([n])
    steps = 0
    t0 = time.perf_counter()
    while True:
        for hh in range(w.hkv):
            kn = oquant.quantize(knew[hh], kc)
            vn = oquant.quantize(vnew[hh], vc)
            kd = np.concatenate([oatt.dequantize_cache(ks[hh], kc), oatt.dequantize_cache(kn, kc)], axis=2)
            vd = np.concatenate([oatt.dequantize_cache(vs[hh], vc), oatt.dequantize_cache(vn, vc)], axis=2)
            oatt.decode_attention(q[:, hh * g:(hh + 1) * g], kd, vd, lens, scale)
            del kd, vd
        steps += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            break
    return {
        "value": n * steps / dt,
        "unit": "KV tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"one layer of {w.name}: all {w.hkv} KV heads x {n} cached tokens" +
                  ("" if n == w.n else f" (of the layer's {w.n}; the oracle's work per cached token does not "
                                       f"depend on the length, so the rate carries over)") +
                  f"; {steps} step(s) of quantise {w.q_len} new K/V tokens per head + oracle decode (dequantise, "
                  f"float64 attention) in {dt:.1f} s; rate = attended token positions / time",
        "extrapolated_step_s": w.n * max(1, w.layers) / (n * steps / dt),
        "extrapolation": f"seconds for one whole step ({max(1, w.layers)} layer(s) x {w.n} tokens) at this rate",
    }


def quality_report(tq, w, kc, vc, sample, out_rows, state, scale, decode_oracle_state) -> dict:
    """Quality and full-size parity of one sampled head of layer 0, outside any
    timed region (the only bench leg besides cpu_baseline that calls the
    oracle).  ``sample`` holds the head's unquantised attended K and V and its
    query rows (host float64), ``out_rows`` the GPU decode output of those
    rows, ``state`` the GPU's packed state of the head.
      * cos-sim of the GPU output to exact attention on the unquantised K, V
        ("turboquant validate_moe_phase2.py", Test 1's metric);
      * the oracle's quantisation of the same K, V: coordinates within 1e-6 of
        a decision threshold (the window), and GPU/oracle code differences
        outside it (must be 0) and inside it;
      * parity of the decode at full size: ``decode_oracle_state`` writes the
        oracle's state of the head over the GPU's and returns the GPU decode of
        the sampled rows, compared with the oracle's decode of that state."""
    from oracle import attention as oatt
    from oracle import codec as ocodec
    from oracle import packing
    from oracle import quant as oquant

    t0 = time.perf_counter()
    kh, vh, qh = sample["k"], sample["v"], sample["q"]
    n = kh.shape[2]
    okc = ocodec.make_codec(w.d, w.kbits, 0, w.kmode)
    ovc = ocodec.make_codec(w.d, w.vbits, 1, w.vmode)
    ref = oatt.reference_attention(qh, kh, vh, np.array([n]), scale)
    cos = np.sum(out_rows * ref, -1) / (np.linalg.norm(out_rows, axis=-1) * np.linalg.norm(ref, axis=-1))
    res = {"sample": f"layer 0, sequence {sample['b']}, KV head {sample['g']}: {n} tokens, "
                     f"{out_rows.shape[1] * out_rows.shape[2]} query rows",
           "cos_sim_mean": float(cos.mean()), "cos_sim_min": float(cos.min())}
    ora = {}
    for name, x, oc, key in (("keys", kh, okc, "k"), ("values", vh, ovc, "v")):
        st = oquant.quantize(x, oc)
        ora[key] = st
        gw = state[key]["idx"]
        win = 1e-6
        if oc.mode == ocodec.MODE_GROUP:
            codes, want = packing.unpack(gw, oc.bits, w.d), st["q"][0, 0]
            inwin = st["margin"][0, 0] < win * ((1 << oc.bits) - 1)
        else:
            codes, want = packing.unpack(gw, oc.mse_bits, w.d), st["idx"][0, 0]
            inwin = st["margin"][0, 0] < win
        diff = codes != want
        entry = {"coords": int(diff.size), "window": int(inwin.sum()),
                 "differ_outside_window": int((diff & ~inwin).sum()), "differ_inside_window": int((diff & inwin).sum())}
        if oc.mode != ocodec.MODE_GROUP:
            entry["norm_max_rel_diff"] = float(np.max(np.abs(state[key]["norm"] - st["norm"][0, 0]) /
                                                      np.maximum(st["norm"][0, 0], 1e-30)))
        res[name] = entry
    want = oatt.decode_attention_rotated(qh, ora["k"], okc, ora["v"], ovc, np.array([n]), scale)
    got = decode_oracle_state(ora["k"], ora["v"])
    err = np.linalg.norm(got - want, axis=-1) / np.linalg.norm(want, axis=-1)
    res["decode_on_oracle_state_rel_l2_max"] = float(err.max())
    res["decode_on_oracle_state_bar"] = 1e-4
    res["seconds"] = time.perf_counter() - t0
    return res


def traffic_from_profile(kernel_source: str) -> tuple:
    """HBM bytes per decode call from the committed counter summary, or None
    when the kernel source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        "traffic_decode_fast_l64_d128_n256k_mse3.txt")
    if not os.path.exists(path):
        return None, "no counter summary"
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    with open(kernel_source, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    if fields.get("kernel_source_sha256") != digest:
        return None, "kernel changed since the counters were taken"
    return float(fields["traffic_bytes_per_call"]), path


def bulk_prefill(tq, wl, w, kc, vc, dev, stream, warmup: int, reps: int, tokens: int = 8192) -> dict:
    """Bulk quantise-on-append of ``tokens`` new tokens for every KV head of one
    sequence (keys and values in one tq_quantize_append_kv call), timed with
    HIP events on the launch stream: microseconds per call, the bytes it moves
    (bf16/fp32 inputs read + packed state written) per second, and the
    rotation FLOPs (Pi for keys and MSE values, S as well for Prod keys) per
    second."""
    import torch
    K = tq.allocate_cache(kc, 1, w.hkv, tokens, dev)
    V = tq.allocate_cache(vc, 1, w.hkv, tokens, dev)
    kx = wl.device_normal((1, w.hkv, tokens, w.d), 0, 0, 900, w.bf16, dev)
    vx = wl.device_normal((1, w.hkv, tokens, w.d), 0, 0, 901, w.bf16, dev)
    pos = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(max(1, warmup)):
        tq.tq_quantize_append_kv(kc, vc, kx, vx, K, V, pos, tokens)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for e0, e1 in ev:
        e0.record(stream)
        tq.tq_quantize_append_kv(kc, vc, kx, vx, K, V, pos, tokens)
        e1.record(stream)
    torch.cuda.synchronize()
    us = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev])) * 1000.0
    vectors = w.hkv * tokens
    in_bytes = 2 * vectors * w.d * (2 if w.bf16 else 4)
    out_bytes = vectors * (kc.info["bytes_per_token"] + vc.info["bytes_per_token"])
    rot = 2 * w.d * w.d * vectors
    flops = rot * ((2 if w.kmode == 1 else 1) + (1 if w.vmode != 2 else 0))
    return {"tokens": tokens, "kv_heads": w.hkv, "us": us, "gbps": (in_bytes + out_bytes) / (us * 1e-6) / 1e9,
            "gflops": flops / (us * 1e-6) / 1e9, "bytes": in_bytes + out_bytes, "flop": flops}


def prefill_timing(tq, wl, w, kc, vc, K, V, lens, max_len, dev, stream, reps: int, q_len: int = 64) -> dict:
    """tq_prefill_attention of ``q_len`` new tokens per sequence over one
    layer's cache, timed with HIP events on the launch stream: microseconds per
    call, query tokens per second, and the layer's state bytes per second.  On
    every workload here the rows of each KV head run on a shared-tile kernel in
    groups of 128 (head_dim 128) or 64 (head_dim 256), each group walking the
    whole state: ``row_groups`` passes over it (served in part by the caches),
    and ``state_gbps`` counts the state once."""
    import torch
    q = wl.device_normal((w.batch, w.hq, q_len, w.d), 0, 0, 902, w.bf16, dev)
    out = torch.empty((w.batch, w.hq, q_len, w.d), dtype=torch.float32, device=dev)
    ws = tq.allocate_prefill_workspace(kc, vc, w.batch, w.hq, w.hkv, q_len, max_len, dev)
    scale = 1.0 / math.sqrt(w.d)
    tq.tq_prefill_attention(kc, vc, q, K, V, lens, max_len, scale, out, ws)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for e0, e1 in ev:
        e0.record(stream)
        tq.tq_prefill_attention(kc, vc, q, K, V, lens, max_len, scale, out, ws)
        e1.record(stream)
    torch.cuda.synchronize()
    us = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev])) * 1000.0
    rows = (w.hq // w.hkv) * q_len
    group = 128 if w.d <= 128 else 64
    state = int(w.lens().sum()) * w.hkv * (kc.info["bytes_per_token"] + vc.info["bytes_per_token"])
    return {"q_len": q_len, "rows_per_kv_head": rows, "row_groups": -(-rows // group), "us": us,
            "query_tokens_per_s": w.batch * q_len / (us * 1e-6),
            "state_gbps": state / (us * 1e-6) / 1e9}


def gather_timing(tq, w, kc, vc, K, V, dev, stream, reps: int) -> dict:
    """tq_cache_gather of one layer's K and V records into fresh caches (the
    first half of the sequences, or the only one), timed with HIP events on the
    launch stream; bytes = records read + written."""
    import torch
    lens = [int(x) for x in w.lens()]
    keep = list(range(max(1, w.batch // 2)))
    cap = max(lens[i] for i in keep)
    Kd, Vd = tq.allocate_cache(kc, len(keep), w.hkv, cap, dev), tq.allocate_cache(vc, len(keep), w.hkv, cap, dev)
    starts, counts = [0] * len(keep), [lens[i] for i in keep]

    def run():
        tq.tq_cache_gather(kc, K, kc, Kd, keep, starts, counts)
        tq.tq_cache_gather(vc, V, vc, Vd, keep, starts, counts)

    run()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for e0, e1 in ev:
        e0.record(stream)
        run()
        e1.record(stream)
    torch.cuda.synchronize()
    us = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev])) * 1000.0
    nbytes = 2 * sum(counts) * w.hkv * (kc.info["bytes_per_token"] + vc.info["bytes_per_token"])
    del Kd, Vd
    return {"sequences": len(keep), "tokens": sum(counts), "us": us, "bytes": nbytes,
            "gbps": nbytes / (us * 1e-6) / 1e9}


def hybrid_timing(tq, wl, w, kc, vc, K, V, lens_h, max_len, dev, stream, reps: int, buf: int = 128) -> dict:
    """Hybrid cache of the recent-token ring in front of one layer's
    compressed caches ("turboquant validate_moe_phase2.py", Test 5's
    buffer_size): each sequence is taken to hold N = len - 64 tokens, its first
    floor(N / buf) * buf in the layer's compressed records and the rest (64 at
    these lengths) in a ring of seeded values.  Timed with HIP events on the
    launch stream: tq_hybrid_append of the step's new tokens that only stage
    into the rings, one that fills each ring (its buf tokens quantised into
    copies of the compressed caches, one ring below each sequence's length, so
    the layer's own records stay as the rest of the bench reads them), and
    tq_hybrid_decode_attention over both parts; bytes of the decode =
    compressed records + ring tokens read."""
    import dataclasses
    import torch
    B, hkv, hq, d, qlen = w.batch, w.hkv, w.hq, w.d, w.q_len
    dt = torch.bfloat16 if w.bf16 else torch.float32
    n_h = np.maximum(lens_h - 64, 1).astype(np.int64)
    nc = (n_h // buf) * buf
    kb = tq.allocate_ring(B, hkv, buf, d, dtype=dt, device=dev)
    vb = tq.allocate_ring(B, hkv, buf, d, dtype=dt, device=dev)
    kb.copy_(wl.device_normal((B, hkv, buf, d), 0, 0, 903, w.bf16, dev))
    vb.copy_(wl.device_normal((B, hkv, buf, d), 0, 0, 904, w.bf16, dev))
    kn = wl.device_normal((B, hkv, qlen, d), 0, 0, 905, w.bf16, dev)
    vn = wl.device_normal((B, hkv, qlen, d), 0, 0, 906, w.bf16, dev)
    q = wl.device_normal((B, hq, qlen, d), 0, 0, 907, w.bf16, dev)
    out = torch.empty((B, hq, qlen, d), dtype=torch.float32, device=dev)
    ln = torch.tensor(n_h, dtype=torch.int32, device=dev)
    # lengths at which the step's tokens complete every ring (a ring below N)
    nf = np.maximum(n_h // buf - 1, 0) * buf + (buf - qlen)
    lf = torch.tensor(nf, dtype=torch.int32, device=dev)
    clone = lambda c: dataclasses.replace(c, **{f: getattr(c, f).clone() for f in
                                                ("idx", "norm", "rnorm", "sign", "scale", "gmin")
                                                if getattr(c, f) is not None})
    Kc, Vc = clone(K), clone(V)
    ws = torch.zeros(tq.tq_hybrid_decode_workspace_size(kc, vc, B, hq, hkv, qlen, max_len, buf), dtype=torch.uint8,
                     device=dev)
    scale = 1.0 / math.sqrt(d)

    def timed(fn):
        fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for e0, e1 in ev:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev])) * 1000.0

    stage_us = timed(lambda: tq.tq_hybrid_append(kc, vc, kn, vn, K, V, kb, vb, ln, int(n_h.max()) + qlen))
    flush_us = timed(lambda: tq.tq_hybrid_append(kc, vc, kn, vn, Kc, Vc, kb, vb, lf, int(nf.max()) + qlen))
    del Kc, Vc
    dec_us = timed(lambda: tq.tq_hybrid_decode_attention(kc, vc, q, K, V, kb, vb, ln, max_len, scale, out, ws))
    esz = 2 if w.bf16 else 4
    nbytes = (int(nc.sum()) * (kc.info["bytes_per_token"] + vc.info["bytes_per_token"])
              + int((n_h - nc).sum()) * 2 * d * esz) * hkv
    del kb, vb, ws, out
    return {"buf_size": buf, "compressed_tokens": int(nc.sum()), "ring_tokens": int((n_h - nc).sum()),
            "append_stage_us": stage_us, "append_fill_flush_us": flush_us, "decode_us": dec_us,
            "decode_bytes": nbytes, "decode_gbps": nbytes / (dec_us * 1e-6) / 1e9,
            "decode_frac": nbytes / (dec_us * 1e-6) / 1e9 / HBM_PEAK_GBPS}


def split_timing(tq, wl, w, dev, stream, reps: int) -> dict:
    """Fractional bit-widths and the split state at the workload's shape, over
    one layer filled with bulk appends: keys and values of a 3.5-bit and a
    2.5-bit cache (tq_codec_create_kv: 3-bit keys and 4-bit values, 2-bit keys
    and 3-bit values) and of 2.5-bit split codecs (tq_codec_create_split, keys
    and values alike).  Timed with HIP events on
    the launch stream: one decode call of the workload's query rows; bytes =
    the packed records of every attended token-head."""
    import torch
    B, hkv, hq, d, qlen = w.batch, w.hkv, w.hq, w.d, w.q_len
    lens_h = w.lens()
    max_len = int(lens_h.max())
    lens = torch.tensor(lens_h, dtype=torch.int32, device=dev)
    q = wl.device_normal((B, hq, qlen, d), 0, 0, 908, w.bf16, dev)
    out = torch.empty((B, hq, qlen, d), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(d)
    res = {}
    for label, (kc, vc) in (("fractional_3.5", tq.tq_codec_create_kv(d, 3.5, 0)),
                            ("fractional_2.5", tq.tq_codec_create_kv(d, 2.5, 0)),
                            ("split_2.5", (tq.tq_codec_create_split(d, 2.5, 0), tq.tq_codec_create_split(d, 2.5, 1)))):
        K, V = tq.allocate_cache(kc, B, hkv, max_len, dev), tq.allocate_cache(vc, B, hkv, max_len, dev)
        for s0 in range(0, max_len, 65536):
            n = min(65536, max_len - s0)
            pos = torch.full((B,), s0, dtype=torch.int32, device=dev)
            kx = wl.device_normal((B, hkv, n, d), 0, 0, 100 + s0 // 65536, w.bf16, dev)
            vx = wl.device_normal((B, hkv, n, d), 0, 0, 200000 + s0 // 65536, w.bf16, dev)
            tq.tq_quantize_append_kv(kc, vc, kx, vx, K, V, pos, s0 + n)
            del kx, vx
        ws = tq.allocate_workspace(kc, vc, B, hq, hkv, qlen, max_len, dev)
        tq.tq_decode_attention(kc, vc, q, K, V, lens, max_len, scale, out, ws)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for e0, e1 in ev:
            e0.record(stream)
            tq.tq_decode_attention(kc, vc, q, K, V, lens, max_len, scale, out, ws)
            e1.record(stream)
        torch.cuda.synchronize()
        us = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev])) * 1000.0
        nbytes = int(lens_h.sum()) * hkv * (kc.info["bytes_per_token"] + vc.info["bytes_per_token"])
        res[label] = {"k_bits": kc.info["bits"], "v_bits": vc.info["bits"],
                      "split_high_dims": [kc.info["split_high_dim"], vc.info["split_high_dim"]],
                      "bytes_per_token_head": kc.info["bytes_per_token"] + vc.info["bytes_per_token"],
                      "decode_us": us, "gbps": nbytes / (us * 1e-6) / 1e9,
                      "frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS}
        del K, V, ws
    return res


def layer_view(c, l: int):
    """Layer l of a cache allocated with the layers as its batch: the same
    arrays sliced to batch 1 (contiguous, so only the base pointers move)."""
    import dataclasses
    sl = lambda t: None if t is None else t[l:l + 1]
    return dataclasses.replace(c, batch=1, idx=sl(c.idx), norm=sl(c.norm), rnorm=sl(c.rnorm), sign=sl(c.sign),
                               scale=sl(c.scale), gmin=sl(c.gmin))


def stream_read_reference(tq, dev, stream, reps: int = 10, gib: int = 4) -> dict:
    """A streaming read of the same run: the library's own read-only kernel
    (tq_stream_read: 16-byte loads, eight in flight per thread) over ``gib``
    GiB, well past the last-level cache, timed with HIP events on the launch
    stream; the best of a few grid sizes."""
    import torch
    nbytes = gib * (1 << 30)
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    best = None
    for per_cu in (4, 8, 16):
        blocks = 256 * per_cu
        sink = torch.zeros(blocks * 256, dtype=torch.int32, device=dev)
        tq.tq_stream_read(buf, sink, blocks)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for a, b in ev:
            a.record(stream)
            tq.tq_stream_read(buf, sink, blocks)
            b.record(stream)
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
        r = {"kernel": f"tq_stream_read over {gib} GiB, {blocks} workgroups of 256 threads", "bytes": nbytes,
             "us": ms * 1000.0, "gbps": nbytes / (ms / 1000.0) / 1e9}
        if best is None or r["gbps"] > best["gbps"]:
            best = r
        del sink
    del buf
    return best


def decode_read_reference(tq, kc, vc, kcs, vcs, lens, max_len, dev, stream, reps: int) -> dict:
    """The decode call's own state reads alone: tq_decode_read_reference over
    the same layer caches in turn (the int8 decode kernel's grid, chunks, tile
    loads and prefetch depth, no arithmetic), timed with HIP events on the
    launch stream around each call."""
    import torch
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)
    for K, V in zip(kcs, vcs):
        tq.tq_decode_read_reference(kc, vc, K, V, lens, max_len, sink)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps) for _ in kcs]
    i = 0
    for _ in range(reps):
        for K, V in zip(kcs, vcs):
            ev[i][0].record(stream)
            tq.tq_decode_read_reference(kc, vc, K, V, lens, max_len, sink)
            ev[i][1].record(stream)
            i += 1
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1000.0
    nbytes = int(lens.sum().item()) * kcs[0].heads * (kc.info["bytes_per_token"] + vc.info["bytes_per_token"])
    return {"kernel": "tq_decode_read_reference: decode_fast_kernel's grid and tile loads with no arithmetic",
            "state_bytes": nbytes, "us": us, "gbps": nbytes / (us / 1e6) / 1e9}


def main():
    args = _args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path runs on a single GPU)",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import torch

    import quantized_decode_attention_04_amd as tq
    from quantized_decode_attention_04_amd import _binding
    from quantized_decode_attention_04_amd import workloads as wl

    w = wl.configs()[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kc = tq.tq_codec_create(w.d, w.kbits, 0, w.kmode)
    vc = tq.tq_codec_create(w.d, w.vbits, 1, w.vmode)
    tq.tq_codec_upload(kc)
    tq.tq_codec_upload(vc)
    lens_h = w.lens()
    append = w.q_len
    B, hkv, hq, d, qlen = w.batch, w.hkv, w.hq, w.d, w.q_len
    max_len = int(lens_h.max())
    state_bytes_tok = kc.info["bytes_per_token"] + vc.info["bytes_per_token"]
    layer_state_bytes = int(lens_h.sum()) * hkv * state_bytes_tok
    layers = w.layers if w.layers > 1 else max(1, min(64, math.ceil(1e9 / layer_state_bytes)))
    if args.layers:
        layers = args.layers

    # ---- set-up (not timed): per-layer compressed caches, queries, new tokens.
    # With one sequence per layer the layers' caches and queries are slices of
    # one allocation batched over the layers, so that one extra call can also
    # read every layer at once (the labelled upper bound below).
    stacked = B == 1 and layers > 1
    if stacked:
        K_all = tq.allocate_cache(kc, layers, hkv, max_len, dev)
        V_all = tq.allocate_cache(vc, layers, hkv, max_len, dev)
        q_all = torch.empty((layers, hq, qlen, d), dtype=torch.bfloat16 if w.bf16 else torch.float32, device=dev)
    kcs, vcs, qs, kn, vn = [], [], [], [], []
    pos0 = torch.zeros(B, dtype=torch.int32, device=dev)
    # the unquantised history of one head of layer 0, kept on the host for the
    # quality report (cpu_baseline leg only)
    b_s, g_s = 0, hkv // 2
    k_sample, v_sample = [], []
    for l in range(layers):
        if stacked:
            K, V = layer_view(K_all, l), layer_view(V_all, l)
        else:
            K = tq.allocate_cache(kc, B, hkv, max_len, dev)
            V = tq.allocate_cache(vc, B, hkv, max_len, dev)
        ksc = wl.outlier_scales(0, l, hkv, d, 0) if w.outliers else None
        vsc = wl.outlier_scales(0, l, hkv, d, 1) if w.outliers else None
        hist = max_len - append
        step_tok = 65536
        for s0 in range(0, hist, step_tok):
            n = min(step_tok, hist - s0)
            pos = torch.full((B,), s0, dtype=torch.int32, device=dev)
            kx = wl.device_normal((B, hkv, n, d), 0, l, 100 + s0 // step_tok, w.bf16, dev, ksc)
            vx = wl.device_normal((B, hkv, n, d), 0, l, 200000 + s0 // step_tok, w.bf16, dev, vsc)
            tq.tq_quantize_append(kc, kx, K, pos, s0 + n)
            tq.tq_quantize_append(vc, vx, V, pos, s0 + n)
            if l == 0 and not args.no_cpu_baseline:
                k_sample.append(kx[b_s, g_s].float().cpu().numpy())
                v_sample.append(vx[b_s, g_s].float().cpu().numpy())
            del kx, vx
        kcs.append(K)
        vcs.append(V)
        qs.append(wl.device_normal((B, hq, qlen, d), 0, l, wl.STREAM_Q, w.bf16, dev))
        if stacked:
            q_all[l:l + 1].copy_(qs[-1])
            qs[-1] = q_all[l:l + 1]
        kn.append(wl.device_normal((B, hkv, append, d), 0, l, wl.STREAM_KNEW, w.bf16, dev, ksc))
        vn.append(wl.device_normal((B, hkv, append, d), 0, l, wl.STREAM_VNEW, w.bf16, dev, vsc))
    torch.cuda.synchronize()
    # the new tokens go to len-append .. len-1 of each sequence; the history
    # beyond a ragged sequence's length is never attended
    pos_new = torch.tensor(lens_h - append, dtype=torch.int32, device=dev)
    lens = torch.tensor(lens_h, dtype=torch.int32, device=dev)
    ws_bytes = tq.tq_decode_workspace_size(kc, vc, B, hq, hkv, qlen, max_len)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((B, hq, qlen, d), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(d)

    # ---- pre-marshalled C calls (the same entry points the binding wraps)
    lib = _binding._lib
    dt_code = tq.TQ_BF16 if w.bf16 else tq.TQ_F32
    keep = []

    def make_calls(stream_handle):
        sp = ctypes.c_void_p(stream_handle)
        calls = []
        for l in range(layers):
            ks_, vs_ = kcs[l].as_struct(), vcs[l].as_struct()
            kstr = (ctypes.c_int64 * 4)(*kn[l].stride())
            vstr = (ctypes.c_int64 * 4)(*vn[l].stride())
            keep.append((ks_, vs_, kstr, vstr))
            calls.append(((kc.handle, vc.handle, ctypes.c_void_p(kn[l].data_ptr()), ctypes.c_void_p(vn[l].data_ptr()),
                           dt_code, B, hkv, append, kstr, vstr, ctypes.byref(ks_), ctypes.byref(vs_),
                           ctypes.c_void_p(pos_new.data_ptr()), max_len, sp),
                          (kc.handle, vc.handle, ctypes.c_void_p(qs[l].data_ptr()), dt_code, B, hq, hkv, qlen,
                           ctypes.byref(ks_), ctypes.byref(vs_), ctypes.c_void_p(lens.data_ptr()), max_len,
                           ctypes.c_float(scale), ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                           ws_bytes, sp)))
        return calls

    def check(st):
        if st != 0:
            raise RuntimeError(tq.tq_last_error())

    stream = torch.cuda.current_stream()
    calls = make_calls(stream.cuda_stream)

    def step(events=None, app_events=None):
        for i, c in enumerate(calls):
            if app_events is not None:
                app_events[i].record(stream)
            check(lib.tq_quantize_append_kv(*c[0]))
            if events is not None:
                events[i][0].record(stream)
            check(lib.tq_decode_attention(*c[1]))
            if events is not None:
                events[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # decode-call time: HIP events on the launch stream around every call of
    # an eager pass (the dominant kernels; roofline.achieved)
    events = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
              for _ in range(args.steps)]
    # the append call is bracketed by an event recorded before it and the
    # decode call's start event
    app_events = [[torch.cuda.Event(enable_timing=True) for _ in calls] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        step(events[s_], app_events[s_])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step_eager = (t1 - t0) * 1000.0 / args.steps
    dec_ms = [e0.elapsed_time(e1) for row in events for (e0, e1) in row]
    app_ms = [a.elapsed_time(ev[0]) for arow, erow in zip(app_events, events) for a, ev in zip(arow, erow)]
    dec_ms_avg = float(np.mean(dec_ms))

    # the step as one HIP graph (the per-layer kernels without launch gaps):
    # value and ms_per_step
    ms_per_step = ms_per_step_eager
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        with torch.cuda.graph(graph, stream=cap):
            for c in make_calls(torch.cuda.current_stream().cuda_stream):
                check(lib.tq_quantize_append_kv(*c[0]))
                check(lib.tq_decode_attention(*c[1]))
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms_per_step = (t1 - t0) * 1000.0 / args.steps

    prefill = bulk_prefill(tq, wl, w, kc, vc, dev, stream, args.warmup, max(args.steps, 5))
    gather = gather_timing(tq, w, kc, vc, kcs[0], vcs[0], dev, stream, max(3, args.steps // 2))
    prefill_attn = prefill_timing(tq, wl, w, kc, vc, kcs[0], vcs[0], lens, max_len, dev, stream,
                                  max(3, args.steps // 2))
    hybrid = hybrid_timing(tq, wl, w, kc, vc, kcs[0], vcs[0], lens_h, max_len, dev, stream, max(3, args.steps // 2))
    split = split_timing(tq, wl, w, dev, stream, max(3, args.steps // 2))

    single = "not run (bench.py --all-layers-call)" if stacked else None
    if stacked and args.all_layers_call:
        # upper bound, not the step: one call over every layer as a batch of
        # `layers` sequences; a real decode step cannot do this, since each
        # layer's query needs the previous layer's output
        lens_all = torch.full((layers,), int(lens_h[0]), dtype=torch.int32, device=dev)
        ws_all = torch.zeros(tq.tq_decode_workspace_size(kc, vc, layers, hq, hkv, qlen, max_len), dtype=torch.uint8,
                             device=dev)
        out_all = torch.empty((layers, hq, qlen, d), dtype=torch.float32, device=dev)
        tq.tq_decode_attention(kc, vc, q_all, K_all, V_all, lens_all, max_len, scale, out_all, ws_all)
        torch.cuda.synchronize()
        reps = max(3, args.steps // 2)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b_ in ev:
            a.record(stream)
            tq.tq_decode_attention(kc, vc, q_all, K_all, V_all, lens_all, max_len, scale, out_all, ws_all)
            b_.record(stream)
        torch.cuda.synchronize()
        sms = float(np.median([a.elapsed_time(b_) for a, b_ in ev]))
        sbytes = layer_state_bytes * layers
        single = {"label": f"upper bound, not a decode step: one tq_decode_attention over all {layers} layers as a "
                           f"batch of {layers} sequences",
                  "us": sms * 1000.0, "state_bytes": sbytes, "gbps": sbytes / (sms / 1000.0) / 1e9,
                  "frac": sbytes / (sms / 1000.0) / 1e9 / HBM_PEAK_GBPS}
        del ws_all, out_all
    stream_ref = stream_read_reference(tq, dev, stream)
    # the library takes the int8 matrix-core path for d 128 with 3-bit MSE keys
    # and values and at most 16 query rows per KV head (a label only)
    rows = (hq // hkv) * qlen
    fast = d == 128 and (w.kmode, w.kbits, w.vmode, w.vbits) == (0, 3, 0, 3) and rows <= 16
    read_ref = (decode_read_reference(tq, kc, vc, kcs, vcs, lens, max_len, dev, stream, max(3, args.steps))
                if fast else None)

    tokens_per_step = float(lens_h.sum()) * layers
    value = tokens_per_step / (ms_per_step / 1000.0)
    # algorithmic bytes of one decode call: the packed state of every attended
    # token-head, the queries, the output and the two rotations it reads
    q_bytes = B * hq * qlen * d * (2 if w.bf16 else 4)
    out_bytes = B * hq * qlen * d * 4
    table_bytes = 2 * d * d * 4 + (d * d * 4 if w.kmode == 1 else 0)
    alg_bytes = layer_state_bytes + q_bytes + out_bytes + table_bytes
    achieved = alg_bytes / (dec_ms_avg / 1000.0) / 1e9
    kcode_bits = w.kbits - 1 if w.kmode == 1 else w.kbits
    bf16_path = (not fast and d in (128, 256) and w.kmode in (0, 1) and kcode_bits in (1, 2)
                 and ((w.vmode == 0 and w.vbits in (1, 2, 4)) or (w.vmode == 2 and w.vbits == 2))
                 and rows <= (16 if d == 128 else 8))
    kernels = ("decode_fast_kernel + merge_fast_kernel" if fast
               else "qprep_kernel + decode_bf16_kernel + merge_kernel" if bf16_path
               else "qprep_kernel + decode_kernel + merge_kernel")
    dtype = "i8+f32" if fast else "bf16x2+f32" if bf16_path else "f32"
    traffic, traffic_src = None, "counters taken on l64_d128_n256k_mse3_mtp2 only"
    if w.name == "l64_d128_n256k_mse3_mtp2":
        src = os.path.join(os.path.dirname(os.path.abspath(tq.__file__)), "csrc", "decode_fast.hip")
        traffic, traffic_src = traffic_from_profile(src)

    res = {
        "metric": "compressed-KV decode attn: KV tokens/s + HBM GB/s (% peak) at 256k ctx",
        "value": value,
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic: seeded N(0,1)*0.02 bf16 K/V/q" + (" with per-channel outliers" if w.outliers else ""),
        "config": {
            "workload": w.name,
            "layers": layers,
            "batch": B,
            "kv_heads": hkv,
            "q_heads": hq,
            "head_dim": d,
            "cached_tokens": int(lens_h.sum()),
            "q_len": qlen,
            "k_codec": f"{w.kbits}-bit {'Prod' if w.kmode == 1 else 'MSE'}",
            "v_codec": f"{w.vbits}-bit {'group32' if w.vmode == 2 else 'MSE'}",
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
        },
        "detail": {
            "decode_call": f"tq_decode_attention = {kernels}, timed with HIP events on the launch stream "
                           "around each call",
            "traffic_source": traffic_src,
            "decode_call_us": dec_ms_avg * 1000.0,
            "decode_call_us_p10_p50_p90": [float(np.percentile(dec_ms, q)) * 1000.0 for q in (10, 50, 90)],
            "append_call": f"tq_quantize_append_kv of the {append} new K and V tokens of every sequence and KV head "
                           "of a layer, timed with HIP events on the launch stream",
            "append_call_us": float(np.mean(app_ms)) * 1000.0,
            "step": f"one HIP graph of the {layers} per-layer (append K+V, decode) calls" if not args.no_graph
                    else "eager launches",
            "ms_per_step_eager": ms_per_step_eager,
            "decode_alg_bytes_per_call": alg_bytes,
            "state_bytes_per_step": layer_state_bytes * layers,
            "step_gbps_state": layer_state_bytes * layers / (ms_per_step / 1000.0) / 1e9,
            "ws_bytes": ws_bytes,
            "bulk_prefill": prefill,
            "prefill_attention": prefill_attn,
            "cache_gather": gather,
            "hybrid_decode": hybrid,
            "split_decode": split,
            "stream_read_reference": stream_ref,
            "achieved_vs_stream_read": achieved / stream_ref["gbps"],
            "decode_read_reference": read_ref,
            "decode_call_vs_its_reads": (read_ref["us"] / (dec_ms_avg * 1000.0)) if read_ref else None,
            "single_launch_all_layers": single,
        },
    }
    if not args.no_cpu_baseline:
        # quality and full-size parity of the sampled head, from a decode of
        # layer 0 after the timed steps (its new tokens are appended)
        n_b = int(lens_h[b_s])
        G = hq // hkv
        out_q = torch.zeros((B, hq, qlen, d), dtype=torch.float32, device=dev)
        tq.tq_decode_attention(kc, vc, qs[0], kcs[0], vcs[0], lens, max_len, scale, out_q, ws)
        torch.cuda.synchronize()
        cat = lambda parts, new: np.concatenate([np.concatenate(parts)[:n_b - append],
                                                 new[b_s, g_s].float().cpu().numpy()])[None, None].astype(np.float64)
        sample = {"b": b_s, "g": g_s, "k": cat(k_sample, kn[0]), "v": cat(v_sample, vn[0]),
                  "q": qs[0][b_s, g_s * G:(g_s + 1) * G].float().cpu().numpy().astype(np.float64)[None]}
        rows = out_q[b_s, g_s * G:(g_s + 1) * G].cpu().numpy().astype(np.float64)[None]

        def head_state(c):
            st = {"idx": c.idx[b_s, g_s, :n_b].cpu().numpy().view(np.uint32)}
            if c.norm is not None:
                st["norm"] = c.norm[b_s, g_s, :n_b].cpu().numpy().astype(np.float64)
            return st

        def put(c, st, mode):
            t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(np.asarray(a)[0, 0]).astype(dt)).to(dev)
            c.idx[b_s, g_s, :n_b] = t(np.asarray(st["words"], dtype=np.uint32).view(np.int32), np.int32)
            if mode in (0, 1):
                c.norm[b_s, g_s, :n_b] = t(st["norm"], np.float32)
            if mode == 1:
                c.rnorm[b_s, g_s, :n_b] = t(st["rnorm"], np.float32)
                c.sign[b_s, g_s, :n_b] = t(np.asarray(st["sign_words"], dtype=np.uint32).view(np.int32), np.int32)
            if mode == 2:
                c.scale[b_s, g_s, :n_b] = t(st["scale"], np.float32)
                c.gmin[b_s, g_s, :n_b] = t(st["min"], np.float32)

        def decode_oracle_state(ks_, vs_):
            put(kcs[0], ks_, w.kmode)
            put(vcs[0], vs_, w.vmode)
            tq.tq_decode_attention(kc, vc, qs[0], kcs[0], vcs[0], lens, max_len, scale, out_q, ws)
            torch.cuda.synchronize()
            return out_q[b_s, g_s * G:(g_s + 1) * G].cpu().numpy().astype(np.float64)[None]

        res["quality"] = quality_report(tq, w, kc, vc, sample, rows, {"k": head_state(kcs[0]), "v": head_state(vcs[0])},
                                        scale, decode_oracle_state)
        del k_sample, v_sample, sample, out_q
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_tokens, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
