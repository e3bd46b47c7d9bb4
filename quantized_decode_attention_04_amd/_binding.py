"""ctypes marshalling for libtq.so (see include/tq.h for the semantics).

Tensors are torch tensors on a HIP device; the binding checks dtype, device,
shape and contiguity so that the raw pointers it passes are valid, then calls
the C function on the current torch stream.  Nothing here computes.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libtq.so")

TQ_OK = 0
TQ_MODE_MSE, TQ_MODE_PROD, TQ_MODE_GROUP, TQ_MODE_SPLIT = 0, 1, 2, 3
TQ_F32, TQ_BF16 = 0, 1


class TQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{tq_status_string(status)}: {message}")
        self.status = status


class _CodecInfo(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int32), ("bits", ctypes.c_int32), ("mode", ctypes.c_int32),
        ("mse_bits", ctypes.c_int32), ("levels", ctypes.c_int32), ("idx_words", ctypes.c_int32),
        ("sign_words", ctypes.c_int32), ("groups", ctypes.c_int32), ("grid_exp", ctypes.c_int32),
        ("split_high_dim", ctypes.c_int32), ("seed", ctypes.c_uint64), ("bytes_per_token", ctypes.c_uint64),
    ]


class _Cache(ctypes.Structure):
    _fields_ = [
        ("idx", ctypes.c_void_p), ("norm", ctypes.c_void_p), ("rnorm", ctypes.c_void_p),
        ("sign", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("gmin", ctypes.c_void_p),
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("cap", ctypes.c_int64),
    ]


def _load() -> ctypes.CDLL:
    # torch ships its own HIP runtime with the same soname as /opt/rocm's; it
    # must be loaded first so that libtq.so binds to that one runtime instead
    # of pulling a second copy into the process
    import torch  # noqa: F401
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built: run `python quantized_decode_attention_04_amd/build_lib.py`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, U64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t
    sigs = {
        "tq_codec_create": (I32, [I32, I32, U64, I32, ctypes.POINTER(P)]),
        "tq_codec_destroy": (None, [P]),
        "tq_codec_create_kv": (I32, [I32, ctypes.c_double, U64, ctypes.POINTER(P), ctypes.POINTER(P)]),
        "tq_codec_create_split": (I32, [I32, ctypes.c_double, U64, ctypes.POINTER(P)]),
        "tq_codec_part": (I32, [P, I32, ctypes.POINTER(P)]),
        "tq_codec_get_info": (I32, [P, ctypes.POINTER(_CodecInfo)]),
        "tq_codec_export": (I32, [P, P, P, P, P]),
        "tq_codec_upload": (I32, [P]),
        "tq_quantize_append": (I32, [P, P, I32, I32, I32, I32, ctypes.POINTER(I64), ctypes.POINTER(_Cache), P, I64,
                                     P]),
        "tq_quantize_append_kv": (I32, [P, P, P, P, I32, I32, I32, I32, ctypes.POINTER(I64), ctypes.POINTER(I64),
                                        ctypes.POINTER(_Cache), ctypes.POINTER(_Cache), P, I64, P]),
        "tq_decode_workspace_size": (I32, [P, P, I32, I32, I32, I32, I64, ctypes.POINTER(SZ)]),
        "tq_decode_attention": (I32, [P, P, P, I32, I32, I32, I32, I32, ctypes.POINTER(_Cache),
                                      ctypes.POINTER(_Cache), P, I64, ctypes.c_float, P, P, SZ, P]),
        "tq_prefill_workspace_size": (I32, [P, P, I32, I32, I32, I32, I64, ctypes.POINTER(SZ)]),
        "tq_cache_gather": (I32, [P, ctypes.POINTER(_Cache), P, ctypes.POINTER(_Cache), ctypes.POINTER(I32),
                                  ctypes.POINTER(I32), ctypes.POINTER(I32), P]),
        "tq_prefill_attention": (I32, [P, P, P, I32, I32, I32, I32, I32, ctypes.POINTER(_Cache),
                                       ctypes.POINTER(_Cache), P, I64, ctypes.c_float, P, P, SZ, P]),
        "tq_stream_read": (I32, [P, U64, P, I32, P]),
        "tq_decode_read_reference": (I32, [P, P, I32, I32, ctypes.POINTER(_Cache), ctypes.POINTER(_Cache), P, I64,
                                           P, ctypes.c_uint32, P]),
        "tq_hybrid_append": (I32, [P, P, P, P, I32, I32, I32, I32, ctypes.POINTER(I64), ctypes.POINTER(I64),
                                   ctypes.POINTER(_Cache), ctypes.POINTER(_Cache), P, P, I32, P, I64, P]),
        "tq_hybrid_decode_workspace_size": (I32, [P, P, I32, I32, I32, I32, I64, I32, ctypes.POINTER(SZ)]),
        "tq_hybrid_decode_attention": (I32, [P, P, P, I32, I32, I32, I32, I32, ctypes.POINTER(_Cache),
                                             ctypes.POINTER(_Cache), P, P, I32, I32, P, I64, ctypes.c_float, P, P,
                                             SZ, P]),
        "tq_decode_attention_noalloc": (I32, [P, P, P, I32, I32, I32, I32, I32, ctypes.POINTER(_Cache),
                                              ctypes.POINTER(_Cache), P, I64, ctypes.c_float, P, P]),
        "tq_last_error": (ctypes.c_char_p, []),
        "tq_status_string": (ctypes.c_char_p, [I32]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()

EXPORTED = (
    "tq_codec_create", "tq_codec_destroy", "tq_codec_get_info", "tq_codec_export", "tq_codec_upload",
    "tq_quantize_append", "tq_quantize_append_kv", "tq_decode_workspace_size", "tq_decode_attention",
    "tq_prefill_workspace_size", "tq_prefill_attention", "tq_cache_gather", "tq_stream_read", "tq_last_error",
    "tq_status_string", "tq_decode_attention_noalloc", "tq_codec_create_kv", "tq_codec_create_split", "tq_codec_part",
    "tq_hybrid_append", "tq_hybrid_decode_workspace_size", "tq_hybrid_decode_attention", "tq_decode_read_reference",
)


def lib_path() -> str:
    return _LIB_PATH


def tq_status_string(status: int) -> str:
    return _lib.tq_status_string(int(status)).decode()


def tq_last_error() -> str:
    return _lib.tq_last_error().decode()


def _check(status: int) -> None:
    if status != TQ_OK:
        raise TQError(status, tq_last_error())


class Codec:
    """Owner of a ``tq_codec*`` handle (destroyed with the object), or a
    borrowed part of a split codec (``owner`` keeps the split codec alive and
    the part is never destroyed on its own)."""

    def __init__(self, handle: int, owner: "Optional[Codec]" = None):
        self._h = ctypes.c_void_p(handle)
        self._owner = owner
        self.info = tq_codec_get_info(self)

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._h is None:
            raise ValueError("codec was destroyed")
        return self._h

    def __del__(self):
        if getattr(self, "_h", None) is not None and getattr(self, "_owner", None) is None:
            _lib.tq_codec_destroy(self._h)
            self._h = None


def tq_codec_create(head_dim: int, bits: int, seed: int, mode: int) -> Codec:
    out = ctypes.c_void_p()
    _check(_lib.tq_codec_create(int(head_dim), int(bits), ctypes.c_uint64(int(seed) & (2**64 - 1)), int(mode),
                                ctypes.byref(out)))
    return Codec(out.value)


def tq_codec_create_kv(head_dim: int, bits: float, seed: int):
    """(key codec, value codec) of a cache of width ``bits`` (floor / ceil
    for a fractional width; see include/tq.h)."""
    k, v = ctypes.c_void_p(), ctypes.c_void_p()
    _check(_lib.tq_codec_create_kv(int(head_dim), float(bits), ctypes.c_uint64(int(seed) & (2**64 - 1)),
                                   ctypes.byref(k), ctypes.byref(v)))
    return Codec(k.value), Codec(v.value)


def tq_codec_create_split(head_dim: int, bits: float, seed: int) -> Codec:
    out = ctypes.c_void_p()
    _check(_lib.tq_codec_create_split(int(head_dim), float(bits), ctypes.c_uint64(int(seed) & (2**64 - 1)),
                                      ctypes.byref(out)))
    return Codec(out.value)


def tq_codec_part(codec: Codec, which: int) -> Codec:
    """The low (0) or high (1) MSE part of a split codec (borrowed)."""
    out = ctypes.c_void_p()
    _check(_lib.tq_codec_part(codec.handle, int(which), ctypes.byref(out)))
    return Codec(out.value, owner=codec)


def tq_codec_destroy(codec: Codec) -> None:
    if getattr(codec, "_owner", None) is not None:
        raise ValueError("a part of a split codec is owned by the split codec")
    if codec._h is not None:
        _lib.tq_codec_destroy(codec._h)
        codec._h = None


def tq_codec_get_info(codec: Codec) -> dict:
    info = _CodecInfo()
    _check(_lib.tq_codec_get_info(codec.handle, ctypes.byref(info)))
    return {name: getattr(info, name) for name, _ in _CodecInfo._fields_}


def tq_codec_export(codec: Codec) -> dict:
    """Host copies of the float32 tables (empty dict for group codecs)."""
    info = codec.info
    if info["mode"] == TQ_MODE_GROUP:
        return {}
    d, L = info["head_dim"], info["levels"]
    rot = np.zeros((d, d), dtype=np.float32)
    cent = np.zeros(L, dtype=np.float32)
    bnd = np.zeros(L - 1, dtype=np.float32)
    sk = np.zeros((d, d), dtype=np.float32) if info["mode"] == TQ_MODE_PROD else None
    ptr = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)
    _check(_lib.tq_codec_export(codec.handle, ptr(rot), ptr(cent), ptr(bnd), ptr(sk)))
    out = {"rot": rot, "centroids": cent, "boundaries": bnd}
    if sk is not None:
        out["sketch"] = sk
    return out


def tq_codec_upload(codec: Codec) -> None:
    _check(_lib.tq_codec_upload(codec.handle))


# ---- caches -----------------------------------------------------------------

@dataclass
class Cache:
    """Device arrays of one compressed cache (K or V), [batch][heads][cap][...]."""
    codec_info: dict
    batch: int
    heads: int
    cap: int
    idx: "object"
    norm: Optional["object"] = None
    rnorm: Optional["object"] = None
    sign: Optional["object"] = None
    scale: Optional["object"] = None
    gmin: Optional["object"] = None

    def as_struct(self) -> _Cache:
        p = lambda t: None if t is None else t.data_ptr()
        return _Cache(p(self.idx), p(self.norm), p(self.rnorm), p(self.sign), p(self.scale), p(self.gmin),
                      self.batch, self.heads, self.cap)

    def arrays(self) -> dict:
        return {k: getattr(self, k) for k in ("idx", "norm", "rnorm", "sign", "scale", "gmin")
                if getattr(self, k) is not None}


def allocate_cache(codec: Codec, batch: int, heads: int, cap: int, device="cuda") -> Cache:
    """Zero-filled torch tensors shaped for ``codec``'s state (uint32 words are
    held in int32 tensors)."""
    import torch
    info = codec.info
    shp = (batch, heads, cap)
    z = lambda *tail, dt=torch.float32: torch.zeros(shp + tail, dtype=dt, device=device)
    c = Cache(info, batch, heads, cap, idx=z(info["idx_words"], dt=torch.int32))
    if info["mode"] in (TQ_MODE_MSE, TQ_MODE_PROD):
        c.norm = z()
    if info["mode"] == TQ_MODE_PROD:
        c.rnorm = z()
        c.sign = z(info["sign_words"], dt=torch.int32)
    if info["mode"] == TQ_MODE_SPLIT:
        c.norm = z()          # the low part's norm
        c.rnorm = z()         # the high part's norm
    if info["mode"] == TQ_MODE_GROUP:
        c.scale = z(info["groups"])
        c.gmin = z(info["groups"])
    return c


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(getattr(stream, "cuda_stream", stream)))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return TQ_F32
    if t.dtype == torch.bfloat16:
        return TQ_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _on_device(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensor must be on a HIP device")


def tq_quantize_append(codec: Codec, x, cache: Cache, pos, pos_end: int, stream=None) -> None:
    """Quantise x [batch, heads, n_new, head_dim] into ``cache`` at positions
    pos[b] + t (pos: int32 device tensor [batch]); ``pos_end`` is the caller's
    host bound on pos[b] + n_new (TQError CAPACITY above cache.cap)."""
    import torch
    _on_device(x, pos, *cache.arrays().values())
    if x.dim() != 4 or x.shape[3] != codec.info["head_dim"] or x.stride(3) != 1:
        raise ValueError("x must be [batch, heads, n_new, head_dim] with unit coordinate stride")
    if pos.dtype != torch.int32 or pos.numel() != x.shape[0] or not pos.is_contiguous():
        raise ValueError("pos must be a contiguous int32 tensor of length batch")
    strides = (ctypes.c_int64 * 4)(*x.stride())
    st = cache.as_struct()
    _check(_lib.tq_quantize_append(codec.handle, ctypes.c_void_p(x.data_ptr()), _dtype_code(x), int(x.shape[0]),
                                   int(x.shape[1]), int(x.shape[2]), strides, ctypes.byref(st),
                                   ctypes.c_void_p(pos.data_ptr()), int(pos_end), _stream(stream)))


def tq_quantize_append_kv(kc: Codec, vc: Codec, k, v, kcache: Cache, vcache: Cache, pos, pos_end: int,
                          stream=None) -> None:
    """Quantise the new keys k and values v [batch, heads, n_new, head_dim]
    (same dtype and sizes) into their caches at positions pos[b] + t, in one
    launch; ``pos_end`` bounds pos[b] + n_new as in tq_quantize_append."""
    import torch
    _on_device(k, v, pos, *kcache.arrays().values(), *vcache.arrays().values())
    for x in (k, v):
        if x.dim() != 4 or x.stride(3) != 1:
            raise ValueError("k and v must be [batch, heads, n_new, head_dim] with unit coordinate stride")
    if tuple(k.shape) != tuple(v.shape) or k.dtype != v.dtype:
        raise ValueError("k and v must have the same shape and dtype")
    if k.shape[3] != kc.info["head_dim"]:
        raise ValueError("head_dim of k does not match the key codec")
    if pos.dtype != torch.int32 or pos.numel() != k.shape[0] or not pos.is_contiguous():
        raise ValueError("pos must be a contiguous int32 tensor of length batch")
    ks_, vs_ = (ctypes.c_int64 * 4)(*k.stride()), (ctypes.c_int64 * 4)(*v.stride())
    kst, vst = kcache.as_struct(), vcache.as_struct()
    _check(_lib.tq_quantize_append_kv(kc.handle, vc.handle, ctypes.c_void_p(k.data_ptr()),
                                      ctypes.c_void_p(v.data_ptr()), _dtype_code(k), int(k.shape[0]),
                                      int(k.shape[1]), int(k.shape[2]), ks_, vs_, ctypes.byref(kst),
                                      ctypes.byref(vst), ctypes.c_void_p(pos.data_ptr()), int(pos_end),
                                      _stream(stream)))


def tq_decode_workspace_size(kc: Codec, vc: Codec, batch: int, n_q_heads: int, n_kv_heads: int, q_len: int,
                             max_len: int) -> int:
    n = ctypes.c_size_t()
    _check(_lib.tq_decode_workspace_size(kc.handle, vc.handle, int(batch), int(n_q_heads), int(n_kv_heads),
                                         int(q_len), int(max_len), ctypes.byref(n)))
    return n.value


def allocate_workspace(kc: Codec, vc: Codec, batch: int, n_q_heads: int, n_kv_heads: int, q_len: int,
                       max_len: int, device="cuda"):
    """A device workspace for tq_decode_attention with these sizes."""
    import torch
    return torch.zeros(tq_decode_workspace_size(kc, vc, batch, n_q_heads, n_kv_heads, q_len, max_len),
                       dtype=torch.uint8, device=device)


def _attention(fn, kc: Codec, vc: Codec, q, kcache: Cache, vcache: Cache, lens, max_len: int, scale: float, out, ws,
               stream) -> None:
    import torch
    _on_device(q, lens, out, ws, *kcache.arrays().values(), *vcache.arrays().values())
    if q.dim() != 4 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [batch, n_q_heads, q_len, head_dim] tensor")
    if out.dtype != torch.float32 or not out.is_contiguous() or tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must be a contiguous float32 tensor shaped like q")
    if lens.dtype != torch.int32 or lens.numel() != q.shape[0] or not lens.is_contiguous():
        raise ValueError("lens must be a contiguous int32 tensor of length batch")
    ks, vs = kcache.as_struct(), vcache.as_struct()
    nbytes = ws.numel() * ws.element_size()
    _check(fn(kc.handle, vc.handle, ctypes.c_void_p(q.data_ptr()), _dtype_code(q), int(q.shape[0]), int(q.shape[1]),
              int(kcache.heads), int(q.shape[2]), ctypes.byref(ks), ctypes.byref(vs), ctypes.c_void_p(lens.data_ptr()),
              int(max_len), ctypes.c_float(scale), ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
              nbytes, _stream(stream)))


def tq_decode_attention(kc: Codec, vc: Codec, q, kcache: Cache, vcache: Cache, lens, max_len: int, scale: float,
                        out, ws, stream=None) -> None:
    """out[b, h, i, :] = attention of q[b, h, i] over the compressed cache.
    q: [batch, n_q_heads, q_len, head_dim] contiguous f32/bf16; lens: int32
    device [batch]; out: float32 contiguous like q; ws: device byte tensor of at
    least tq_decode_workspace_size(...) bytes (allocate_workspace)."""
    _attention(_lib.tq_decode_attention, kc, vc, q, kcache, vcache, lens, max_len, scale, out, ws, stream)


def tq_decode_attention_noalloc(kc: Codec, vc: Codec, q, kcache: Cache, vcache: Cache, lens, max_len: int,
                                scale: float, out, stream=None) -> None:
    """tq_decode_attention with the library's own device scratch instead of a
    workspace (allocates nothing; the codecs' tables must be on the device
    already, tq_codec_upload)."""
    import torch
    _on_device(q, lens, out, *kcache.arrays().values(), *vcache.arrays().values())
    if q.dim() != 4 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [batch, n_q_heads, q_len, head_dim] tensor")
    if out.dtype != torch.float32 or not out.is_contiguous() or tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must be a contiguous float32 tensor shaped like q")
    if lens.dtype != torch.int32 or lens.numel() != q.shape[0] or not lens.is_contiguous():
        raise ValueError("lens must be a contiguous int32 tensor of length batch")
    ks, vs = kcache.as_struct(), vcache.as_struct()
    _check(_lib.tq_decode_attention_noalloc(kc.handle, vc.handle, ctypes.c_void_p(q.data_ptr()), _dtype_code(q),
                                            int(q.shape[0]), int(q.shape[1]), int(kcache.heads), int(q.shape[2]),
                                            ctypes.byref(ks), ctypes.byref(vs), ctypes.c_void_p(lens.data_ptr()),
                                            int(max_len), ctypes.c_float(scale), ctypes.c_void_p(out.data_ptr()),
                                            _stream(stream)))


def tq_prefill_workspace_size(kc: Codec, vc: Codec, batch: int, n_q_heads: int, n_kv_heads: int, q_len: int,
                              max_len: int) -> int:
    n = ctypes.c_size_t()
    _check(_lib.tq_prefill_workspace_size(kc.handle, vc.handle, int(batch), int(n_q_heads), int(n_kv_heads),
                                          int(q_len), int(max_len), ctypes.byref(n)))
    return n.value


def allocate_prefill_workspace(kc: Codec, vc: Codec, batch: int, n_q_heads: int, n_kv_heads: int, q_len: int,
                               max_len: int, device="cuda"):
    """A device workspace for tq_prefill_attention with these sizes."""
    import torch
    return torch.zeros(tq_prefill_workspace_size(kc, vc, batch, n_q_heads, n_kv_heads, q_len, max_len),
                       dtype=torch.uint8, device=device)


def tq_prefill_attention(kc: Codec, vc: Codec, q, kcache: Cache, vcache: Cache, lens, max_len: int, scale: float,
                         out, ws, stream=None) -> None:
    """Like tq_decode_attention for any q_len (the q_len new tokens attend to
    the cache and causally to each other); ws: at least
    tq_prefill_workspace_size(...) bytes (allocate_prefill_workspace)."""
    _attention(_lib.tq_prefill_attention, kc, vc, q, kcache, vcache, lens, max_len, scale, out, ws, stream)


def tq_cache_gather(src_codec: Codec, src: Cache, dst_codec: Codec, dst: Cache, src_batch, src_start, count,
                    stream=None) -> None:
    """Copy token records: destination sequence b gets tokens src_start[b] ..
    src_start[b]+count[b]-1 of source sequence src_batch[b] (skipped when
    src_batch[b] < 0) in slots 0 .. count[b]-1.  The three lists have
    dst.batch entries (host integers)."""
    _on_device(*src.arrays().values(), *dst.arrays().values())
    n = int(dst.batch)
    if not (len(src_batch) == len(src_start) == len(count) == n):
        raise ValueError("src_batch, src_start and count need one entry per destination sequence")
    arr = lambda xs: (ctypes.c_int32 * n)(*[int(x) for x in xs])
    ss, ds = src.as_struct(), dst.as_struct()
    _check(_lib.tq_cache_gather(src_codec.handle, ctypes.byref(ss), dst_codec.handle, ctypes.byref(ds),
                                arr(src_batch), arr(src_start), arr(count), _stream(stream)))


def tq_stream_read(buf, sink, blocks: int, stream=None) -> None:
    """Measurement: one streaming read of the device tensor ``buf`` (all its
    bytes; 16-byte aligned, a multiple of 16 bytes); ``sink``: a device tensor
    of at least blocks * 256 32-bit elements."""
    _on_device(buf, sink)
    nbytes = buf.numel() * buf.element_size()
    if sink.numel() * sink.element_size() < 4 * 256 * int(blocks):
        raise ValueError("sink needs blocks * 256 32-bit elements")
    _check(_lib.tq_stream_read(ctypes.c_void_p(buf.data_ptr()), ctypes.c_uint64(nbytes),
                               ctypes.c_void_p(sink.data_ptr()), int(blocks), _stream(stream)))


def tq_decode_read_reference(kc: Codec, vc: Codec, kcache: Cache, vcache: Cache, lens, max_len: int, sink,
                             stream=None) -> None:
    """Measurement: the packed K/V state that tq_decode_attention reads for
    these caches, read once in the int8 decode kernel's own grid and load
    pattern with no arithmetic (3-bit MSE head_dim 128 codecs only).
    ``sink``: a device tensor of 32-bit elements (any length >= 1)."""
    import torch
    _on_device(lens, sink, *kcache.arrays().values(), *vcache.arrays().values())
    if lens.dtype != torch.int32 or not lens.is_contiguous():
        raise ValueError("lens must be a contiguous int32 tensor of length batch")
    words = sink.numel() * sink.element_size() // 4
    if words < 1:
        raise ValueError("sink needs at least one 32-bit element")
    ks, vs = kcache.as_struct(), vcache.as_struct()
    _check(_lib.tq_decode_read_reference(kc.handle, vc.handle, int(kcache.batch), int(kcache.heads),
                                         ctypes.byref(ks), ctypes.byref(vs), ctypes.c_void_p(lens.data_ptr()),
                                         int(max_len), ctypes.c_void_p(sink.data_ptr()), ctypes.c_uint32(words),
                                         _stream(stream)))


# ---- hybrid cache (recent-token rings in front of the compressed caches) -------

def allocate_ring(batch: int, heads: int, buf_size: int, head_dim: int, dtype=None, device="cuda"):
    """A zero-filled recent-token ring [batch, heads, buf_size, head_dim]."""
    import torch
    return torch.zeros((batch, heads, buf_size, head_dim), dtype=dtype or torch.bfloat16, device=device)


def tq_hybrid_append(kc: Codec, vc: Codec, k, v, kcache: Cache, vcache: Cache, kbuf, vbuf, lens, len_end: int,
                     stream=None) -> None:
    """Append k, v [batch, heads, n_new, head_dim] to hybrid caches whose
    sequences hold lens[b] tokens (int32 device tensor); the rings kbuf, vbuf
    [batch, heads, buf_size, head_dim] have the inputs' dtype; len_end bounds
    lens[b] + n_new on the host."""
    import torch
    _on_device(k, v, kbuf, vbuf, lens, *kcache.arrays().values(), *vcache.arrays().values())
    for x in (k, v):
        if x.dim() != 4 or x.stride(3) != 1:
            raise ValueError("k and v must be [batch, heads, n_new, head_dim] with unit coordinate stride")
    if tuple(k.shape) != tuple(v.shape) or k.dtype != v.dtype or kbuf.dtype != k.dtype or vbuf.dtype != k.dtype:
        raise ValueError("k, v and the rings must share shape and dtype")
    for r in (kbuf, vbuf):
        if r.dim() != 4 or not r.is_contiguous() or r.shape[0] != k.shape[0] or r.shape[1] != k.shape[1] \
                or r.shape[3] != k.shape[3]:
            raise ValueError("rings must be contiguous [batch, heads, buf_size, head_dim]")
    if lens.dtype != torch.int32 or lens.numel() != k.shape[0] or not lens.is_contiguous():
        raise ValueError("lens must be a contiguous int32 tensor of length batch")
    ks_, vs_ = (ctypes.c_int64 * 4)(*k.stride()), (ctypes.c_int64 * 4)(*v.stride())
    kst, vst = kcache.as_struct(), vcache.as_struct()
    _check(_lib.tq_hybrid_append(kc.handle, vc.handle, ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                                 _dtype_code(k), int(k.shape[0]), int(k.shape[1]), int(k.shape[2]), ks_, vs_,
                                 ctypes.byref(kst), ctypes.byref(vst), ctypes.c_void_p(kbuf.data_ptr()),
                                 ctypes.c_void_p(vbuf.data_ptr()), int(kbuf.shape[2]),
                                 ctypes.c_void_p(lens.data_ptr()), int(len_end), _stream(stream)))


def tq_hybrid_decode_workspace_size(kc: Codec, vc: Codec, batch: int, n_q_heads: int, n_kv_heads: int, q_len: int,
                                    max_len: int, buf_size: int) -> int:
    n = ctypes.c_size_t()
    _check(_lib.tq_hybrid_decode_workspace_size(kc.handle, vc.handle, int(batch), int(n_q_heads), int(n_kv_heads),
                                                int(q_len), int(max_len), int(buf_size), ctypes.byref(n)))
    return n.value


def tq_hybrid_decode_attention(kc: Codec, vc: Codec, q, kcache: Cache, vcache: Cache, kbuf, vbuf, lens,
                               max_len: int, scale: float, out, ws, stream=None) -> None:
    """Decode attention over hybrid caches (lens: whole lengths, device int32)."""
    import torch
    _on_device(q, lens, out, ws, kbuf, vbuf, *kcache.arrays().values(), *vcache.arrays().values())
    if q.dim() != 4 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [batch, n_q_heads, q_len, head_dim] tensor")
    if out.dtype != torch.float32 or not out.is_contiguous() or tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must be a contiguous float32 tensor shaped like q")
    if kbuf.dtype != vbuf.dtype or tuple(kbuf.shape) != tuple(vbuf.shape) or not kbuf.is_contiguous() \
            or not vbuf.is_contiguous():
        raise ValueError("rings must be contiguous tensors of one shape and dtype")
    if lens.dtype != torch.int32 or lens.numel() != q.shape[0] or not lens.is_contiguous():
        raise ValueError("lens must be a contiguous int32 tensor of length batch")
    ks, vs = kcache.as_struct(), vcache.as_struct()
    _check(_lib.tq_hybrid_decode_attention(kc.handle, vc.handle, ctypes.c_void_p(q.data_ptr()), _dtype_code(q),
                                           int(q.shape[0]), int(q.shape[1]), int(kcache.heads), int(q.shape[2]),
                                           ctypes.byref(ks), ctypes.byref(vs), ctypes.c_void_p(kbuf.data_ptr()),
                                           ctypes.c_void_p(vbuf.data_ptr()), _dtype_code(kbuf), int(kbuf.shape[2]),
                                           ctypes.c_void_p(lens.data_ptr()), int(max_len), ctypes.c_float(scale),
                                           ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                                           ws.numel() * ws.element_size(), _stream(stream)))
