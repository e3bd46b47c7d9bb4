"""TurboQuant compressed KV cache and decode attention for AMD MI355X.

Thin Python binding over the C ABI of ``libtq.so`` (``include/tq.h``): the
functions keep the C names and only marshal arguments (torch tensors to device
pointers, the current HIP stream, status codes to exceptions).  Every step of
the hot path runs in the library's HIP kernels; there is no Python or CPU
fallback -- importing the binding fails if the library is not built.
"""
from ._binding import (  # noqa: F401
    TQ_BF16,
    TQ_F32,
    TQ_MODE_GROUP,
    TQ_MODE_MSE,
    TQ_MODE_PROD,
    TQ_MODE_SPLIT,
    Cache,
    Codec,
    TQError,
    allocate_cache,
    allocate_prefill_workspace,
    allocate_ring,
    allocate_workspace,
    lib_path,
    tq_cache_gather,
    tq_codec_create,
    tq_codec_create_kv,
    tq_codec_create_split,
    tq_codec_part,
    tq_codec_destroy,
    tq_codec_export,
    tq_codec_get_info,
    tq_codec_upload,
    tq_decode_attention,
    tq_decode_attention_noalloc,
    tq_decode_read_reference,
    tq_decode_workspace_size,
    tq_hybrid_append,
    tq_hybrid_decode_attention,
    tq_hybrid_decode_workspace_size,
    tq_last_error,
    tq_prefill_attention,
    tq_prefill_workspace_size,
    tq_quantize_append,
    tq_quantize_append_kv,
    tq_status_string,
    tq_stream_read,
)
