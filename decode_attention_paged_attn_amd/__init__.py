"""Paged decode attention for MI355X: thin Python binding over the HIP C ABI.

Every step of the computation runs in the HIP kernels of ``libpagedattn.so``;
this package only checks tensor shapes, takes device pointers and torch's
current stream, and allocates the caller-side buffers.  If the library is not
built the calls raise; there is no fallback.
"""
from ._binding import (  # noqa: F401
    PdaError,
    cascade_decode_attn,
    decode_workspace_size,
    lds_probe,
    library_path,
    load_library,
    merge_partials,
    multi_query_workspace_size,
    paged_decode_attn,
    paged_decode_attn_append,
    paged_decode_attn_noalloc,
    paged_decode_attn_partial,
    paged_kv_append,
    paged_multi_query_attn,
    paged_multi_query_attn_partial,
    stream_read,
    workspace_layout,
    workspace_size,
)

__all__ = [
    "PdaError",
    "cascade_decode_attn",
    "decode_workspace_size",
    "lds_probe",
    "library_path",
    "load_library",
    "merge_partials",
    "multi_query_workspace_size",
    "paged_decode_attn",
    "paged_decode_attn_append",
    "paged_decode_attn_noalloc",
    "paged_decode_attn_partial",
    "paged_kv_append",
    "paged_multi_query_attn",
    "paged_multi_query_attn_partial",
    "stream_read",
    "workspace_layout",
    "workspace_size",
]
