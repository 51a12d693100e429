"""Paged-KV decode attention for MI355X (gfx950): Python face of libpa.so.

The entry points mirror include/pa.h one to one; see ``_lib`` for the
marshalling.  Build the library with ``python -m paged_kv_decode_pa_amd.build``.
"""
from ._lib import (  # noqa: F401
    LIB_PATH,
    PAGE_SIZE,
    SCRATCH_BYTES,
    PaError,
    load,
    pa_chunk_attention,
    pa_chunk_attention_split,
    pa_chunk_attention_split_noalloc,
    pa_decode,
    pa_decode_append,
    pa_decode_cascade,
    pa_decode_reduce,
    pa_decode_valu,
    pa_export_pages,
    pa_import_pages,
    pa_reshape_and_cache,
    status_string,
    version,
)
from .pager import Pager, PagerError, page_hash, prefix_groups  # noqa: F401,E402
