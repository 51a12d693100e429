"""Plain fp64 CPU oracle for paged-KV decode attention (and multi-token
causal queries over the same cache, and the page export/import of a KV
hand-off).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers or constants) and imports nothing from
``paged_kv_decode_pa_amd``.

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
invariants, a library routine and brute force; no function here is "parity
unpinned".
"""
from .paged_attention import (  # noqa: F401
    attention,
    bf16_bits_to_float64,
    bf16_ulp_distance,
    cache_write,
    causal_attention,
    chunk_attention,
    combine_partitions,
    decode,
    decode_partials,
    export_pages,
    gather_sequence,
    import_pages,
    partition_attention,
    round_to_bf16_bits,
    to_float64,
)
