"""ctypes binding of libpa.so: argument marshalling only.

Each function takes torch tensors that live in GPU memory, checks their
shapes against each other, and passes raw device pointers, sizes and the
current HIP stream to the C entry point of the same name.  All arithmetic
runs in the library's kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_OK = 0
PA_ERR_INVALID_ARGUMENT = 1
PA_ERR_UNSUPPORTED = 2
PA_ERR_LAUNCH = 3
PA_ERR_SCRATCH_LIMIT = 4
SCRATCH_BYTES = 64 * 1024 * 1024  # the per-GPU array of pa_chunk_attention_split_noalloc
PA_DTYPE_F32 = 0
PA_DTYPE_BF16 = 1
PAGE_SIZE = 16

_c_void_p = ctypes.c_void_p
_i32 = ctypes.c_int
_i64 = ctypes.c_int64
_f32 = ctypes.c_float

_SIGNATURES = {
    "pa_reshape_and_cache": [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i32,
                             _i32, _i32, _i64, _i32, _c_void_p],
    "pa_decode": [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i32,
                  _i32, _i32, _i32, _i32, _i64, _f32, _i32, _i32, _c_void_p, _c_void_p,
                  _c_void_p, _i32, _c_void_p],
    "pa_decode_valu": [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32,
                       _i32, _i32, _i32, _i32, _i32, _i64, _f32, _i32, _i32, _c_void_p,
                       _c_void_p, _c_void_p, _i32, _c_void_p],
    "pa_decode_append": [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                         _c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32, _i32, _i32, _i32,
                         _i64, _f32, _i32, _i32, _c_void_p, _c_void_p, _c_void_p, _i32,
                         _c_void_p],
    "pa_decode_cascade": [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                          _c_void_p, _c_void_p, _i32, _i32, _i32, _i32, _i32, _i32, _i64, _f32,
                          _i32, _i32, _c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32, _i32,
                          _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _c_void_p],
    "pa_chunk_attention": [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                           _c_void_p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i64,
                           _f32, _i32, _c_void_p],
    "pa_chunk_attention_split": [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                 _c_void_p, _c_void_p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                 _i32, _i64, _f32, _i32, _i32, _c_void_p, _c_void_p, _c_void_p,
                                 _i32, _c_void_p],
    "pa_chunk_attention_split_noalloc": [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                         _c_void_p, _c_void_p, _i32, _i32, _i32, _i32, _i32,
                                         _i32, _i32, _i32, _i64, _f32, _i32, _i32, _i32,
                                         _c_void_p],
    "pa_decode_reduce": [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32,
                         _i32, _i32, _i32, _c_void_p],
    "pa_export_pages": [_c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p, _i64, _i32, _i32, _i32,
                        _i64, _i32, _c_void_p],
    "pa_import_pages": [_c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p, _i64, _i32, _i32, _i32,
                        _i64, _i32, _c_void_p],
    "pa_status_string": [_i32],
    "pa_version": [],
}

_lib = None


class PaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpa.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m paged_kv_decode_pa_amd.build` "
            "(there is no fallback implementation)")
    # torch ships its own HIP runtime; loading it first makes libpa.so bind to
    # that same runtime (one HIP context per process) instead of a second copy.
    import torch  # noqa: F401

    lib = ctypes.CDLL(path)
    for name, argtypes in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = ctypes.c_char_p if name == "pa_status_string" else ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().pa_status_string(status).decode()


def version() -> int:
    return load().pa_version()


def _check(fn: str, status: int) -> None:
    if status != PA_OK:
        raise PaError(fn, status)


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return PA_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return PA_DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream) -> int:
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("tensors must be contiguous and in GPU memory")
    return t.data_ptr()


def pa_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, stream=None) -> None:
    """key/value [T][Hkv][D]; k_cache [pages][Hkv][16][D]; v_cache [pages][Hkv][D][16];
    slot_mapping int64 [T]."""
    T, Hkv, D = key.shape
    if value.shape != key.shape or tuple(slot_mapping.shape) != (T,):
        raise ValueError("key, value and slot_mapping disagree")
    if k_cache.shape[1:] != (Hkv, PAGE_SIZE, D) or v_cache.shape[1:] != (Hkv, D, PAGE_SIZE):
        raise ValueError("pool shape does not match key")
    if not (key.dtype == value.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("key, value and pools must share one dtype")
    lib = load()
    _check("pa_reshape_and_cache", lib.pa_reshape_and_cache(
        _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), T, Hkv, D,
        PAGE_SIZE, k_cache.shape[0], _dtype_code(key), _stream(stream)))


def _decode(name, out, query, k_cache, v_cache, block_tables, context_lens, scale,
            partition_size=0, partial_out=None, partial_max=None, partial_sum=None,
            stream=None) -> None:
    B, Hq, D = query.shape
    Hkv = k_cache.shape[1]
    if k_cache.shape[2:] != (PAGE_SIZE, D) or v_cache.shape[1:] != (Hkv, D, PAGE_SIZE):
        raise ValueError("pool shape does not match query")
    if block_tables.shape[0] != B or tuple(context_lens.shape) != (B,):
        raise ValueError("block_tables / context_lens do not match the batch")
    max_parts = 0
    if partition_size:
        max_parts = partial_max.shape[2]
        if (partial_out.shape != (B, Hq, max_parts, D) or partial_max.shape != (B, Hq, max_parts)
                or partial_sum.shape != (B, Hq, max_parts)):
            raise ValueError("partial buffers have the wrong shape")
    elif out is None or out.shape != query.shape or out.dtype != query.dtype:
        raise ValueError("out must match query")
    lib = load()
    _check(name, getattr(lib, name)(
        _ptr(out), _ptr(query), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        _ptr(context_lens), B, Hq, Hkv, D, PAGE_SIZE, block_tables.shape[1], k_cache.shape[0],
        float(scale), int(partition_size), max_parts, _ptr(partial_out), _ptr(partial_max),
        _ptr(partial_sum), _dtype_code(query), _stream(stream)))


def pa_decode(out, query, k_cache, v_cache, block_tables, context_lens, scale,
              partition_size=0, partial_out=None, partial_max=None, partial_sum=None,
              stream=None) -> None:
    """Decode attention; see include/pa.h.  With partition_size > 0 only the
    partial buffers are written (then call pa_decode_reduce)."""
    _decode("pa_decode", out, query, k_cache, v_cache, block_tables, context_lens, scale,
            partition_size, partial_out, partial_max, partial_sum, stream)


def pa_decode_append(out, query, key, value, slot_mapping, k_cache, v_cache, block_tables,
                     context_lens, scale, partition_size=0, partial_out=None, partial_max=None,
                     partial_sum=None, stream=None) -> None:
    """One decode step: write each sequence's new token (key/value [B][Hkv][D],
    slot_mapping int64 [B]) and attend; see include/pa.h."""
    B, Hq, D = query.shape
    Hkv = k_cache.shape[1]
    if key.shape != (B, Hkv, D) or value.shape != key.shape or tuple(slot_mapping.shape) != (B,):
        raise ValueError("key, value and slot_mapping must hold one token per sequence")
    if not (key.dtype == value.dtype == query.dtype == k_cache.dtype):
        raise TypeError("key, value, query and pools must share one dtype")
    if k_cache.shape[2:] != (PAGE_SIZE, D) or v_cache.shape[1:] != (Hkv, D, PAGE_SIZE):
        raise ValueError("pool shape does not match query")
    if block_tables.shape[0] != B or tuple(context_lens.shape) != (B,):
        raise ValueError("block_tables / context_lens do not match the batch")
    max_parts = 0
    if partition_size:
        max_parts = partial_max.shape[2]
        if (partial_out.shape != (B, Hq, max_parts, D) or partial_max.shape != (B, Hq, max_parts)
                or partial_sum.shape != (B, Hq, max_parts)):
            raise ValueError("partial buffers have the wrong shape")
    elif out is None or out.shape != query.shape or out.dtype != query.dtype:
        raise ValueError("out must match query")
    lib = load()
    _check("pa_decode_append", lib.pa_decode_append(
        _ptr(out), _ptr(query), _ptr(key), _ptr(value), _ptr(slot_mapping), _ptr(k_cache),
        _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), B, Hq, Hkv, D, PAGE_SIZE,
        block_tables.shape[1], k_cache.shape[0], float(scale), int(partition_size), max_parts,
        _ptr(partial_out), _ptr(partial_max), _ptr(partial_sum), _dtype_code(query),
        _stream(stream)))


def pa_decode_cascade(query, k_cache, v_cache, block_tables, context_lens, scale,
                      partition_size, partial_out, partial_max, partial_sum, groups,
                      key=None, value=None, slot_mapping=None, stream=None) -> None:
    """Split-KV partials with shared prefixes read once per group; `groups`
    holds device int32 tensors group_start / group_seqs / group_partitions /
    seq_first_partition and the host ints num_groups / max_group_size /
    max_group_partitions / max_suffix_partitions (optional: 0 = no bound)
    (paged_kv_decode_pa_amd.prefix_groups gives them on the host).  Merge with pa_decode_reduce.  See include/pa.h."""
    B, Hq, D = query.shape
    Hkv = k_cache.shape[1]
    if k_cache.shape[2:] != (PAGE_SIZE, D) or v_cache.shape[1:] != (Hkv, D, PAGE_SIZE):
        raise ValueError("pool shape does not match query")
    if block_tables.shape[0] != B or tuple(context_lens.shape) != (B,):
        raise ValueError("block_tables / context_lens do not match the batch")
    P = partial_max.shape[2]
    if (partial_out.shape != (B, Hq, P, D) or partial_max.shape != (B, Hq, P)
            or partial_sum.shape != (B, Hq, P)):
        raise ValueError("partial buffers have the wrong shape")
    if key is not None and (key.shape != (B, Hkv, D) or value.shape != key.shape
                            or tuple(slot_mapping.shape) != (B,)):
        raise ValueError("key, value and slot_mapping must hold one token per sequence")
    lib = load()
    _check("pa_decode_cascade", lib.pa_decode_cascade(
        _ptr(query), _ptr(key), _ptr(value), _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache),
        _ptr(block_tables), _ptr(context_lens), B, Hq, Hkv, D, PAGE_SIZE, block_tables.shape[1],
        k_cache.shape[0], float(scale), int(partition_size), P, _ptr(partial_out),
        _ptr(partial_max), _ptr(partial_sum), int(groups["num_groups"]),
        int(groups["max_group_size"]), int(groups["max_group_partitions"]),
        int(groups.get("max_suffix_partitions", 0)),
        _ptr(groups.get("group_start")), _ptr(groups.get("group_seqs")),
        _ptr(groups.get("group_partitions")), _ptr(groups.get("seq_first_partition")),
        _dtype_code(query), _stream(stream)))


def pa_chunk_attention(out, query, k_cache, v_cache, block_tables, context_lens, query_start,
                       max_query_len, scale, stream=None) -> None:
    """Causal attention of several new tokens per sequence; see include/pa.h.
    query/out [T][Hq][D] bf16; query_start int32 [B + 1]; max_query_len is a
    host bound on every sequence's new-token count."""
    T, Hq, D = query.shape
    B = context_lens.shape[0]
    Hkv = k_cache.shape[1]
    if k_cache.shape[2:] != (PAGE_SIZE, D) or v_cache.shape[1:] != (Hkv, D, PAGE_SIZE):
        raise ValueError("pool shape does not match query")
    if block_tables.shape[0] != B or tuple(query_start.shape) != (B + 1,):
        raise ValueError("block_tables / query_start do not match the batch")
    if out.shape != query.shape or out.dtype != query.dtype:
        raise ValueError("out must match query")
    lib = load()
    _check("pa_chunk_attention", lib.pa_chunk_attention(
        _ptr(out), _ptr(query), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        _ptr(context_lens), _ptr(query_start), B, T, int(max_query_len), Hq, Hkv, D, PAGE_SIZE,
        block_tables.shape[1], k_cache.shape[0], float(scale), _dtype_code(query),
        _stream(stream)))


def pa_chunk_attention_split(out, query, k_cache, v_cache, block_tables, context_lens,
                             query_start, max_query_len, scale, partition_size, partial_out,
                             partial_max, partial_sum, stream=None) -> None:
    """pa_chunk_attention as split-KV units and their merge, in one call; see
    include/pa.h.  partial_out [T][Hq][P][D], partial_max / partial_sum
    [T][Hq][P] fp32 workspace."""
    T, Hq, D = query.shape
    B = context_lens.shape[0]
    Hkv = k_cache.shape[1]
    if k_cache.shape[2:] != (PAGE_SIZE, D) or v_cache.shape[1:] != (Hkv, D, PAGE_SIZE):
        raise ValueError("pool shape does not match query")
    if block_tables.shape[0] != B or tuple(query_start.shape) != (B + 1,):
        raise ValueError("block_tables / query_start do not match the batch")
    if out.shape != query.shape or out.dtype != query.dtype:
        raise ValueError("out must match query")
    P = partial_max.shape[2]
    if (partial_out.shape != (T, Hq, P, D) or partial_max.shape != (T, Hq, P)
            or partial_sum.shape != (T, Hq, P)):
        raise ValueError("partial buffers have the wrong shape")
    lib = load()
    _check("pa_chunk_attention_split", lib.pa_chunk_attention_split(
        _ptr(out), _ptr(query), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        _ptr(context_lens), _ptr(query_start), B, T, int(max_query_len), Hq, Hkv, D, PAGE_SIZE,
        block_tables.shape[1], k_cache.shape[0], float(scale), int(partition_size), P,
        _ptr(partial_out), _ptr(partial_max), _ptr(partial_sum), _dtype_code(query),
        _stream(stream)))


def pa_chunk_attention_split_noalloc(out, query, k_cache, v_cache, block_tables, context_lens,
                                     query_start, max_query_len, scale, partition_size,
                                     max_num_partitions, stream=None) -> None:
    """pa_chunk_attention_split with its partials in the library's fixed
    per-GPU scratch array (SCRATCH_BYTES): the call allocates nothing.  Calls
    that overlap on one GPU race; see include/pa.h."""
    T, Hq, D = query.shape
    B = context_lens.shape[0]
    Hkv = k_cache.shape[1]
    if k_cache.shape[2:] != (PAGE_SIZE, D) or v_cache.shape[1:] != (Hkv, D, PAGE_SIZE):
        raise ValueError("pool shape does not match query")
    if block_tables.shape[0] != B or tuple(query_start.shape) != (B + 1,):
        raise ValueError("block_tables / query_start do not match the batch")
    if out.shape != query.shape or out.dtype != query.dtype:
        raise ValueError("out must match query")
    lib = load()
    _check("pa_chunk_attention_split_noalloc", lib.pa_chunk_attention_split_noalloc(
        _ptr(out), _ptr(query), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        _ptr(context_lens), _ptr(query_start), B, T, int(max_query_len), Hq, Hkv, D, PAGE_SIZE,
        block_tables.shape[1], k_cache.shape[0], float(scale), int(partition_size),
        int(max_num_partitions), _dtype_code(query), _stream(stream)))


def _page_copy(name, buffer, k_cache, v_cache, page_ids, stream):
    n = page_ids.shape[0]
    Hkv, D = k_cache.shape[1], k_cache.shape[3]
    if k_cache.shape[2] != PAGE_SIZE or v_cache.shape != (k_cache.shape[0], Hkv, D, PAGE_SIZE):
        raise ValueError("k_cache / v_cache shapes disagree")
    if not (buffer.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("buffer and pools must share one dtype")
    if page_ids.dim() != 1:
        raise ValueError("page_ids must be one-dimensional")
    lib = load()
    _check(name, getattr(lib, name)(
        _ptr(buffer), buffer.numel() * buffer.element_size(), _ptr(k_cache), _ptr(v_cache),
        _ptr(page_ids), n, Hkv, D, PAGE_SIZE, k_cache.shape[0], _dtype_code(k_cache),
        _stream(stream)))


def pa_export_pages(buffer, k_cache, v_cache, page_ids, stream=None) -> None:
    """Gather pages page_ids (int32 [n]) into buffer [2][n][Hkv][16*D]: the K
    blocks, then the V blocks, each in the pool's own page layout."""
    _page_copy("pa_export_pages", buffer, k_cache, v_cache, page_ids, stream)


def pa_import_pages(buffer, k_cache, v_cache, page_ids, stream=None) -> None:
    """Scatter a buffer laid out as pa_export_pages writes it into pages page_ids."""
    _page_copy("pa_import_pages", buffer, k_cache, v_cache, page_ids, stream)


def pa_decode_valu(out, query, k_cache, v_cache, block_tables, context_lens, scale,
                   partition_size=0, partial_out=None, partial_max=None, partial_sum=None,
                   stream=None) -> None:
    """pa_decode with the vector-ALU kernel forced (same contract)."""
    _decode("pa_decode_valu", out, query, k_cache, v_cache, block_tables, context_lens, scale,
            partition_size, partial_out, partial_max, partial_sum, stream)


def pa_decode_reduce(out, partial_out, partial_max, partial_sum, context_lens, partition_size,
                     stream=None) -> None:
    """Merge split-KV partials [B][Hq][P][D] into out [B][Hq][D]."""
    B, Hq, P, D = partial_out.shape
    if out.shape != (B, Hq, D) or partial_max.shape != (B, Hq, P) or partial_sum.shape != (B, Hq, P):
        raise ValueError("reduce buffers disagree")
    lib = load()
    _check("pa_decode_reduce", lib.pa_decode_reduce(
        _ptr(out), _ptr(partial_out), _ptr(partial_max), _ptr(partial_sum), _ptr(context_lens),
        B, Hq, D, int(partition_size), P, _dtype_code(out), _stream(stream)))
