"""fp64 reference for the paged-KV decode step — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this module.  It is written from the definitions below and
shares nothing with the HIP library.

What the step computes.  The llm-d router blog post (opening section, on what
vLLM/SGLang do at the node level) names paged attention and continuous
batching as the engine's core technique and, in its disaggregated-P/D
paragraph, notes that decode is memory-bandwidth bound.  None of the pages
writes the attention formula down; the plainest reading, taken here, is
textbook scaled dot-product softmax attention of one new query token per
sequence over that sequence's cached tokens:

    out[b, h] = sum_t softmax_t(scale * q[b, h] . k[b, t, g(h)]) * v[b, t, g(h)]

with t over the sequence's context_len tokens (the appended token included)
and g(h) = h // (Hq / Hkv) the key/value head a query head reads (contiguous
grouped-query groups).

Where the cached tokens live.  A shared pool of fixed-size pages
(``page_size`` / ``num_pages`` in the llm-d blog post's engine metric spec;
``num_gpu_blocks`` / ``block_size`` on the vLLM EngineCoreClient page,
"Archivos clave"), indexed per sequence through a block table; sequences with
a common prefix point at the same physical pages (llm-d blog post, the
prefix-cache producer section).  Pool layout read by this oracle:

    k_cache[page][kv_head][slot_in_page][dim]
    v_cache[page][kv_head][dim][slot_in_page]

Token position p of sequence b lives at page block_tables[b][p // page_size],
in-page slot p % page_size.

Precision: every floating-point step runs in float64; bf16 storage is widened
exactly (a bf16 value is the top 16 bits of an IEEE binary32).
"""
from __future__ import annotations

import math

import numpy as np


def bf16_bits_to_float64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64, exactly."""
    wide = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return wide.view(np.float32).astype(np.float64)


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (round to nearest, ties to even) in one
    step, returning the uint16 bit patterns.

    The pages fix no output rounding; the reading taken is that a bf16 output
    is the exact result rounded once to nearest-even.  bf16 keeps 8
    significant bits over binary32's exponent range: normal values have the
    quantum 2^(e - 7) for 2^e <= |x| < 2^(e + 1), e >= -126; below 2^-126 the
    quantum stays 2^-133 (subnormals).  Magnitudes that round past the largest
    finite value (2 - 2^-7) * 2^127 become infinity; NaN becomes 0x7FC0.
    """
    a = np.asarray(x, dtype=np.float64)
    flat = a.reshape(-1)
    out = np.zeros(flat.shape, dtype=np.uint16)
    for i, v in enumerate(flat.tolist()):
        if v != v:
            out[i] = 0x7FC0
            continue
        sign = 0x8000 if math.copysign(1.0, v) < 0 else 0
        m = abs(v)
        if m == 0.0:
            out[i] = sign
            continue
        if m != math.inf:
            e = max(math.frexp(m)[1] - 1, -126)    # 2^e <= m < 2^(e+1), or subnormal
            quantum = math.ldexp(1.0, e - 7)
            m = round(m / quantum) * quantum       # Python round(): ties to even
        if m >= math.ldexp(1.0, 128):
            out[i] = sign | 0x7F80
            continue
        # m is now a bf16 value: its binary32 pattern ends in 16 zero bits.
        bits32 = int(np.array([m], dtype=np.float32).view(np.uint32)[0])
        out[i] = sign | (bits32 >> 16)
    return out.reshape(a.shape)


def bf16_ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Number of bf16 values between two finite bf16 patterns, counted along
    the number line (+0 and -0 are the same point)."""
    def ordered(bits):
        b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
        mag = b & 0x7FFF
        return np.where(b & 0x8000, -mag, mag)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def to_float64(values: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array ("f32" floats, "bf16" bit patterns, or "f64") -> float64."""
    if dtype == "f64":
        return np.asarray(values, dtype=np.float64)
    if dtype == "f32":
        return np.asarray(values, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_float64(values)
    raise ValueError(dtype)


def cache_write(k_cache, v_cache, key, value, slot_mapping, page_size):
    """Place each token's K and V rows at its slot; return new pool copies.

    Token t with slot s >= 0 goes to page s // page_size, in-page position
    s % page_size, for every kv head; a negative slot means "write nothing".
    This is the slot-mapped cache write that appends one decode step's tokens
    to the page pool (the KV cache the llm-d blog post's prefix-cache section
    describes vLLM allocating and evicting page by page).  Pure data movement:
    the stored bits are the input bits.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    pages = slots[keep] // page_size
    offs = slots[keep] % page_size
    key = np.asarray(key)[keep]
    value = np.asarray(value)[keep]
    for i in range(pages.shape[0]):
        kc[pages[i], :, offs[i], :] = key[i]
        vc[pages[i], :, :, offs[i]] = value[i]
    return kc, vc


def gather_sequence(k_cache, v_cache, table_row, context_len, page_size):
    """Collect one sequence's first ``context_len`` tokens into contiguous
    ``K[t][kv_head][dim]`` and ``V[t][kv_head][dim]`` (storage dtype).

    Only the first ceil(context_len / page_size) block-table entries are read.
    """
    L = int(context_len)
    n = (L + page_size - 1) // page_size
    pages = np.asarray(table_row[:n], dtype=np.int64)
    K = np.asarray(k_cache)[pages]                  # [n][Hkv][P][D]
    V = np.asarray(v_cache)[pages]                  # [n][Hkv][D][P]
    Hkv, D = K.shape[1], K.shape[3]
    K = K.transpose(0, 2, 1, 3).reshape(n * page_size, Hkv, D)[:L]
    V = V.transpose(0, 3, 1, 2).reshape(n * page_size, Hkv, D)[:L]
    return K, V


def attention(q, K, V, scale):
    """Textbook softmax attention of one query token per head.

    q: [Hq][D], K and V: [L][Hkv][D] (float64); query head h reads kv head
    h // (Hq // Hkv).  Returns [Hq][D].  An empty context (L = 0) yields zeros.
    """
    Hq, D = q.shape
    L, Hkv = K.shape[0], K.shape[1]
    group = Hq // Hkv
    out = np.zeros((Hq, D), dtype=np.float64)
    if L == 0:
        return out
    for h in range(Hq):
        g = h // group
        s = scale * (K[:, g, :] @ q[h])             # [L]
        p = np.exp(s - s.max())
        p = p / p.sum()
        out[h] = p @ V[:, g, :]
    return out


def decode(query, k_cache, v_cache, block_tables, context_lens, scale, page_size, dtype):
    """Decode attention for a whole batch; returns float64 [B][Hq][D].

    Each sequence gathers its own pages (so pages shared by several block
    tables are simply read by each of them) and runs :func:`attention`.
    """
    q64 = to_float64(query, dtype)
    B, Hq, D = q64.shape
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        K, V = gather_sequence(k_cache, v_cache, block_tables[b], context_lens[b], page_size)
        out[b] = attention(q64[b], to_float64(K, dtype), to_float64(V, dtype), scale)
    return out


def partition_attention(q, K, V, scale, partition_size):
    """Split-KV partials of one sequence.

    Tokens are cut at multiples of ``partition_size`` from position 0.  For
    partition k and head h:  m = max of its scaled scores,
    l = sum_t exp(s_t - m),  o = sum_t exp(s_t - m) v_t / l.
    Returns m [Hq][n], l [Hq][n], o [Hq][n][D] with n = ceil(L / partition_size).
    """
    Hq, D = q.shape
    L, Hkv = K.shape[0], K.shape[1]
    group = Hq // Hkv
    n = (L + partition_size - 1) // partition_size
    m = np.zeros((Hq, n))
    lsum = np.zeros((Hq, n))
    o = np.zeros((Hq, n, D))
    for h in range(Hq):
        g = h // group
        for k in range(n):
            lo, hi = k * partition_size, min((k + 1) * partition_size, L)
            s = scale * (K[lo:hi, g, :] @ q[h])
            m[h, k] = s.max()
            e = np.exp(s - m[h, k])
            lsum[h, k] = e.sum()
            o[h, k] = (e @ V[lo:hi, g, :]) / lsum[h, k]
    return m, lsum, o


def combine_partitions(m, lsum, o):
    """Log-sum-exp merge of split-KV partials for one sequence.

    With M = max_k m_k and w_k = l_k exp(m_k - M):  out = sum_k w_k o_k / sum_k w_k.
    m, lsum: [Hq][n]; o: [Hq][n][D].  n = 0 gives zeros.
    """
    Hq, n, D = o.shape
    if n == 0:
        return np.zeros((Hq, D))
    M = m.max(axis=1, keepdims=True)
    w = lsum * np.exp(m - M)                        # [Hq][n]
    return (w[:, :, None] * o).sum(axis=1) / w.sum(axis=1, keepdims=True)


def decode_partials(query, k_cache, v_cache, block_tables, context_lens, scale,
                    page_size, dtype, partition_size, max_num_partitions):
    """Split-KV partials for a whole batch, in the pa_decode_reduce input layout.

    Returns (partial_out [B][Hq][P][D], partial_max [B][Hq][P], partial_sum
    [B][Hq][P]) as float64; entries past a sequence's partition count are 0.
    """
    q64 = to_float64(query, dtype)
    B, Hq, D = q64.shape
    po = np.zeros((B, Hq, max_num_partitions, D))
    pm = np.zeros((B, Hq, max_num_partitions))
    ps = np.zeros((B, Hq, max_num_partitions))
    for b in range(B):
        K, V = gather_sequence(k_cache, v_cache, block_tables[b], context_lens[b], page_size)
        m, lsum, o = partition_attention(q64[b], to_float64(K, dtype), to_float64(V, dtype),
                                         scale, partition_size)
        n = m.shape[1]
        if n > max_num_partitions:
            raise ValueError("sequence needs more partitions than max_num_partitions")
        pm[b, :, :n] = m
        ps[b, :, :n] = lsum
        po[b, :, :n] = o
    return po, pm, ps


# ------------------------------------------------------- multi-token queries
# The step on the other side of decode.  The llm-d blog post (the section on
# the two phases of inference, and the disaggregated-P/D paragraph) separates
# prefill (compute bound) from decode (memory-bandwidth bound); TensorRT
# Edge-LLM ("Model Loading") loads an optional draft checkpoint, i.e. several
# proposed tokens per step that the target model then verifies.  Both run
# several query tokens of one sequence against its paged cache at once.  The
# pages give no formula; the plainest reading, taken here, is causal
# attention: the q_len new tokens of sequence b are its last q_len positions,
# already written to the cache, and the token at position p attends to
# positions 0..p.  With q_len = 1 this is exactly :func:`decode`.


def causal_attention(q, K, V, scale, positions):
    """Several query tokens of one sequence, each over the tokens up to and
    including its own position.

    q: [T][Hq][D]; K and V: [L][Hkv][D] (float64); positions: [T] ints in
    [0, L).  Query token i is plain :func:`attention` over K[:positions[i] + 1].
    Returns [T][Hq][D].
    """
    T, Hq, D = q.shape
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for i in range(T):
        p = int(positions[i])
        out[i] = attention(q[i], K[:p + 1], V[:p + 1], scale)
    return out


def chunk_attention(query, k_cache, v_cache, block_tables, context_lens, query_start, scale,
                    page_size, dtype):
    """Multi-token causal attention over paged K/V for a whole batch.

    query: [T][Hq][D] (storage dtype) holds the new tokens of all sequences,
    sequence b's in rows query_start[b] .. query_start[b + 1] - 1 (so
    q_len_b = query_start[b + 1] - query_start[b], with q_len_b <= L_b).  Row
    query_start[b] + i is the token at position L_b - q_len_b + i.  Returns
    float64 [T][Hq][D]; rows of a sequence with q_len_b = 0 do not exist.
    """
    q64 = to_float64(query, dtype)
    T, Hq, D = q64.shape
    out = np.zeros((T, Hq, D), dtype=np.float64)
    qs = np.asarray(query_start, dtype=np.int64)
    for b in range(len(qs) - 1):
        lo, hi = int(qs[b]), int(qs[b + 1])
        if hi == lo:
            continue
        L = int(context_lens[b])
        q_len = hi - lo
        if q_len > L:
            raise ValueError("more query tokens than context tokens")
        K, V = gather_sequence(k_cache, v_cache, block_tables[b], L, page_size)
        positions = np.arange(L - q_len, L)
        out[lo:hi] = causal_attention(q64[lo:hi], to_float64(K, dtype), to_float64(V, dtype),
                                      scale, positions)
    return out

# ---------------------------------------------------------------- page hand-off
# The llm-d router blog post (disaggregated prefill/decode section) describes
# the KV cache computed on prefill pods being transferred to decode pods.  The
# part of that hand-off that runs on a GPU is a gather of a sequence's pages
# into one buffer on the sending side and a scatter of that buffer into pages
# of the receiving pool.  Buffer layout read here:
#
#     buffer[0][i] = k_cache[page_ids[i]]   flattened ([Hkv][page_size][D])
#     buffer[1][i] = v_cache[page_ids[i]]   flattened ([Hkv][D][page_size])
#
# Page ids outside [0, num_pages) are skipped: export leaves their buffer
# blocks as they were, import writes nothing for them.  Both directions are
# pure data movement; the bits are the input bits.


def export_pages(k_cache, v_cache, page_ids, buffer=None):
    """Gather the listed pages into a new buffer [2][n][block] (a copy of
    ``buffer`` when one is given, so skipped ids keep its contents)."""
    kc = np.asarray(k_cache)
    vc = np.asarray(v_cache)
    ids = np.asarray(page_ids, dtype=np.int64)
    n = ids.shape[0]
    block = int(np.prod(kc.shape[1:]))
    if buffer is None:
        out = np.zeros((2, n, block), dtype=kc.dtype)
    else:
        out = np.array(buffer, copy=True).reshape(2, n, block)
    for i in range(n):
        p = int(ids[i])
        if 0 <= p < kc.shape[0]:
            out[0, i] = kc[p].reshape(-1)
            out[1, i] = vc[p].reshape(-1)
    return out


def import_pages(k_cache, v_cache, buffer, page_ids):
    """Scatter buffer [2][n][block] into the listed pages; return new pool
    copies (every page not listed keeps its bits)."""
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    ids = np.asarray(page_ids, dtype=np.int64)
    n = ids.shape[0]
    buf = np.asarray(buffer).reshape(2, n, -1)
    for i in range(n):
        p = int(ids[i])
        if 0 <= p < kc.shape[0]:
            kc[p] = buf[0, i].reshape(kc.shape[1:])
            vc[p] = buf[1, i].reshape(vc.shape[1:])
    return kc, vc
