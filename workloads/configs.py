"""The five synthetic decode workloads and a generator for custom ones.

Everything here is input drawing: lengths, physical page placement, block
tables, slot mappings and Q/K/V values.  No attention arithmetic lives here.

Shapes follow the serving problem as the source pages frame it: a batch of
sequences (Dragon "Inference Service" guide, "vLLM Integration":
``max_num_seqs`` / ``max_model_len``), each with a context length and a block
table into one shared pool of fixed-size pages (llm-d router blog post, the
engine metric spec naming ``page_size`` / ``num_pages``; vLLM
"EngineCoreClient" page, "Archivos clave": ``num_gpu_blocks`` /
``block_size``), some pages shared across sequences by prefix reuse (llm-d
blog post, the prefix-cache section on reusing a prompt's KV cache).

Pool layout (the storage order the arrays below are destined for):
  K pool  [num_pages][num_kv_heads][page_size][head_dim]
  V pool  [num_pages][num_kv_heads][head_dim][page_size]
Slot ``s`` names page ``s // page_size``, in-page position ``s % page_size``.

Draw order per workload, from ``numpy.random.default_rng(1000 + config_id)``:
  1. context lengths   2. Q   3. K   4. V   5. physical page permutation
K and V are drawn for every logical token once: cached tokens in (logical
page, position) order, then each sequence's appended token (position L-1).
Values are N(0, 1) float32; bf16 workloads round them to nearest-even bf16.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, Optional, Sequence

import numpy as np

PAGE_SIZE = 16


@dataclass(frozen=True)
class DecodeConfig:
    config_id: int
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str  # "f32" or "bf16"
    description: str
    page_size: int = PAGE_SIZE
    # split-KV partition (tokens) the benchmark uses; 0 = single pass
    bench_partition_size: int = 0
    # the benchmark reads shared prefix pages once per group (pa_decode_cascade),
    # at this partition size
    bench_cascade: bool = False
    cascade_partition_size: int = 0
    # number of sequences that share one prefix (0 = no sharing)
    prefix_group_size: int = 0
    prefix_tokens: int = 0

    @property
    def gqa(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


CONFIGS = [
    DecodeConfig(1, "tiny_f32", 4, 8, 2, 64, "f32",
                 "4 sequences, lengths {17,64,100,255}, 8 q / 2 kv heads, D=64, fp32, "
                 "64-page pool placed by a seeded permutation"),
    DecodeConfig(2, "llama3_8b_bf16", 64, 32, 8, 128, "bf16",
                 "batch 64, 32 q / 8 kv heads, D=128, bf16, lengths U[512,4096], "
                 "pages scattered in a pool of 1.25x need",
                 bench_partition_size=0),
    DecodeConfig(3, "prefix_reuse_bf16", 128, 32, 8, 128, "bf16",
                 "batch 128 = 8 groups x 16 sharing a 2048-token prefix, private "
                 "suffixes U[64,512], 32 q / 8 kv heads, D=128, bf16",
                 bench_partition_size=0, prefix_group_size=16, prefix_tokens=2048,
                 bench_cascade=True, cascade_partition_size=2048),
    DecodeConfig(4, "long_splitkv_bf16", 8, 32, 8, 128, "bf16",
                 "batch 8, lengths U[16384,32768], 32 q / 8 kv heads, D=128, bf16, "
                 "512-token partitions reduced by log-sum-exp",
                 bench_partition_size=512),
    DecodeConfig(5, "llama70b_tp8_share_bf16", 256, 8, 1, 128, "bf16",
                 "batch 256, 8 q / 1 kv head, D=128, bf16, lengths log-uniform "
                 "[128,8192] with 25% of sequences at length <= 32",
                 bench_partition_size=512),
]


def config_by_id(config_id: int) -> DecodeConfig:
    for c in CONFIGS:
        if c.config_id == config_id:
            return c
    raise KeyError(config_id)


@dataclass
class Workload:
    """One decode step's inputs, in host memory.

    Token payloads (``query``, ``*_key``, ``*_value``) are float32 arrays for
    fp32 workloads and uint16 arrays holding bf16 bit patterns otherwise.
    """
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    dtype: str
    scale: float
    num_pages: int
    context_lens: np.ndarray      # int32 [B]
    block_tables: np.ndarray      # int32 [B][max_pages_per_seq], -1 padded
    query: np.ndarray             # [B][Hq][D]
    prefill_key: np.ndarray       # [T][Hkv][D]  every cached token except the new one
    prefill_value: np.ndarray
    prefill_slots: np.ndarray     # int64 [T]
    new_key: np.ndarray           # [B][Hkv][D]  the token each sequence appends this step
    new_value: np.ndarray
    new_slots: np.ndarray         # int64 [B]
    unique_pages: int             # distinct physical pages referenced
    name: str = "custom"
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest-even) with torch's CPU cast; return the bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _payload(x: np.ndarray, dtype: str) -> np.ndarray:
    return x.astype(np.float32) if dtype == "f32" else bf16_bits_from_f32(x)


def _build(
    rng: np.random.Generator,
    lengths: np.ndarray,
    *,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    dtype: str,
    page_size: int,
    pool_pages: Optional[int],
    pool_factor: float,
    group_of: Optional[np.ndarray],
    prefix_tokens: int,
    share_prefix: bool,
    placement_rng: Optional[np.random.Generator],
    max_pages_per_seq: Optional[int],
    name: str,
    scale: Optional[float] = None,
    value_fn: Optional[Callable] = None,
) -> Workload:
    lengths = np.asarray(lengths, dtype=np.int64)
    B = int(lengths.shape[0])
    P = page_size
    if prefix_tokens % P:
        raise ValueError("shared prefixes must be whole pages")
    shared_pages = prefix_tokens // P
    n_pages = (lengths + P - 1) // P

    # Logical pages in (sequence, logical page) order; a shared prefix page is
    # one logical page owned by its group.
    page_keys = []
    page_index = {}
    seq_page_keys = []
    for b in range(B):
        keys_b = []
        for j in range(int(n_pages[b])):
            shared = group_of is not None and group_of[b] >= 0 and j < shared_pages
            if shared and j * P + P > lengths[b]:
                raise ValueError("a shared prefix page must be full in every sharer")
            key = ("g", int(group_of[b]), j) if shared else ("s", b, j)
            if key not in page_index:
                page_index[key] = len(page_keys)
                page_keys.append(key)
            keys_b.append(key)
        seq_page_keys.append(keys_b)

    # Physical placement: (un)shared copies are separate physical pages.
    placed_keys = []
    placed_index = {}
    seq_placed = []
    for b in range(B):
        row = []
        for key in seq_page_keys[b]:
            pkey = key if (share_prefix or key[0] == "s") else ("c", b, key[2])
            if pkey not in placed_index:
                placed_index[pkey] = len(placed_keys)
                placed_keys.append(pkey)
            row.append(placed_index[pkey])
        seq_placed.append(row)
    unique = len(placed_keys)
    num_pages = pool_pages if pool_pages is not None else int(math.ceil(pool_factor * unique))
    if num_pages < unique:
        raise ValueError("pool smaller than the pages in use")

    mp = max_pages_per_seq if max_pages_per_seq is not None else max(1, int(n_pages.max(initial=0)))
    if mp < int(n_pages.max(initial=0)):
        raise ValueError("max_pages_per_seq too small")

    # Logical tokens: the cached ones in (logical page, position) order, then
    # each sequence's appended token (position L-1) in batch order.
    appended = set()
    for b in range(B):
        L = int(lengths[b])
        if L == 0:
            continue
        key = seq_page_keys[b][(L - 1) // P]
        if key[0] != "s":
            raise ValueError("the appended token must sit in a private page")
        appended.add((key, L - 1))
    tok_owner = []  # (page key, position)
    for key in page_keys:
        kind, who, j = key
        last = (j + 1) * P if kind == "g" else min((j + 1) * P, int(lengths[who]))
        for pos in range(j * P, last):
            if (key, pos) not in appended:
                tok_owner.append((key, pos))
    n_cached = len(tok_owner)
    for b in range(B):
        L = int(lengths[b])
        if L:
            tok_owner.append((seq_page_keys[b][(L - 1) // P], L - 1))
    T = len(tok_owner)

    # Draws 2-4: values.  The logical tokens do not depend on placement or on
    # whether prefixes are shared, so neither changes any value.
    Hq, Hkv, D = num_q_heads, num_kv_heads, head_dim
    q32 = rng.standard_normal((B, Hq, D), dtype=np.float32)
    k32 = rng.standard_normal((T, Hkv, D), dtype=np.float32)
    v32 = rng.standard_normal((T, Hkv, D), dtype=np.float32)
    if value_fn is not None:
        q32, k32, v32 = value_fn(q32, k32, v32, tok_owner, lengths)

    # Draw 5: the physical permutation; placed page u gets physical id perm[u].
    # A placement-only variant draws it from its own stream instead.
    perm = (placement_rng if placement_rng is not None else rng).permutation(num_pages)
    tables = np.full((B, mp), -1, dtype=np.int32)
    for b in range(B):
        for j, u in enumerate(seq_placed[b]):
            tables[b, j] = perm[u]

    # Slots.  Key -> physical page of its first placement; an unshared copy of
    # a group page belongs to sequence b.
    phys_of = {}
    for b in range(B):
        for j, key in enumerate(seq_page_keys[b]):
            pkey = key if (share_prefix or key[0] == "s") else ("c", b, key[2])
            phys_of.setdefault(pkey, int(tables[b, j]))
    pos_arr = np.fromiter((p for _, p in tok_owner), dtype=np.int64, count=T)
    page_arr = np.fromiter((phys_of[k] if (share_prefix or k[0] == "s") else -1
                            for k, _ in tok_owner), dtype=np.int64, count=T)
    slots = page_arr * P + pos_arr % P
    pre_idx = None
    if not share_prefix and group_of is not None:
        # Each sequence's private copy of a group page receives the same values.
        idx, sl = [], []
        for i in range(n_cached):
            key, pos = tok_owner[i]
            if key[0] == "s":
                idx.append(i)
                sl.append(slots[i])
            else:
                for b in np.nonzero(group_of == key[1])[0]:
                    if key[2] < len(seq_page_keys[b]):
                        idx.append(i)
                        sl.append(phys_of[("c", int(b), key[2])] * P + pos % P)
        pre_idx = np.asarray(idx, dtype=np.int64)
        pre_slots = np.asarray(sl, dtype=np.int64)
    else:
        pre_slots = slots[:n_cached].copy()

    new_slot = np.full(B, -1, dtype=np.int64)
    new_rows = np.zeros(B, dtype=np.int64)
    i = n_cached
    for b in range(B):
        if lengths[b]:
            new_slot[b] = slots[i]
            new_rows[b] = i
            i += 1
    has_new = bool((lengths > 0).all())

    kc = k32[:n_cached] if pre_idx is None else k32[pre_idx]
    vc = v32[:n_cached] if pre_idx is None else v32[pre_idx]
    kn = k32[n_cached:] if has_new else k32[new_rows]
    vn = v32[n_cached:] if has_new else v32[new_rows]
    wl = Workload(
        num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=P, dtype=dtype,
        scale=float(scale if scale is not None else 1.0 / math.sqrt(D)),
        num_pages=int(num_pages),
        context_lens=lengths.astype(np.int32),
        block_tables=tables,
        query=_payload(q32, dtype),
        prefill_key=_payload(kc, dtype),
        prefill_value=_payload(vc, dtype),
        prefill_slots=pre_slots,
        new_key=_payload(kn, dtype),
        new_value=_payload(vn, dtype),
        new_slots=new_slot,
        unique_pages=unique,
        name=name,
    )
    return wl


def _lengths_for(cfg: DecodeConfig, rng: np.random.Generator) -> np.ndarray:
    if cfg.config_id == 1:
        return np.array([17, 64, 100, 255], dtype=np.int64)
    if cfg.config_id == 2:
        return rng.integers(512, 4096, size=cfg.num_seqs, endpoint=True)
    if cfg.config_id == 3:
        return cfg.prefix_tokens + rng.integers(64, 512, size=cfg.num_seqs, endpoint=True)
    if cfg.config_id == 4:
        return rng.integers(16384, 32768, size=cfg.num_seqs, endpoint=True)
    if cfg.config_id == 5:
        n_short = cfg.num_seqs // 4
        short = rng.integers(1, 32, size=n_short, endpoint=True)
        u = rng.uniform(math.log(128.0), math.log(8192.0), size=cfg.num_seqs - n_short)
        long = np.clip(np.rint(np.exp(u)), 128, 8192).astype(np.int64)
        lens = np.concatenate([short, long])
        return lens[rng.permutation(cfg.num_seqs)]
    raise KeyError(cfg.config_id)


def make_workload(cfg: DecodeConfig, *, share_prefix: bool = True,
                  placement_seed: Optional[int] = None) -> Workload:
    """Draw config ``cfg``'s workload.

    ``share_prefix=False`` gives each sequence private copies of its group's
    prefix pages (same values); ``placement_seed`` re-draws only the physical
    page permutation.  Both keep every token value and every length unchanged.
    """
    rng = np.random.default_rng(1000 + cfg.config_id)
    lengths = _lengths_for(cfg, rng)
    group_of = None
    if cfg.prefix_group_size:
        group_of = np.arange(cfg.num_seqs) // cfg.prefix_group_size
    return _build(
        rng, lengths,
        num_q_heads=cfg.num_q_heads, num_kv_heads=cfg.num_kv_heads, head_dim=cfg.head_dim,
        dtype=cfg.dtype, page_size=cfg.page_size,
        pool_pages=64 if cfg.config_id == 1 else None, pool_factor=1.25,
        group_of=group_of, prefix_tokens=cfg.prefix_tokens, share_prefix=share_prefix,
        placement_rng=None if placement_seed is None else np.random.default_rng(placement_seed),
        max_pages_per_seq=None, name=cfg.name,
    )


def make_custom_workload(
    lengths: Sequence[int],
    *,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    dtype: str = "bf16",
    seed: int = 0,
    page_size: int = PAGE_SIZE,
    pool_factor: float = 1.25,
    pool_pages: Optional[int] = None,
    group_size: int = 0,
    group_of: Optional[Sequence[int]] = None,
    prefix_tokens: int = 0,
    share_prefix: bool = True,
    placement_seed: Optional[int] = None,
    max_pages_per_seq: Optional[int] = None,
    scale: Optional[float] = None,
    value_fn: Optional[Callable] = None,
    name: str = "custom",
) -> Workload:
    """A workload with explicit lengths, drawn from ``default_rng(seed)`` in the
    same order as the fixed configs (lengths are given, so draws start at Q).

    ``value_fn(q, k, v, tok_owner, lengths)`` may replace the drawn float32
    values, e.g. to plant a needle token; ``tok_owner[i] = (page_key, position)``.
    Prefix groups are either contiguous runs of ``group_size`` sequences or
    given per sequence by ``group_of`` (-1 = no group), in any batch order.
    """
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int64)
    if group_of is not None:
        group_of = np.asarray(group_of, dtype=np.int64)
        if group_of.shape != lengths.shape:
            raise ValueError("group_of needs one entry per sequence")
    elif group_size:
        group_of = np.arange(len(lengths)) // group_size
    return _build(
        rng, lengths,
        num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
        dtype=dtype, page_size=page_size, pool_pages=pool_pages, pool_factor=pool_factor,
        group_of=group_of, prefix_tokens=prefix_tokens, share_prefix=share_prefix,
        placement_rng=None if placement_seed is None else np.random.default_rng(placement_seed),
        max_pages_per_seq=max_pages_per_seq, name=name, scale=scale, value_fn=value_fn,
    )


def make_chunk_queries(wl: Workload, q_lens: Sequence[int], seed: int = 0,
                       value_fn: Optional[Callable] = None):
    """Query rows for multi-token attention over workload ``wl``'s cache.

    Sequence b gets ``q_lens[b]`` (<= its context length) new query tokens,
    stored back to back: returns (query [T][Hq][D] payload in wl's dtype,
    query_start int32 [B + 1]).  The tokens are the sequence's last q_len
    positions, whose K/V the workload already writes to the pool.  Values are
    N(0,1) float32 from ``default_rng(seed)``, optionally replaced by
    ``value_fn(q32, query_start)``.
    """
    q_lens = np.asarray(q_lens, dtype=np.int64)
    if q_lens.shape != (wl.num_seqs,):
        raise ValueError("one query length per sequence")
    if (q_lens < 0).any() or (q_lens > wl.context_lens).any():
        raise ValueError("query lengths must lie in [0, context length]")
    query_start = np.zeros(wl.num_seqs + 1, dtype=np.int32)
    query_start[1:] = np.cumsum(q_lens)
    rng = np.random.default_rng(seed)
    q32 = rng.standard_normal((int(query_start[-1]), wl.num_q_heads, wl.head_dim),
                              dtype=np.float32)
    if value_fn is not None:
        q32 = value_fn(q32, query_start)
    return _payload(q32, wl.dtype), query_start
