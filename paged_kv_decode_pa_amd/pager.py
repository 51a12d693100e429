"""Python face of libpa_pager.so (include/pa_pager.h): the host-side owner of
the KV page pool.  Marshalling only; the policy lives in the C++ library."""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

import numpy as np

from . import build as _build

PAGER_LIB_PATH = _build.PAGER_LIB

OK, INVALID_ARGUMENT, OUT_OF_PAGES, UNKNOWN_SEQUENCE, SEQUENCE_EXISTS, SEQUENCE_FULL = range(6)
EVENT_STORED, EVENT_REMOVED = 0, 1
_NAMES = ["PA_PAGER_OK", "PA_PAGER_INVALID_ARGUMENT", "PA_PAGER_OUT_OF_PAGES",
          "PA_PAGER_UNKNOWN_SEQUENCE", "PA_PAGER_SEQUENCE_EXISTS", "PA_PAGER_SEQUENCE_FULL"]


class PagerError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        name = _NAMES[status] if 0 <= status < len(_NAMES) else str(status)
        super().__init__(f"{fn} failed: {name}")


class _Stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "num_pages", "in_use", "cached_free", "empty_free", "registered", "live_sequences",
        "prefix_hit_tokens", "evictions", "cow_copies")]


_lib = None
_P = ctypes.c_void_p
# Host arrays travel as plain addresses (numpy's .ctypes.data): converting
# to typed ctypes pointers costs microseconds per argument.
_I32P = _I64P = _U64P = ctypes.c_void_p


def load(path: str = PAGER_LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_kv_decode_pa_amd.build`")
    lib = ctypes.CDLL(path)
    sig = {
        "pa_pager_create": ([ctypes.c_int64, ctypes.c_int, ctypes.c_int], _P),
        "pa_pager_destroy": ([_P], None),
        "pa_pager_add_sequence": ([_P, ctypes.c_int64, _I32P, ctypes.c_int64, _I64P, _I64P],
                                  ctypes.c_int),
        "pa_pager_append": ([_P, ctypes.c_int64, ctypes.c_int32, _I64P, _I64P, _I64P],
                            ctypes.c_int),
        "pa_pager_append_batch": ([_P, _I64P, _I32P, ctypes.c_int64, _I64P, _I64P, _I64P, _I64P],
                                  ctypes.c_int),
        "pa_pager_fork": ([_P, ctypes.c_int64, ctypes.c_int64], ctypes.c_int),
        "pa_pager_free_sequence": ([_P, ctypes.c_int64], ctypes.c_int),
        "pa_pager_block_tables": ([_P, _I64P, ctypes.c_int64, _I32P, _I32P], ctypes.c_int),
        "pa_pager_get_stats": ([_P, ctypes.POINTER(_Stats)], ctypes.c_int),
        "pa_pager_drain_events": ([_P, _I32P, _I64P, _U64P, ctypes.c_int64, _I64P], ctypes.c_int),
        "pa_pager_page_hash": ([ctypes.c_uint64, _I32P, ctypes.c_int], ctypes.c_uint64),
        "pa_pager_prefix_groups": ([_I32P, _I32P, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                    _I32P, _I32P, _I32P, _I32P, _I64P, _I64P, _I64P, _I64P],
                                   ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _ptr(a: np.ndarray, ctype=None):
    return a.ctypes.data


def page_hash(parent: int, tokens: Sequence[int]) -> int:
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    return int(load().pa_pager_page_hash(parent, _ptr(t, ctypes.c_int32), len(t)))


def prefix_groups(block_tables, context_lens, pages_per_partition: int) -> dict:
    """Groups of sequences sharing their first pages (host arrays), in the
    form pa_decode_cascade takes; see pa_pager_prefix_groups."""
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    B, max_pages = bt.shape
    start = np.zeros(B + 1, dtype=np.int32)
    seqs = np.zeros(max(B, 1), dtype=np.int32)
    parts = np.zeros(max(B, 1), dtype=np.int32)
    first = np.zeros(max(B, 1), dtype=np.int32)
    ng, mg, mp, ms = (ctypes.c_int64() for _ in range(4))
    st = load().pa_pager_prefix_groups(
        _ptr(bt), _ptr(lens), B, max_pages, int(pages_per_partition), _ptr(start), _ptr(seqs),
        _ptr(parts), _ptr(first), ctypes.byref(ng), ctypes.byref(mg), ctypes.byref(mp),
        ctypes.byref(ms))
    if st != OK:
        raise PagerError("pa_pager_prefix_groups", st)
    n = ng.value
    return {"num_groups": n, "max_group_size": mg.value, "max_group_partitions": mp.value,
            "max_suffix_partitions": ms.value,
            "group_start": start[:n + 1].copy(), "group_seqs": seqs[:start[n]].copy(),
            "group_partitions": parts[:n].copy(), "seq_first_partition": first[:B].copy()}


class Pager:
    """Owner of a pool of `num_pages` pages of `page_size` tokens."""

    def __init__(self, num_pages: int, page_size: int = 16, max_pages_per_seq: int = 512):
        self._lib = load()
        self._h = self._lib.pa_pager_create(num_pages, page_size, max_pages_per_seq)
        if not self._h:
            raise ValueError("bad pager shape")
        self.page_size = page_size
        self.max_pages_per_seq = max_pages_per_seq

    def close(self) -> None:
        if self._h:
            self._lib.pa_pager_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001  (interpreter shutdown)
            pass

    def _check(self, fn: str, status: int) -> None:
        if status != OK:
            raise PagerError(fn, status)

    def add_sequence(self, seq_id: int, tokens: Sequence[int]) -> Tuple[np.ndarray, int]:
        """Slot of every prompt token and how many leading tokens are cached."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        slots = np.empty(len(t), dtype=np.int64)
        cached = ctypes.c_int64(0)
        self._check("pa_pager_add_sequence", self._lib.pa_pager_add_sequence(
            self._h, seq_id, _ptr(t, ctypes.c_int32), len(t), _ptr(slots, ctypes.c_int64),
            ctypes.byref(cached)))
        return slots, cached.value

    def append(self, seq_id: int, token: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Slot of one new token, and the (src, dst) page copy to make first, if any."""
        slot, src, dst = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        self._check("pa_pager_append", self._lib.pa_pager_append(
            self._h, seq_id, token, ctypes.byref(slot), ctypes.byref(src), ctypes.byref(dst)))
        return slot.value, (None if src.value < 0 else (src.value, dst.value))

    def append_batch(self, seq_ids, tokens, out=None):
        """One token for each listed sequence, in order: (slots int64 [n],
        copies as (src, dst) int64 arrays with -1 where there is none).  `out`
        may pass those three arrays to fill (an engine reuses them every
        step).  On a failure raises PagerError with `.done` = appends made."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        toks = np.ascontiguousarray(tokens, dtype=np.int32)
        n = len(ids)
        if len(toks) != n:
            raise ValueError("one token per sequence")
        if out is None:
            slots, src, dst = (np.empty(n, dtype=np.int64) for _ in range(3))
        else:
            slots, src, dst = out
            for a in out:
                if a.dtype != np.int64 or a.shape != (n,) or not a.flags.c_contiguous:
                    raise ValueError("out arrays must be contiguous int64 [n]")
        done = ctypes.c_int64()
        st = self._lib.pa_pager_append_batch(
            self._h, _ptr(ids, ctypes.c_int64), _ptr(toks, ctypes.c_int32), n,
            _ptr(slots, ctypes.c_int64), _ptr(src, ctypes.c_int64), _ptr(dst, ctypes.c_int64),
            ctypes.byref(done))
        if st != OK:
            err = PagerError("pa_pager_append_batch", st)
            err.done = done.value
            raise err
        return slots, (src, dst)

    def fork(self, parent: int, child: int) -> None:
        self._check("pa_pager_fork", self._lib.pa_pager_fork(self._h, parent, child))

    def free_sequence(self, seq_id: int) -> None:
        self._check("pa_pager_free_sequence", self._lib.pa_pager_free_sequence(self._h, seq_id))

    def block_tables(self, seq_ids: Sequence[int], out=None) -> Tuple[np.ndarray, np.ndarray]:
        """int32 [n][max_pages_per_seq] (padded with -1) and int32 [n]; `out`
        may pass the (tables, lens) arrays to fill."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = len(ids)
        if out is None:
            tables = np.empty((n, self.max_pages_per_seq), dtype=np.int32)
            lens = np.empty(n, dtype=np.int32)
        else:
            tables, lens = out
            if (tables.dtype != np.int32 or tables.shape != (n, self.max_pages_per_seq) or
                    lens.dtype != np.int32 or lens.shape != (n,) or
                    not (tables.flags.c_contiguous and lens.flags.c_contiguous)):
                raise ValueError("out arrays must be contiguous int32 [n][max_pages], [n]")
        self._check("pa_pager_block_tables", self._lib.pa_pager_block_tables(
            self._h, _ptr(ids, ctypes.c_int64), len(ids), _ptr(tables, ctypes.c_int32),
            _ptr(lens, ctypes.c_int32)))
        return tables, lens

    def stats(self) -> dict:
        s = _Stats()
        self._check("pa_pager_get_stats", self._lib.pa_pager_get_stats(self._h, ctypes.byref(s)))
        return {name: getattr(s, name) for name, _ in _Stats._fields_}

    def drain_events(self, capacity: int = 4096) -> List[Tuple[int, int, int]]:
        """Pending (kind, page, hash) events, oldest first."""
        out: List[Tuple[int, int, int]] = []
        kinds = np.empty(capacity, dtype=np.int32)
        pages = np.empty(capacity, dtype=np.int64)
        hashes = np.empty(capacity, dtype=np.uint64)
        while True:
            n = ctypes.c_int64()
            self._check("pa_pager_drain_events", self._lib.pa_pager_drain_events(
                self._h, _ptr(kinds, ctypes.c_int32), _ptr(pages, ctypes.c_int64),
                _ptr(hashes, ctypes.c_uint64), capacity, ctypes.byref(n)))
            out += [(int(kinds[i]), int(pages[i]), int(hashes[i])) for i in range(n.value)]
            if n.value < capacity:
                return out
