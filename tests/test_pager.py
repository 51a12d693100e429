"""The native page pool owner (libpa_pager.so) against the plain policy model
in ``oracle.pager``, on the CPU: every returned slot, cached-prefix length,
copy-on-write move, block table, statistic and event must agree, over
scripted cases and seeded random operation streams.  An emulated pool that
stores token ids in slots checks the property the kernels rely on: every
live sequence reads back exactly its own token history, and no slot is
written while its page is shared or registered."""
import numpy as np
import pytest

import paged_kv_decode_pa_amd as pa
from oracle.pager import PagerModel
from paged_kv_decode_pa_amd import pager as pgr

M64 = (1 << 64) - 1


def splitmix_step(z):
    """One output of the splitmix64 generator from state z (Steele, Lea and
    Flood 2014; Vigna's published constants), written from its definition."""
    z = (z + 0x9E3779B97F4A7C15) & M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def test_page_hash_is_the_documented_splitmix_chain():
    # published first outputs of splitmix64 seeded with 0
    assert splitmix_step(0) == 0xE220A8397B1DCDAF
    assert splitmix_step(0x9E3779B97F4A7C15) == 0x6E789E6AA1B965F4
    rng = np.random.default_rng(5)
    for _ in range(50):
        parent = int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2))
        toks = rng.integers(-2**31, 2**31, size=int(rng.integers(1, 40))).astype(np.int32)
        h = splitmix_step(parent ^ 0x5A17C0DE)
        for t in toks.tolist():
            h = splitmix_step(h ^ (t & 0xFFFFFFFF))
        assert pa.page_hash(parent, toks) == h


class Both:
    """Drive the native pager and the model with the same calls and compare."""

    def __init__(self, num_pages, P, max_pages):
        self.n = pa.Pager(num_pages, P, max_pages)
        self.m = PagerModel(num_pages, P, max_pages)
        self.P = P
        self.pool = np.full(num_pages * P, -1, dtype=np.int64)  # emulated K/V: token per slot
        self.history = {}

    def _status(self, fn, *a):
        try:
            return 0, fn(*a)
        except pgr.PagerError as e:
            return e.status, None

    def _written_ok(self, slot):
        page = slot // self.P
        assert self.m.ref[page] == 1, "write to a shared page"

    def add(self, sid, tokens):
        st, res = self._status(self.n.add_sequence, sid, tokens)
        mst, mslots, mcached = self.m.add_sequence(sid, list(tokens))
        assert st == mst
        if st:
            return st
        slots, cached = res
        assert cached == mcached and slots.tolist() == mslots
        for t in range(cached):  # reused: the content must already be there
            assert self.pool[slots[t]] == tokens[t]
        for t in range(cached, len(tokens)):
            self._written_ok(int(slots[t]))
            self.pool[slots[t]] = tokens[t]
        self.history[sid] = list(tokens)
        return 0

    def append(self, sid, token):
        st, res = self._status(self.n.append, sid, token)
        mst, mslot, mcopy = self.m.append(sid, token)
        assert st == mst
        if st:
            return st
        slot, copy = res
        assert slot == mslot and copy == mcopy
        if copy:
            src, dst = copy
            self.pool[dst * self.P:(dst + 1) * self.P] = self.pool[src * self.P:(src + 1) * self.P]
        self._written_ok(slot)
        self.pool[slot] = token
        self.history[sid].append(token)
        return 0

    def fork(self, parent, child):
        st, _ = self._status(self.n.fork, parent, child)
        assert st == self.m.fork(parent, child)
        if st == 0:
            self.history[child] = list(self.history[parent])
        return st

    def free(self, sid):
        st, _ = self._status(self.n.free_sequence, sid)
        assert st == self.m.free_sequence(sid)
        if st == 0:
            del self.history[sid]
        return st

    def check(self):
        assert self.n.stats() == self.m.stats()
        ev = self.n.drain_events()
        assert [(k, p) for k, p, _ in ev] == self.m.drain_events()
        sids = sorted(self.history)
        if not sids:
            return
        tables, lens = self.n.block_tables(sids)
        mrows, mlens = self.m.block_tables(sids)
        assert tables.tolist() == mrows and lens.tolist() == mlens
        for i, sid in enumerate(sids):
            L = int(lens[i])
            assert L == len(self.history[sid])
            got = [int(self.pool[tables[i, t // self.P] * self.P + t % self.P]) for t in range(L)]
            assert got == self.history[sid], sid


def test_prefix_reuse_fork_and_copy_on_write():
    b = Both(num_pages=10, P=4, max_pages=6)
    assert b.add(1, [1, 2, 3, 4, 5, 6, 7, 8, 9]) == 0           # pages 0 1 2 (2 partial)
    assert b.add(2, [1, 2, 3, 4, 5, 6, 7, 8, 20, 21]) == 0      # reuses 0 1
    assert b.n.stats()["prefix_hit_tokens"] == 8
    b.check()
    assert b.fork(1, 3) == 0
    assert b.append(3, 30) == 0                                  # tail page 2 shared: moves
    assert b.n.stats()["cow_copies"] == 1
    assert b.append(1, 31) == 0                                  # page 2 now private: in place
    assert b.n.stats()["cow_copies"] == 1
    b.check()
    for t in range(5):
        assert b.append(3, 40 + t) == 0
    b.check()


def test_lru_eviction_order_and_clean_failure():
    b = Both(num_pages=6, P=4, max_pages=6)
    assert b.add(1, list(range(12))) == 0                       # 3 full registered pages
    assert b.add(2, [100 + i for i in range(8)]) == 0           # 2 more
    assert b.free(1) == 0                                       # cached, released 2, 1, 0
    b.check()
    before = b.n.stats()
    assert b.add(3, [200 + i for i in range(20)]) == pgr.OUT_OF_PAGES  # 5 needed, 4 free
    assert b.n.stats() == before and b.n.drain_events() == [] and b.m.drain_events() == []
    assert b.add(4, [300 + i for i in range(8)]) == 0           # empty page 5, then evicts 2
    b.check()
    assert b.add(5, list(range(8)) + [7]) == pgr.OUT_OF_PAGES  # reuses 0 1, no page left
    assert b.add(5, list(range(8))) == 0                        # pages 0 1 still cached: reused
    assert b.n.stats()["prefix_hit_tokens"] == 8
    b.check()
    assert b.free(2) == 0                                       # cached 4, 3 (in that order)
    assert b.add(6, [1, 2, 3]) == 0                             # evicts page 4
    assert b.n.stats()["evictions"] == 2
    b.check()


def test_errors():
    b = Both(num_pages=4, P=4, max_pages=2)
    assert b.add(1, list(range(12))) == pgr.SEQUENCE_FULL
    assert b.add(1, list(range(8))) == 0
    assert b.add(1, [1]) == pgr.SEQUENCE_EXISTS
    assert b.append(1, 5) == pgr.SEQUENCE_FULL                 # would open a third page
    assert b.append(9, 5) == pgr.UNKNOWN_SEQUENCE
    assert b.fork(9, 10) == pgr.UNKNOWN_SEQUENCE
    assert b.fork(1, 1) == pgr.SEQUENCE_EXISTS
    assert b.free(9) == pgr.UNKNOWN_SEQUENCE
    assert b.add(2, []) == 0                                    # empty prompt: no pages
    assert b.append(2, 3) == 0
    b.check()
    with pytest.raises(ValueError):
        pa.Pager(0, 16, 4)
    with pytest.raises(ValueError):
        pa.Pager(8, 65, 4)


@pytest.mark.parametrize("seed", range(12))
def test_random_operation_streams(seed):
    """Prompts drawn from a few shared stems (so prefixes repeat), appends,
    forks and frees at random, in a pool small enough to evict and to run
    out; the model and the native pager agree after every operation."""
    rng = np.random.default_rng(seed)
    P = int(rng.choice([2, 4, 16]))
    b = Both(num_pages=int(rng.integers(6, 40)), P=P, max_pages=int(rng.integers(3, 12)))
    stems = [rng.integers(0, 50, size=int(rng.integers(0, 5 * P))).tolist() for _ in range(4)]
    next_id = 0
    for _ in range(250):
        live = sorted(b.history)
        op = rng.random()
        if op < 0.3 or not live:
            stem = stems[int(rng.integers(len(stems)))]
            cut = int(rng.integers(0, len(stem) + 1))
            tail = rng.integers(0, 50, size=int(rng.integers(0, 3 * P))).tolist()
            b.add(next_id, stem[:cut] + tail)
            next_id += 1
        elif op < 0.7:
            b.append(live[int(rng.integers(len(live)))], int(rng.integers(0, 50)))
        elif op < 0.8:
            b.fork(live[int(rng.integers(len(live)))], next_id)
            next_id += 1
        else:
            b.free(live[int(rng.integers(len(live)))])
        b.check()


def test_library_exports_every_declared_symbol():
    import os
    import re
    header = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "include", "pa_pager.h")
    names = set(re.findall(r"^\s*(?:int|void|uint64_t|pa_pager\*)\s+(pa_pager_\w+)\s*\(",
                           open(header).read(), re.M))
    assert {"pa_pager_create", "pa_pager_add_sequence", "pa_pager_append", "pa_pager_fork",
            "pa_pager_free_sequence", "pa_pager_block_tables", "pa_pager_drain_events"} <= names
    lib = pgr.load()
    for n in names:
        assert hasattr(lib, n), n


def test_null_and_negative_arguments_are_rejected():
    import ctypes
    lib = pgr.load()
    h = lib.pa_pager_create(8, 16, 4)
    assert h
    try:
        n = ctypes.c_int64()
        toks = (ctypes.c_int32 * 4)(1, 2, 3, 4)
        slots = (ctypes.c_int64 * 4)()
        assert lib.pa_pager_add_sequence(None, 1, toks, 4, slots, ctypes.byref(n)) == pgr.INVALID_ARGUMENT
        assert lib.pa_pager_add_sequence(h, 1, None, 4, slots, ctypes.byref(n)) == pgr.INVALID_ARGUMENT
        assert lib.pa_pager_add_sequence(h, 1, toks, -1, slots, ctypes.byref(n)) == pgr.INVALID_ARGUMENT
        assert lib.pa_pager_add_sequence(h, 1, toks, 4, None, ctypes.byref(n)) == pgr.INVALID_ARGUMENT
        assert lib.pa_pager_append(h, 1, 5, None, ctypes.byref(n), ctypes.byref(n)) == pgr.INVALID_ARGUMENT
        assert lib.pa_pager_block_tables(h, None, 2, None, None) == pgr.INVALID_ARGUMENT
        assert lib.pa_pager_drain_events(h, None, None, None, 4, ctypes.byref(n)) == pgr.INVALID_ARGUMENT
        assert lib.pa_pager_get_stats(h, None) == pgr.INVALID_ARGUMENT
        assert not lib.pa_pager_create(8, 0, 4) and not lib.pa_pager_create(8, 16, 0)
    finally:
        lib.pa_pager_destroy(h)


def test_append_batch_equals_appends_in_order():
    rng = np.random.default_rng(21)
    a = pa.Pager(40, 4, 10)
    m = PagerModel(40, 4, 10)
    for sid in range(6):
        toks = rng.integers(0, 9, size=int(rng.integers(0, 14))).tolist()
        a.add_sequence(sid, toks)
        m.add_sequence(sid, toks)
    a.fork(2, 6)
    m.fork(2, 6)
    for _ in range(12):
        ids = rng.permutation(7)
        toks = rng.integers(0, 9, size=7)
        try:
            slots, (src, dst) = a.append_batch(ids, toks)
            done, status = 7, 0
        except pgr.PagerError as e:
            done, status = e.done, e.status
            slots = src = dst = None
        for i in range(7):
            mst, mslot, mcopy = m.append(int(ids[i]), int(toks[i]))
            if i < done:
                assert mst == 0 and slots is not None
                assert slots[i] == mslot
                assert (None if src[i] < 0 else (src[i], dst[i])) == mcopy
            else:
                assert mst == status
                break
        assert a.stats() == m.stats()
        if status:
            break


def _prefix_groups_by_hand(tables, lens, pp):
    """Plain rendering of the grouping rule: same page in column 0, then the
    longest common run of page ids over every member's pages that lie wholly
    before its last token, in whole partitions; groups of 2+ members."""
    B = len(lens)
    whole = [min(max(int(L) - 1, 0) // 16, tables.shape[1]) for L in lens]
    order, buckets = [], {}
    for b in range(B):
        if whole[b] < pp:
            continue
        key = int(tables[b, 0])
        if key not in buckets:
            buckets[key] = []
            order.append(key)
        buckets[key].append(b)
    groups, first = [], [0] * B
    for key in order:
        m = buckets[key]
        if len(m) < 2:
            continue
        lcp = whole[m[0]]
        for b in m[1:]:
            l = 0
            while l < min(lcp, whole[b]) and tables[b, l] == tables[m[0], l]:
                l += 1
            lcp = l
        if lcp // pp >= 1:
            groups.append((m, lcp // pp))
            for b in m:
                first[b] = lcp // pp
    return groups, first


@pytest.mark.parametrize("seed", range(8))
def test_prefix_groups_match_the_rule(seed):
    rng = np.random.default_rng(seed)
    B, max_pages, pp = int(rng.integers(1, 40)), 40, int(rng.choice([1, 2, 4]))
    stems = [rng.permutation(1000)[:max_pages] for _ in range(4)]
    tables = np.full((B, max_pages), -1, dtype=np.int32)
    lens = rng.integers(0, max_pages * 16, size=B).astype(np.int32)
    fresh = 2000
    for b in range(B):
        n = -(-int(lens[b]) // 16)
        s = stems[int(rng.integers(4))]
        cut = int(rng.integers(0, n + 1))
        tables[b, :cut] = s[:cut]
        tables[b, cut:n] = np.arange(fresh, fresh + n - cut)
        fresh += n - cut
    got = pa.prefix_groups(tables, lens, pp)
    groups, first = _prefix_groups_by_hand(tables, lens, pp)
    assert got["num_groups"] == len(groups)
    starts = got["group_start"].tolist()
    for g, (members, parts) in enumerate(groups):
        assert got["group_seqs"][starts[g]:starts[g + 1]].tolist() == members
        assert int(got["group_partitions"][g]) == parts
    assert got["seq_first_partition"].tolist() == first
    assert got["max_group_size"] == max([len(m) for m, _ in groups], default=0)
    assert got["max_group_partitions"] == max([p for _, p in groups], default=0)
    parts = [-(-min(-(-int(L) // 16), max_pages) // pp) for L in lens]
    assert got["max_suffix_partitions"] == max(parts[b] - first[b] for b in range(B))
