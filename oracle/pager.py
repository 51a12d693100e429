"""Plain model of the page pool's ownership policy — TEST INFRASTRUCTURE ONLY
(same rules as the rest of ``oracle/``: only ``tests/``, ``__graft_entry__``'s
smoke run and ``bench.py``'s cpu_baseline leg may use it; it shares nothing
with the native pager).

The pages ask for a fixed pool of fixed-size pages (llm-d router blog post,
engine metric spec; vLLM EngineCoreClient page, "Archivos clave"), reuse of
a cached prompt prefix with allocation and eviction events (llm-d blog post,
prefix-cache scorer and precise KV-cache producer sections), and one native
owner of the pages under a single-writer contract (TensorRT Edge-LLM,
"Request Lifecycle" and "Extension Rules").  They fix no policy; this model
states the one the native pager implements, step by step, with plain Python
containers and no hashing: a full page is keyed by the exact tuple of every
token from the start of its sequence through its last token.

    free pages: "empty" (nothing registered; taken lowest id first) or
                "cached" (a registered full page; evicted least recently
                released first, which unregisters it)
    add:        reuse the longest run of registered full pages matching the
                prompt from the start; allocate the rest; register the new
                full pages (unless the key is taken); fail with no change
                when the pool cannot hold the rest
    append:     a token that opens a page allocates one; a token written to
                a tail page that another sequence also holds first moves to
                a fresh page (copy-on-write: reported as (src, dst)); a page
                that becomes full is registered
    fork:       the child holds every page of the parent
    free:       pages released from the last to the first
"""
from __future__ import annotations

OK, INVALID, OUT_OF_PAGES, UNKNOWN, EXISTS, FULL = 0, 1, 2, 3, 4, 5
STORED, REMOVED = 0, 1


class PagerModel:
    def __init__(self, num_pages, page_size, max_pages_per_seq):
        self.P = page_size
        self.max_pages = max_pages_per_seq
        self.num_pages = num_pages
        self.ref = [0] * num_pages
        self.key_of = [None] * num_pages   # registered key of a page, or None
        self.page_of = {}                  # key -> page
        self.released_at = {}              # cached page -> release tick
        self.tick = 0
        self.seqs = {}                     # id -> {"pages": [...], "tokens": [...]}
        self.events = []                   # (kind, page)
        self.hits = self.evictions = self.cows = 0

    # -- free-page bookkeeping
    def _empty(self):
        return [p for p in range(self.num_pages) if self.ref[p] == 0 and self.key_of[p] is None]

    def _cached(self):
        return sorted((t, p) for p, t in self.released_at.items())

    def _allocate(self):
        empty = self._empty()
        if empty:
            p = empty[0]
        else:
            cached = self._cached()
            if not cached:
                return None
            p = cached[0][1]
            del self.released_at[p]
            del self.page_of[self.key_of[p]]
            self.key_of[p] = None
            self.events.append((REMOVED, p))
            self.evictions += 1
        self.ref[p] = 1
        return p

    def _take(self, p):
        if self.ref[p] == 0:
            del self.released_at[p]
        self.ref[p] += 1

    def _release(self, p):
        self.ref[p] -= 1
        if self.ref[p] == 0 and self.key_of[p] is not None:
            self.tick += 1
            self.released_at[p] = self.tick

    def _register(self, p, key):
        if key in self.page_of:
            return
        self.page_of[key] = p
        self.key_of[p] = key
        self.events.append((STORED, p))

    # -- operations
    def add_sequence(self, sid, tokens):
        P = self.P
        n = len(tokens)
        if sid in self.seqs:
            return EXISTS, None, None
        npages = -(-n // P)
        if npages > self.max_pages:
            return FULL, None, None
        reuse = []
        for k in range(n // P):
            p = self.page_of.get(tuple(tokens[:(k + 1) * P]))
            if p is None:
                break
            reuse.append(p)
        free_now = len(self._empty()) + len(self.released_at)
        free_now -= sum(1 for p in reuse if self.ref[p] == 0)
        if npages - len(reuse) > free_now:
            return OUT_OF_PAGES, None, None
        pages = []
        for p in reuse:
            self._take(p)
            pages.append(p)
        for _ in range(len(reuse), npages):
            pages.append(self._allocate())
        for k in range(len(reuse), n // P):
            self._register(pages[k], tuple(tokens[:(k + 1) * P]))
        self.seqs[sid] = {"pages": pages, "tokens": list(tokens)}
        self.hits += len(reuse) * P
        slots = [pages[t // P] * P + t % P for t in range(n)]
        return OK, slots, len(reuse) * P

    def append(self, sid, token):
        P = self.P
        if sid not in self.seqs:
            return UNKNOWN, None, None
        s = self.seqs[sid]
        off = len(s["tokens"]) % P
        copy = None
        if off == 0:
            if len(s["pages"]) >= self.max_pages:
                return FULL, None, None
            p = self._allocate()
            if p is None:
                return OUT_OF_PAGES, None, None
            s["pages"].append(p)
        elif self.ref[s["pages"][-1]] > 1:
            tail = s["pages"][-1]
            p = self._allocate()
            if p is None:
                return OUT_OF_PAGES, None, None
            self._release(tail)
            s["pages"][-1] = p
            copy = (tail, p)
            self.cows += 1
        page = s["pages"][-1]
        s["tokens"].append(token)
        if len(s["tokens"]) % P == 0:
            self._register(page, tuple(s["tokens"]))
        return OK, page * P + off, copy

    def fork(self, parent, child):
        if parent not in self.seqs:
            return UNKNOWN
        if child in self.seqs:
            return EXISTS
        src = self.seqs[parent]
        for p in src["pages"]:
            self.ref[p] += 1
        self.seqs[child] = {"pages": list(src["pages"]), "tokens": list(src["tokens"])}
        return OK

    def free_sequence(self, sid):
        if sid not in self.seqs:
            return UNKNOWN
        for p in reversed(self.seqs.pop(sid)["pages"]):
            self._release(p)
        return OK

    def block_tables(self, sids):
        rows, lens = [], []
        for sid in sids:
            s = self.seqs[sid]
            rows.append(s["pages"] + [-1] * (self.max_pages - len(s["pages"])))
            lens.append(len(s["tokens"]))
        return rows, lens

    def stats(self):
        cached = len(self.released_at)
        empty = len(self._empty())
        return {"num_pages": self.num_pages, "in_use": self.num_pages - cached - empty,
                "cached_free": cached, "empty_free": empty, "registered": len(self.page_of),
                "live_sequences": len(self.seqs), "prefix_hit_tokens": self.hits,
                "evictions": self.evictions, "cow_copies": self.cows}

    def drain_events(self):
        ev, self.events = self.events, []
        return ev
