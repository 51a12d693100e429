"""The native pager driving the kernels through a small serving loop:
prompts that share stems (prefix reuse), decode steps that append tokens,
forks whose shared tail pages are copied on write (with the page export /
import kernels), and frees in a pool small enough to evict.  After every
step the batch is decoded on the GPU through the pager's block tables and
compared with the oracle's attention over each sequence's logical history,
whose K/V are recomputed from the tokens and never read from the pool."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_pa_amd as pa
from tests.gpu_helpers import DEV, TOL, f64_of, say, to_dev
from workloads import bf16_bits_from_f32

pytestmark = pytest.mark.gpu

HQ, HKV, D, P = 16, 4, 128, 16
SCALE = D ** -0.5


def kv_of(prefix):
    """K and V rows ([Hkv][D] bf16 bits each) of the last token of `prefix`:
    a function of the whole prefix, as in a real model, so equal prefixes
    hold equal K/V and may share pages."""
    rng = np.random.default_rng(abs(hash(tuple(prefix))) % (2**63))
    x = rng.standard_normal((2, HKV, D), dtype=np.float32)
    return bf16_bits_from_f32(x[0]), bf16_bits_from_f32(x[1])


class Engine:
    def __init__(self, num_pages, max_pages):
        self.pager = pa.Pager(num_pages, P, max_pages)
        self.k = torch.full((num_pages, HKV, P, D), float("nan"), dtype=torch.bfloat16, device=DEV)
        self.v = torch.full((num_pages, HKV, D, P), float("nan"), dtype=torch.bfloat16, device=DEV)
        self.hist = {}

    def write(self, prefixes, slots):
        if not slots:
            return
        kv = [kv_of(p) for p in prefixes]
        key = to_dev(np.stack([a for a, _ in kv]), "bf16")
        val = to_dev(np.stack([b for _, b in kv]), "bf16")
        pa.pa_reshape_and_cache(key, val, self.k, self.v,
                                torch.tensor(slots, dtype=torch.int64, device=DEV))

    def copy_page(self, src, dst):
        buf = torch.empty((2, 1, HKV * P * D), dtype=torch.bfloat16, device=DEV)
        pa.pa_export_pages(buf, self.k, self.v, torch.tensor([src], dtype=torch.int32, device=DEV))
        pa.pa_import_pages(buf, self.k, self.v, torch.tensor([dst], dtype=torch.int32, device=DEV))

    def add(self, sid, tokens):
        slots, cached = self.pager.add_sequence(sid, tokens)
        self.write([tokens[:t + 1] for t in range(cached, len(tokens))],
                   slots[cached:].tolist())
        self.hist[sid] = list(tokens)
        return cached

    def append(self, sid, token):
        try:
            slot, copy = self.pager.append(sid, token)
        except pa.PagerError as e:  # pool full: preempt the sequence (the call changed nothing)
            assert e.status == pa.pager.OUT_OF_PAGES
            self.free(sid)
            return None
        if copy:
            self.copy_page(*copy)
        self.hist[sid].append(token)
        self.write([list(self.hist[sid])], [slot])
        return copy

    def fork(self, parent, child):
        self.pager.fork(parent, child)
        self.hist[child] = list(self.hist[parent])

    def free(self, sid):
        self.pager.free_sequence(sid)
        del self.hist[sid]

    def check(self, rng):
        sids = sorted(self.hist)
        tables, lens = self.pager.block_tables(sids)
        q32 = rng.standard_normal((len(sids), HQ, D), dtype=np.float32)
        qbits = bf16_bits_from_f32(q32)
        q = to_dev(qbits, "bf16")
        bt = torch.from_numpy(tables).to(DEV)
        cl = torch.from_numpy(lens).to(DEV)
        ref = np.zeros((len(sids), HQ, D))
        q64 = oracle.to_float64(qbits, "bf16")
        for i, sid in enumerate(sids):
            h = self.hist[sid]
            kv = [kv_of(h[:t + 1]) for t in range(len(h))]
            K = oracle.to_float64(np.stack([a for a, _ in kv]), "bf16")
            V = oracle.to_float64(np.stack([b for _, b in kv]), "bf16")
            ref[i] = oracle.attention(q64[i], K, V, SCALE)
        out = torch.empty((len(sids), HQ, D), dtype=torch.bfloat16, device=DEV)
        pa.pa_decode(out, q, self.k, self.v, bt, cl, SCALE)
        n = int(-(-int(lens.max()) // 64))
        po = torch.empty((len(sids), HQ, n, D), dtype=torch.float32, device=DEV)
        pm = torch.empty((len(sids), HQ, n), dtype=torch.float32, device=DEV)
        ps = torch.empty((len(sids), HQ, n), dtype=torch.float32, device=DEV)
        out2 = torch.empty_like(out)
        pa.pa_decode(None, q, self.k, self.v, bt, cl, SCALE, 64, po, pm, ps)
        pa.pa_decode_reduce(out2, po, pm, ps, cl, 64)
        torch.cuda.synchronize()
        for o in (out, out2):
            assert float(np.abs(f64_of(o) - ref).max()) <= TOL["bf16"]


def test_serving_loop_with_prefix_reuse_forks_and_eviction():
    say("[serving loop] pager + cache write + decode + page copies")
    rng = np.random.default_rng(11)
    eng = Engine(num_pages=56, max_pages=40)  # tight: cached pages get evicted
    stems = [rng.integers(0, 1000, size=n).tolist() for n in (96, 160, 40)]
    hits = 0
    next_id = 0
    for r in range(10):
        stem = stems[r % 3]
        tail = rng.integers(0, 1000, size=int(rng.integers(1, 40))).tolist()
        hits += eng.add(next_id, stem[:int(rng.integers(len(stem) // 2, len(stem) + 1))] + tail)
        next_id += 1
    assert hits > 0
    eng.check(rng)
    cows = 0
    for step in range(40):
        live = sorted(eng.hist)
        if step % 7 == 3:
            eng.fork(live[int(rng.integers(len(live)))], next_id)
            next_id += 1
        if step % 9 == 5 and len(live) > 4:
            eng.free(live[int(rng.integers(len(live)))])
        for sid in sorted(eng.hist):
            cows += eng.append(sid, int(rng.integers(0, 1000))) is not None
        if step % 5 == 4:
            eng.check(rng)
    s = eng.pager.stats()
    say(f"    prefix hits {s['prefix_hit_tokens']} tokens, copies {s['cow_copies']}, "
        f"evictions {s['evictions']}")
    assert cows > 0 and s["cow_copies"] == cows and s["evictions"] > 0
    eng.check(rng)
