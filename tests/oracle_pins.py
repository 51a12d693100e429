"""Checks that pin the fp64 oracle to something other than itself.

Each ``check_*`` takes the oracle module and raises AssertionError on a
mismatch.  ``test_oracle_pins.py`` runs them against the real oracle;
``test_oracle_mutants.py`` plants plausible mistakes in the oracle and asserts
that some check fails for each, so the pins are known to bite.

The independent references used here:
  * the pool layout written out as flat element offsets (not numpy reshapes);
  * pure-Python scalar loops with ``math.exp`` / ``math.fsum`` (brute force);
  * torch's ``scaled_dot_product_attention`` in float64 on the CPU;
  * closed forms: a one-token context returns V, constant V returns the
    constant, a zero query returns the mean of V, a dominant key returns its V,
    and the hand-derived cases in ``tests/golden/closed_form_decode.json``;
  * invariances of the definition: physical page placement and prefix sharing
    do not change the result; split-KV partials merged by log-sum-exp equal
    the unsplit result.
For multi-token causal queries (``chunk_attention``): one token per sequence
is exactly ``decode``; a causal pure-Python brute force over flat offsets;
torch's attention with an explicit causal offset mask; and causality itself
(changing a later token's K/V leaves earlier rows bit for bit unchanged).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from workloads import make_chunk_queries, make_custom_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_decode.json")


# ---------------------------------------------------------------- helpers
def k_offset(page, head, slot, dim, Hkv, P, D):
    return ((page * Hkv + head) * P + slot) * D + dim


def v_offset(page, head, slot, dim, Hkv, P, D):
    return ((page * Hkv + head) * D + dim) * P + slot


def nan_pools(num_pages, Hkv, P, D, dtype):
    if dtype == "f32":
        k = np.full((num_pages, Hkv, P, D), np.nan, dtype=np.float32)
        v = np.full((num_pages, Hkv, D, P), np.nan, dtype=np.float32)
    else:
        k = np.full((num_pages, Hkv, P, D), 0x7FC0, dtype=np.uint16)
        v = np.full((num_pages, Hkv, D, P), 0x7FC0, dtype=np.uint16)
    return k, v


def fill_pools(orc, wl):
    """Oracle-side pool for a workload: NaN everywhere, then every cached and
    appended token written through the oracle's cache write."""
    k, v = nan_pools(wl.num_pages, wl.num_kv_heads, wl.page_size, wl.head_dim, wl.dtype)
    k, v = orc.cache_write(k, v, wl.prefill_key, wl.prefill_value, wl.prefill_slots, wl.page_size)
    k, v = orc.cache_write(k, v, wl.new_key, wl.new_value, wl.new_slots, wl.page_size)
    return k, v


def oracle_decode(orc, wl):
    k, v = fill_pools(orc, wl)
    return orc.decode(wl.query, k, v, wl.block_tables, wl.context_lens, wl.scale,
                      wl.page_size, wl.dtype)


def brute_force_decode(wl, kpool, vpool):
    """Pure-Python reference that reads the pools through flat offsets."""
    Hq, Hkv, D, P = wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.page_size
    group = Hq // Hkv
    kflat = widen(kpool, wl.dtype).reshape(-1).tolist()
    vflat = widen(vpool, wl.dtype).reshape(-1).tolist()
    q = widen(wl.query, wl.dtype)
    out = np.zeros((wl.num_seqs, Hq, D))
    for b in range(wl.num_seqs):
        L = int(wl.context_lens[b])
        if L == 0:
            continue
        for h in range(Hq):
            g = h // group
            qh = q[b, h].tolist()
            scores = []
            for t in range(L):
                page = int(wl.block_tables[b, t // P])
                acc = math.fsum(qh[d] * kflat[k_offset(page, g, t % P, d, Hkv, P, D)]
                                for d in range(D))
                scores.append(wl.scale * acc)
            mx = max(scores)
            w = [math.exp(s - mx) for s in scores]
            z = math.fsum(w)
            for d in range(D):
                num = math.fsum(w[t] * vflat[v_offset(int(wl.block_tables[b, t // P]), g,
                                                      t % P, d, Hkv, P, D)]
                                for t in range(L))
                out[b, h, d] = num / z
    return out


def widen(a, dtype):
    """Independent widening for the checks: bf16 bits via float32 bit assembly."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    u = np.asarray(a, dtype=np.uint16)
    return (u.astype(np.uint32) * np.uint32(65536)).view(np.float32).astype(np.float64)


def tiny(lengths, Hq=4, Hkv=2, D=8, dtype="f32", seed=0, **kw):
    return make_custom_workload(lengths, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                                dtype=dtype, seed=seed, **kw)


def brute_force_chunk(wl, kpool, vpool, query, query_start):
    """Pure-Python causal reference: query row i of sequence b (position
    L - q_len + i) over that sequence's tokens 0..position, via flat offsets."""
    Hq, Hkv, D, P = wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.page_size
    group = Hq // Hkv
    kflat = widen(kpool, wl.dtype).reshape(-1).tolist()
    vflat = widen(vpool, wl.dtype).reshape(-1).tolist()
    q = widen(query, wl.dtype)
    out = np.zeros((q.shape[0], Hq, D))
    for b in range(wl.num_seqs):
        lo, hi = int(query_start[b]), int(query_start[b + 1])
        L = int(wl.context_lens[b])
        for r in range(lo, hi):
            pos = L - (hi - lo) + (r - lo)
            for h in range(Hq):
                g = h // group
                qh = q[r, h].tolist()
                scores = []
                for t in range(pos + 1):
                    page = int(wl.block_tables[b, t // P])
                    acc = math.fsum(qh[d] * kflat[k_offset(page, g, t % P, d, Hkv, P, D)]
                                    for d in range(D))
                    scores.append(wl.scale * acc)
                mx = max(scores)
                w = [math.exp(x - mx) for x in scores]
                z = math.fsum(w)
                for d in range(D):
                    num = math.fsum(w[t] * vflat[v_offset(int(wl.block_tables[b, t // P]), g,
                                                          t % P, d, Hkv, P, D)]
                                    for t in range(pos + 1))
                    out[r, h, d] = num / z
    return out


# ---------------------------------------------------------------- checks
def check_bf16_widening(orc):
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0xFF80, 0x0001, 0x3F81, 0x0000, 0x8000,
                     0x4049], dtype=np.uint16)
    want = [1.0, -2.0, math.inf, -math.inf, 2.0 ** -133, 1.0 + 2.0 ** -7, 0.0, -0.0,
            3.140625]
    got = orc.bf16_bits_to_float64(bits)
    for g, w in zip(got.tolist(), want):
        assert g == w, (g, w)
    assert math.copysign(1.0, got[7]) == -1.0


def check_cache_write_layout(orc):
    rng = np.random.default_rng(7)
    num_pages, Hkv, P, D = 5, 3, 16, 4
    T = 23
    slots = rng.choice(num_pages * P, size=T, replace=False).astype(np.int64)
    slots[[3, 11]] = -1
    key = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    val = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    k0, v0 = nan_pools(num_pages, Hkv, P, D, "f32")
    k, v = orc.cache_write(k0, v0, key, val, slots, P)
    assert k.shape == k0.shape and v.shape == v0.shape
    assert np.isnan(k0).all() and np.isnan(v0).all(), "inputs must not be modified"
    kf, vf = k.reshape(-1), v.reshape(-1)
    written = 0
    for t in range(T):
        s = int(slots[t])
        if s < 0:
            continue
        written += 1
        page, slot = s // P, s % P
        for h in range(Hkv):
            for d in range(D):
                assert kf[k_offset(page, h, slot, d, Hkv, P, D)] == key[t, h, d]
                assert vf[v_offset(page, h, slot, d, Hkv, P, D)] == val[t, h, d]
    assert int(np.count_nonzero(~np.isnan(kf))) == written * Hkv * D
    assert int(np.count_nonzero(~np.isnan(vf))) == written * Hkv * D


def check_gather_roundtrip(orc):
    wl = tiny([37, 16, 5], Hq=2, Hkv=2, D=3, seed=3)
    k, v = fill_pools(orc, wl)
    # Rebuild each sequence's logical tokens from the workload's slot lists.
    by_slot_k, by_slot_v = {}, {}
    for keys, vals, slots in ((wl.prefill_key, wl.prefill_value, wl.prefill_slots),
                              (wl.new_key, wl.new_value, wl.new_slots)):
        for i, s in enumerate(slots.tolist()):
            by_slot_k[s] = keys[i]
            by_slot_v[s] = vals[i]
    for b in range(wl.num_seqs):
        L = int(wl.context_lens[b])
        K, V = orc.gather_sequence(k, v, wl.block_tables[b], L, wl.page_size)
        assert K.shape == (L, 2, 3) and V.shape == (L, 2, 3)
        for t in range(L):
            s = int(wl.block_tables[b, t // 16]) * 16 + t % 16
            assert np.array_equal(K[t], by_slot_k[s])
            assert np.array_equal(V[t], by_slot_v[s])


def check_single_token_returns_v(orc):
    for dtype in ("f32", "bf16"):
        wl = tiny([1, 1, 1], Hq=6, Hkv=3, D=16, dtype=dtype, seed=11)
        out = oracle_decode(orc, wl)
        v = widen(wl.new_value, dtype)               # the only token is the appended one
        group = wl.num_q_heads // wl.num_kv_heads
        for b in range(wl.num_seqs):
            for h in range(wl.num_q_heads):
                assert np.array_equal(out[b, h], v[b, h // group]), (dtype, b, h)


def check_constant_v(orc):
    consts = np.array([0.75, -1.5], dtype=np.float32)

    def fn(q, k, v, owners, lengths):
        v[:] = consts[None, :, None]
        return q, k, v

    wl = tiny([1, 40, 16, 33], Hq=4, Hkv=2, D=8, seed=5, value_fn=fn)
    out = oracle_decode(orc, wl)
    for h in range(4):
        assert np.allclose(out[:, h, :], consts[h // 2], rtol=1e-15, atol=0)


def check_zero_query_mean(orc):
    def fn(q, k, v, owners, lengths):
        q[:] = 0.0
        return q, k, v

    wl = tiny([3, 20, 47], Hq=4, Hkv=2, D=5, seed=9, value_fn=fn)
    kp, vp = fill_pools(orc, wl)
    out = orc.decode(wl.query, kp, vp, wl.block_tables, wl.context_lens, wl.scale,
                     wl.page_size, wl.dtype)
    vf = widen(vp, "f32")
    for b in range(wl.num_seqs):
        L = int(wl.context_lens[b])
        for h in range(4):
            col = [[vf[int(wl.block_tables[b, t // 16]), h // 2, d, t % 16] for t in range(L)]
                   for d in range(5)]
            mean = np.array([math.fsum(c) / L for c in col])
            assert np.allclose(out[b, h], mean, rtol=0, atol=1e-12)


def check_equal_keys_mean(orc):
    def fn(q, k, v, owners, lengths):
        k[:] = k[0]
        return q, k, v

    wl = tiny([9, 30], Hq=2, Hkv=1, D=6, seed=21, value_fn=fn)
    out = oracle_decode(orc, wl)
    bf = brute_force_decode(wl, *fill_pools(orc, wl))
    assert np.allclose(out, bf, rtol=0, atol=1e-12)
    # all scores equal: the output is the plain mean of the context's V rows
    kp, vp = fill_pools(orc, wl)
    for b in range(2):
        L = int(wl.context_lens[b])
        rows = np.array([[vp[int(wl.block_tables[b, t // 16]), 0, d, t % 16] for d in range(6)]
                         for t in range(L)], dtype=np.float64)
        assert np.allclose(out[b, 0], rows.mean(axis=0), rtol=0, atol=1e-12)


def check_needle(orc):
    """A key aligned with the query and 40x larger than the rest dominates."""
    def fn(q, k, v, owners, lengths):
        q[:] = 0.0
        q[:, :, 0] = 1.0
        k[:] = 0.0
        for i, (key, pos) in enumerate(owners):
            if pos == 17:
                k[i, :, 0] = 40.0 * math.sqrt(8)
        return q, k, v

    wl = tiny([18, 35], Hq=2, Hkv=1, D=8, seed=2, value_fn=fn)
    kp, vp = fill_pools(orc, wl)
    out = orc.decode(wl.query, kp, vp, wl.block_tables, wl.context_lens, wl.scale,
                     wl.page_size, wl.dtype)
    for b in range(2):
        page = int(wl.block_tables[b, 1])
        needle_v = vp[page, 0, :, 1].astype(np.float64)
        assert np.allclose(out[b, 0], needle_v, rtol=0, atol=1e-6)


def check_brute_force(orc):
    cases = [
        dict(lengths=[1, 2, 16], Hq=3, Hkv=3, D=4),
        dict(lengths=[17, 31], Hq=4, Hkv=2, D=8),
        dict(lengths=[40, 15, 33], Hq=6, Hkv=2, D=5),
        dict(lengths=[32], Hq=2, Hkv=1, D=7, dtype="bf16"),
    ]
    for i, c in enumerate(cases):
        wl = tiny(seed=100 + i, **c)
        kp, vp = fill_pools(orc, wl)
        got = orc.decode(wl.query, kp, vp, wl.block_tables, wl.context_lens, wl.scale,
                         wl.page_size, wl.dtype)
        want = brute_force_decode(wl, kp, vp)
        assert np.allclose(got, want, rtol=0, atol=1e-12), (i, np.abs(got - want).max())


def check_sharp_scores(orc):
    """Scores in the thousands: float64 exp overflows (past ~709) unless the
    maximum is subtracted first."""
    def fn(q, k, v, owners, lengths):
        return q * 600.0, k, v

    wl = tiny([29, 50], Hq=4, Hkv=2, D=16, seed=31, value_fn=fn)
    kp, vp = fill_pools(orc, wl)
    got = orc.decode(wl.query, kp, vp, wl.block_tables, wl.context_lens, wl.scale,
                     wl.page_size, wl.dtype)
    assert np.isfinite(got).all()
    want = brute_force_decode(wl, kp, vp)
    assert np.allclose(got, want, rtol=0, atol=1e-12)


def check_torch_sdpa(orc):
    import torch

    wl = tiny([300, 77, 129, 16], Hq=8, Hkv=2, D=32, seed=41)
    kp, vp = fill_pools(orc, wl)
    got = orc.decode(wl.query, kp, vp, wl.block_tables, wl.context_lens, wl.scale,
                     wl.page_size, wl.dtype)
    q = widen(wl.query, "f32")
    group = 4
    for b in range(wl.num_seqs):
        L = int(wl.context_lens[b])
        # contiguous K/V rebuilt from flat offsets, kv heads repeated per group
        K = np.zeros((8, L, 32))
        V = np.zeros((8, L, 32))
        for t in range(L):
            page, slot = int(wl.block_tables[b, t // 16]), t % 16
            for h in range(8):
                K[h, t] = kp[page, h // group, slot, :]
                V[h, t] = vp[page, h // group, :, slot]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[b][:, None, :]), torch.from_numpy(K), torch.from_numpy(V),
            scale=wl.scale)[:, 0, :].numpy()
        assert np.allclose(got[b], ref, rtol=0, atol=1e-12), np.abs(got[b] - ref).max()


def check_permutation_invariance(orc):
    base = tiny([5, 70, 33, 16, 1], Hq=4, Hkv=2, D=8, seed=50)
    moved = tiny([5, 70, 33, 16, 1], Hq=4, Hkv=2, D=8, seed=50, placement_seed=999)
    assert not np.array_equal(base.block_tables, moved.block_tables)
    assert np.array_equal(oracle_decode(orc, base), oracle_decode(orc, moved))


def check_shared_vs_unshared(orc):
    kw = dict(Hq=4, Hkv=2, D=8, seed=60, group_size=3, prefix_tokens=32)
    lens = [40, 33, 64, 50, 48, 35]
    shared = tiny(lens, **kw)
    unshared = tiny(lens, share_prefix=False, **kw)
    assert shared.unique_pages < unshared.unique_pages
    # the group's first two logical pages are one physical page in every sharer
    assert (shared.block_tables[0, :2] == shared.block_tables[1, :2]).all()
    assert np.array_equal(oracle_decode(orc, shared), oracle_decode(orc, unshared))


def check_partitions(orc):
    rng = np.random.default_rng(70)
    for L, ps in ((100, 16), (100, 32), (64, 64), (300, 48), (17, 512)):
        q = rng.standard_normal((4, 8))
        K = rng.standard_normal((L, 2, 8))
        V = rng.standard_normal((L, 2, 8))
        full = orc.attention(q, K, V, 0.3)
        m, lsum, o = orc.partition_attention(q, K, V, 0.3, ps)
        n = -(-L // ps)
        assert m.shape == (4, n) and lsum.shape == (4, n) and o.shape == (4, n, 8)
        # each partition is itself plain attention over its token range
        for k in range(n):
            part = orc.attention(q, K[k * ps:(k + 1) * ps], V[k * ps:(k + 1) * ps], 0.3)
            assert np.allclose(o[:, k], part, rtol=0, atol=1e-13)
        assert np.allclose(orc.combine_partitions(m, lsum, o), full, rtol=0, atol=1e-12)
    # one partition: the merge is the identity
    q = rng.standard_normal((2, 4))
    K = rng.standard_normal((10, 1, 4))
    V = rng.standard_normal((10, 1, 4))
    m, lsum, o = orc.partition_attention(q, K, V, 1.0, 16)
    assert np.allclose(orc.combine_partitions(m, lsum, o), o[:, 0], rtol=1e-15, atol=0)
    # closed form for the merge: two partitions with known weights
    m = np.array([[0.0, math.log(3.0)]])
    lsum = np.array([[1.0, 1.0]])
    o = np.array([[[4.0], [8.0]]])
    assert abs(orc.combine_partitions(m, lsum, o)[0, 0] - 7.0) < 1e-14


def check_decode_partials(orc):
    wl = tiny([100, 7, 64, 65], Hq=4, Hkv=2, D=8, seed=80)
    kp, vp = fill_pools(orc, wl)
    full = orc.decode(wl.query, kp, vp, wl.block_tables, wl.context_lens, wl.scale,
                      wl.page_size, wl.dtype)
    po, pm, pl = orc.decode_partials(wl.query, kp, vp, wl.block_tables, wl.context_lens,
                                     wl.scale, wl.page_size, wl.dtype, 32, 4)
    for b in range(wl.num_seqs):
        n = -(-int(wl.context_lens[b]) // 32)
        merged = orc.combine_partitions(pm[b, :, :n], pl[b, :, :n], po[b, :, :n])
        assert np.allclose(merged, full[b], rtol=0, atol=1e-12)


def check_golden(orc):
    with open(GOLDEN) as f:
        g = json.load(f)
    P, Hkv, D = g["page_size"], g["num_kv_heads"], g["head_dim"]

    def num(x):
        if isinstance(x, str):
            return 0.0 if x == "0" else math.log(float(x[2:]))
        return float(x)

    k, v = nan_pools(g["num_pages"], Hkv, P, D, "f32")
    k = k.astype(np.float64)
    v = v.astype(np.float64)
    tables, lens, qs = [], [], []
    for s in g["sequences"]:
        L = len(s["k"])
        keys = np.array([[[num(x) for x in row]] for row in s["k"]])
        vals = np.array([[[num(x) for x in row]] for row in s["v"]])
        slots = [s["block_table"][t // P] * P + t % P for t in range(L)]
        k, v = orc.cache_write(k, v, keys, vals, slots, P)
        tables.append(s["block_table"] + [-1] * (2 - len(s["block_table"])))
        lens.append(L)
        qs.append(s["q"])
    out = orc.decode(np.array(qs, dtype=np.float64), k, v,
                     np.array(tables), np.array(lens), g["scale"], P, "f64")
    for i, s in enumerate(g["sequences"]):
        assert np.allclose(out[i], np.array(s["expected"]), rtol=0, atol=1e-14), (i, out[i])


def check_chunk_single_token_is_decode(orc):
    wl = tiny([1, 17, 40, 16, 3], Hq=4, Hkv=2, D=8, seed=60)
    kp, vp = fill_pools(orc, wl)
    qs = np.arange(wl.num_seqs + 1, dtype=np.int32)
    got = orc.chunk_attention(wl.query, kp, vp, wl.block_tables, wl.context_lens, qs, wl.scale,
                              wl.page_size, wl.dtype)
    want = orc.decode(wl.query, kp, vp, wl.block_tables, wl.context_lens, wl.scale,
                      wl.page_size, wl.dtype)
    assert np.array_equal(got, want)


def check_chunk_brute_force(orc):
    cases = [
        dict(lengths=[1, 17, 40], q=[1, 5, 40], Hq=4, Hkv=2, D=6),
        dict(lengths=[33, 16], q=[33, 3], Hq=3, Hkv=1, D=5, dtype="bf16"),
        dict(lengths=[20, 9, 50], q=[0, 9, 7], Hq=2, Hkv=2, D=4),
    ]
    for i, c in enumerate(cases):
        q_lens = c.pop("q")
        wl = tiny(seed=70 + i, **c)
        query, qs = make_chunk_queries(wl, q_lens, seed=80 + i)
        kp, vp = fill_pools(orc, wl)
        got = orc.chunk_attention(query, kp, vp, wl.block_tables, wl.context_lens, qs,
                                  wl.scale, wl.page_size, wl.dtype)
        want = brute_force_chunk(wl, kp, vp, query, qs)
        assert np.allclose(got, want, rtol=0, atol=1e-12), (i, np.abs(got - want).max())


def check_chunk_torch_sdpa(orc):
    import torch

    wl = tiny([300, 77, 129], Hq=8, Hkv=2, D=32, seed=61)
    q_lens = [64, 77, 5]
    query, qs = make_chunk_queries(wl, q_lens, seed=62)
    kp, vp = fill_pools(orc, wl)
    got = orc.chunk_attention(query, kp, vp, wl.block_tables, wl.context_lens, qs, wl.scale,
                              wl.page_size, wl.dtype)
    q = widen(query, "f32")
    group = 4
    for b in range(wl.num_seqs):
        L, n = int(wl.context_lens[b]), q_lens[b]
        K = np.zeros((8, L, 32))
        V = np.zeros((8, L, 32))
        for t in range(L):
            page, slot = int(wl.block_tables[b, t // 16]), t % 16
            for h in range(8):
                K[h, t] = kp[page, h // group, slot, :]
                V[h, t] = vp[page, h // group, :, slot]
        allowed = np.arange(L)[None, :] <= (L - n + np.arange(n))[:, None]   # [n][L]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[qs[b]:qs[b + 1]].transpose(1, 0, 2).copy()),
            torch.from_numpy(K), torch.from_numpy(V), attn_mask=torch.from_numpy(allowed),
            scale=wl.scale).numpy().transpose(1, 0, 2)
        assert np.allclose(got[qs[b]:qs[b + 1]], ref, rtol=0, atol=1e-12), \
            np.abs(got[qs[b]:qs[b + 1]] - ref).max()


def check_chunk_causality(orc):
    """Changing the K/V of position p leaves every row before p bit for bit
    unchanged and changes the rows at and after p."""
    wl = tiny([40], Hq=2, Hkv=1, D=8, seed=63)
    query, qs = make_chunk_queries(wl, [12], seed=64)     # positions 28..39
    kp, vp = fill_pools(orc, wl)
    args = (wl.block_tables, wl.context_lens, qs, wl.scale, wl.page_size, wl.dtype)
    base = orc.chunk_attention(query, kp, vp, *args)
    p = 33
    page, slot = int(wl.block_tables[0, p // 16]), p % 16
    kp2, vp2 = kp.copy(), vp.copy()
    kp2[page, 0, slot, :] += 1.0
    vp2[page, 0, :, slot] -= 2.0
    moved = orc.chunk_attention(query, kp2, vp2, *args)
    row_of_p = p - (40 - 12)
    assert np.array_equal(moved[:row_of_p], base[:row_of_p])
    assert (np.abs(moved[row_of_p:] - base[row_of_p:]).max(axis=(1, 2)) > 1e-6).all()


def check_page_export_layout(orc):
    """Export against the pools read through flat offsets: buffer block i of
    section 0 is page ids[i]'s K block and of section 1 its V block, in
    order, duplicates repeated; an id outside the pool keeps the buffer's
    previous contents."""
    rng = np.random.default_rng(71)
    num_pages, Hkv, P, D = 6, 2, 16, 4
    k = rng.standard_normal((num_pages, Hkv, P, D)).astype(np.float32)
    v = rng.standard_normal((num_pages, Hkv, D, P)).astype(np.float32)
    ids = np.array([4, 0, 4, -1, 5, 6], dtype=np.int32)
    block = Hkv * P * D
    prior = np.full((2, len(ids), block), 7.5, dtype=np.float32)
    buf = orc.export_pages(k, v, ids, prior)
    assert buf.shape == (2, len(ids), block)
    kf, vf = k.reshape(-1), v.reshape(-1)
    for i, page in enumerate(ids.tolist()):
        if not 0 <= page < num_pages:
            assert (buf[:, i] == 7.5).all()
            continue
        for h in range(Hkv):
            for t in range(P):
                for d in range(D):
                    assert buf[0, i, (h * P + t) * D + d] == kf[k_offset(page, h, t, d, Hkv, P, D)]
                    assert buf[1, i, (h * D + d) * P + t] == vf[v_offset(page, h, t, d, Hkv, P, D)]


def check_page_import_layout(orc):
    """Import into NaN pools writes exactly the listed pages, element by
    element through flat offsets, and nothing for an id outside the pool."""
    rng = np.random.default_rng(72)
    num_pages, Hkv, P, D = 7, 2, 16, 4
    ids = np.array([3, 6, -2, 0, 9], dtype=np.int32)
    block = Hkv * P * D
    buf = rng.standard_normal((2, len(ids), block)).astype(np.float32)
    k0, v0 = nan_pools(num_pages, Hkv, P, D, "f32")
    k, v = orc.import_pages(k0, v0, buf, ids)
    assert np.isnan(k0).all() and np.isnan(v0).all(), "inputs must not be modified"
    kf, vf = k.reshape(-1), v.reshape(-1)
    written = 0
    for i, page in enumerate(ids.tolist()):
        if not 0 <= page < num_pages:
            continue
        written += 1
        for h in range(Hkv):
            for t in range(P):
                for d in range(D):
                    assert kf[k_offset(page, h, t, d, Hkv, P, D)] == buf[0, i, (h * P + t) * D + d]
                    assert vf[v_offset(page, h, t, d, Hkv, P, D)] == buf[1, i, (h * D + d) * P + t]
    assert int(np.count_nonzero(~np.isnan(kf))) == written * block
    assert int(np.count_nonzero(~np.isnan(vf))) == written * block


def check_page_handoff_preserves_attention(orc):
    """A batch moved page by page into another pool at other page ids, with
    its block tables remapped, gathers the same tokens and decodes to the
    same bits."""
    wl = tiny([37, 16, 5], Hq=4, Hkv=2, D=8, dtype="bf16", seed=73)
    k, v = fill_pools(orc, wl)
    npg = [-(-int(L) // 16) for L in wl.context_lens]
    ids = np.concatenate([wl.block_tables[b, :n] for b, n in enumerate(npg)]).astype(np.int32)
    buf = orc.export_pages(k, v, ids)
    dest_pages = len(ids) + 3
    new_ids = np.random.default_rng(74).permutation(dest_pages)[:len(ids)].astype(np.int32)
    k2, v2 = nan_pools(dest_pages, wl.num_kv_heads, 16, wl.head_dim, "bf16")
    k2, v2 = orc.import_pages(k2, v2, buf, new_ids)
    tables = np.full_like(wl.block_tables, -1)
    at = 0
    for b, n in enumerate(npg):
        tables[b, :n] = new_ids[at:at + n]
        at += n
    for b in range(wl.num_seqs):
        K1, V1 = orc.gather_sequence(k, v, wl.block_tables[b], wl.context_lens[b], 16)
        K2, V2 = orc.gather_sequence(k2, v2, tables[b], wl.context_lens[b], 16)
        assert np.array_equal(K1, K2) and np.array_equal(V1, V2)
    a = orc.decode(wl.query, k, v, wl.block_tables, wl.context_lens, wl.scale, 16, "bf16")
    c = orc.decode(wl.query, k2, v2, tables, wl.context_lens, wl.scale, 16, "bf16")
    assert np.array_equal(a, c)


def check_round_to_bf16(orc):
    """Round-to-nearest-even onto bf16, from float64 in one step."""
    cases = [
        (1.0, 0x3F80), (-2.0, 0xC000), (0.0, 0x0000), (-0.0, 0x8000),
        (1.0 + 2.0 ** -8, 0x3F80),                 # tie between 0x3F80 and 0x3F81: even
        (1.0 + 3 * 2.0 ** -8, 0x3F82),             # tie between 0x3F81 and 0x3F82: even
        (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),    # just past the tie
        (1.0 + 2.0 ** -8 - 2.0 ** -40, 0x3F80),    # just short of it
        (3.140625, 0x4049), (1.0 / 3.0, 0x3EAB), (-1.0 / 3.0, 0xBEAB),
        (2.0 ** -133, 0x0001),                     # smallest subnormal
        (2.0 ** -134, 0x0000),                     # tie with zero: even
        (3 * 2.0 ** -134, 0x0002),                 # tie between 0x0001 and 0x0002
        (2.0 ** -126 - 2.0 ** -140, 0x0080),       # rounds up to the smallest normal
        ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),    # largest finite
        ((2 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),    # tie with the next step: overflow
        (1e300, 0x7F80), (-math.inf, 0xFF80),
    ]
    got = orc.round_to_bf16_bits(np.array([c[0] for c in cases]))
    for (x, want), g in zip(cases, got.tolist()):
        assert g == want, (x, hex(g), hex(want))
    assert orc.round_to_bf16_bits(np.array([math.nan]))[0] == 0x7FC0
    # Every finite bf16 value maps to itself.
    bits = np.arange(0, 1 << 16, 7, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]
    assert np.array_equal(orc.round_to_bf16_bits(orc.bf16_bits_to_float64(bits)), bits)
    # Library routine: values exactly representable in binary32 round as
    # torch's float32 -> bfloat16 cast does (one rounding either way).
    import torch
    rng = np.random.default_rng(11)
    x32 = np.concatenate([rng.standard_normal(4000), rng.uniform(-1e-38, 1e-38, 500),
                          rng.standard_normal(500) * 1e30]).astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.round_to_bf16_bits(x32.astype(np.float64)), want)


def check_bf16_ulp_distance(orc):
    a = np.array([0x3F80, 0x3F80, 0x0000, 0x8000, 0x0001, 0xBF80, 0x7F7F], dtype=np.uint16)
    b = np.array([0x3F81, 0x3F80, 0x8000, 0x0001, 0x8001, 0xBF82, 0x0000], dtype=np.uint16)
    assert orc.bf16_ulp_distance(a, b).tolist() == [1, 0, 0, 1, 2, 2, 0x7F7F]


ALL_CHECKS = [
    check_bf16_widening,
    check_round_to_bf16,
    check_bf16_ulp_distance,
    check_cache_write_layout,
    check_gather_roundtrip,
    check_single_token_returns_v,
    check_constant_v,
    check_zero_query_mean,
    check_equal_keys_mean,
    check_needle,
    check_brute_force,
    check_sharp_scores,
    check_torch_sdpa,
    check_permutation_invariance,
    check_shared_vs_unshared,
    check_partitions,
    check_decode_partials,
    check_golden,
    check_chunk_single_token_is_decode,
    check_chunk_brute_force,
    check_chunk_torch_sdpa,
    check_chunk_causality,
    check_page_export_layout,
    check_page_import_layout,
    check_page_handoff_preserves_attention,
]
