"""The seeded workload generator: reproducible, valid tables, the configs' structure."""
import math

import numpy as np
import pytest

from workloads import CONFIGS, config_by_id, make_custom_workload, make_workload
from workloads.configs import _lengths_for


def _check_valid(wl):
    B, P = wl.num_seqs, wl.page_size
    used = set()
    for b in range(B):
        L = int(wl.context_lens[b])
        n = -(-L // P)
        row = wl.block_tables[b]
        assert (row[:n] >= 0).all() and (row[:n] < wl.num_pages).all()
        assert (row[n:] == -1).all()
        used.update(row[:n].tolist())
        # the appended token's slot is the last position of this sequence
        assert wl.new_slots[b] == int(row[(L - 1) // P]) * P + (L - 1) % P
    assert len(used) == wl.unique_pages <= wl.num_pages
    slots = np.concatenate([wl.prefill_slots, wl.new_slots])
    assert len(np.unique(slots)) == len(slots), "every slot is written once"
    assert (slots >= 0).all() and (slots < wl.num_pages * P).all()
    assert len(slots) == sum(1 for _ in slots)


@pytest.mark.parametrize("cid", [1, 3, 5])
def test_config_valid_and_reproducible(cid):
    cfg = config_by_id(cid)
    a = make_workload(cfg)
    b = make_workload(cfg)
    _check_valid(a)
    for name in ("context_lens", "block_tables", "query", "prefill_key", "prefill_value",
                 "prefill_slots", "new_key", "new_value", "new_slots"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    assert a.query.shape == (cfg.num_seqs, cfg.num_q_heads, cfg.head_dim)
    assert a.query.dtype == (np.float32 if cfg.dtype == "f32" else np.uint16)


def test_config1_shape():
    wl = make_workload(config_by_id(1))
    assert wl.context_lens.tolist() == [17, 64, 100, 255]
    assert wl.num_pages == 64 and wl.unique_pages == 2 + 4 + 7 + 16


def test_config3_sharing():
    cfg = config_by_id(3)
    wl = make_workload(cfg)
    assert (wl.context_lens >= 2048 + 64).all() and (wl.context_lens <= 2048 + 512).all()
    for g in range(8):
        rows = wl.block_tables[g * 16:(g + 1) * 16, :128]
        assert (rows == rows[0]).all(), "a group's 128 prefix pages are one set"
    assert len(set(wl.block_tables[:, 0].tolist())) == 8
    un = make_workload(cfg, share_prefix=False)
    assert un.unique_pages == wl.unique_pages + 8 * 15 * 128
    assert np.array_equal(un.context_lens, wl.context_lens)
    assert np.array_equal(un.query, wl.query) and np.array_equal(un.new_key, wl.new_key)
    need = sum(-(-int(L) // 16) for L in wl.context_lens) - 8 * 15 * 128
    assert wl.unique_pages == need and wl.num_pages == math.ceil(1.25 * need)


def test_config5_mix():
    cfg = config_by_id(5)
    L = make_workload(cfg).context_lens
    assert int((L <= 32).sum()) == 64 and (L >= 1).all()
    long = L[L > 32]
    assert (long >= 128).all() and (long <= 8192).all()
    assert len(long) == 192


@pytest.mark.parametrize("cid,lo,hi", [(2, 512, 4096), (4, 16384, 32768)])
def test_big_config_lengths(cid, lo, hi):
    cfg = config_by_id(cid)
    L = _lengths_for(cfg, np.random.default_rng(1000 + cid))
    assert len(L) == cfg.num_seqs and (L >= lo).all() and (L <= hi).all()


def test_placement_variant_keeps_values():
    a = make_custom_workload([40, 3, 17], num_q_heads=4, num_kv_heads=2, head_dim=8, seed=5)
    b = make_custom_workload([40, 3, 17], num_q_heads=4, num_kv_heads=2, head_dim=8, seed=5,
                             placement_seed=6)
    assert not np.array_equal(a.block_tables, b.block_tables)
    assert np.array_equal(a.prefill_key, b.prefill_key)
    assert np.array_equal(a.new_value, b.new_value)
    _check_valid(a)
    _check_valid(b)


def test_config_table():
    assert [c.config_id for c in CONFIGS] == [1, 2, 3, 4, 5]
    for c in CONFIGS:
        assert c.num_q_heads % c.num_kv_heads == 0 and c.page_size == 16


def test_scattered_groups_share_prefix_pages():
    group_of = [2, -1, 0, 2, 0, -1, 2]
    lens = [70, 10, 100, 65, 90, 33, 81]
    wl = make_custom_workload(lens, num_q_heads=4, num_kv_heads=2, head_dim=64, seed=3,
                              prefix_tokens=64, group_of=group_of)
    t = wl.block_tables
    for a, b in [(0, 3), (0, 6), (2, 4)]:
        assert (t[a, :4] == t[b, :4]).all()
    assert t[0, 0] != t[2, 0] and t[1, 0] != t[5, 0]
    assert len(set(t[:, 4].tolist()) - {-1}) == len([x for x in lens if x > 64])
    private = make_custom_workload(lens, num_q_heads=4, num_kv_heads=2, head_dim=64, seed=3,
                                   prefix_tokens=64, group_of=group_of, share_prefix=False)
    assert len(set(private.block_tables[:, 0].tolist())) == len(lens)


def test_chunk_queries_layout_and_bounds():
    from workloads import make_chunk_queries
    wl = make_custom_workload([5, 20, 33], num_q_heads=4, num_kv_heads=2, head_dim=8, seed=1)
    q, qs = make_chunk_queries(wl, [2, 20, 0], seed=3)
    assert qs.tolist() == [0, 2, 22, 22] and q.shape == (22, 4, 8) and q.dtype == np.uint16
    q2, _ = make_chunk_queries(wl, [2, 20, 0], seed=3)
    assert np.array_equal(q, q2)
    with pytest.raises(ValueError):
        make_chunk_queries(wl, [6, 1, 1])           # more tokens than the context holds
    with pytest.raises(ValueError):
        make_chunk_queries(wl, [1, 1])              # one length per sequence
