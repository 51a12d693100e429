"""pa_chunk_attention (several new tokens per sequence, causal) against the
fp64 oracle, plus the structural properties the bf16 tolerance could hide:
one token per sequence reproduces pa_decode bit for bit, later tokens' K/V
never touch earlier rows, and page placement changes nothing."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_pa_amd as pa
from tests.gpu_helpers import (DEV, TOL, DeviceWorkload, bits_of, config_device, config_workload,
                               f64_of, max_err, say, to_dev)
from tests.oracle_pins import fill_pools
from workloads import make_chunk_queries, make_custom_workload

pytestmark = pytest.mark.gpu

LDS_MIN_COLUMNS = 64  # max_query_len * group above this: the LDS-staged kernel


def run_chunk(dev, query, query_start, max_q=None):
    wl = dev.wl
    q = to_dev(query, wl.dtype)
    qs = torch.from_numpy(np.asarray(query_start, dtype=np.int32)).to(DEV)
    out = torch.full_like(q, float("nan"))
    lens = np.diff(np.asarray(query_start))
    mq = int(lens.max()) if max_q is None else max_q
    pa.pa_chunk_attention(out, q, dev.k_cache, dev.v_cache, dev.block_tables, dev.context_lens,
                          qs, mq, wl.scale)
    torch.cuda.synchronize()
    return out


def chunk_reference(wl, query, query_start):
    k, v = fill_pools(oracle, wl)
    return oracle.chunk_attention(query, k, v, wl.block_tables, wl.context_lens, query_start,
                                  wl.scale, wl.page_size, wl.dtype)


@pytest.mark.parametrize("cid", [2, 5, 3])
def test_one_token_per_sequence_is_decode(cid):
    say(f"[chunk] q_len = 1 equals single-pass decode, config {cid}")
    dev = config_device(cid)
    wl = dev.wl
    qs = np.arange(wl.num_seqs + 1, dtype=np.int32)
    got = run_chunk(dev, wl.query, qs)
    assert np.array_equal(bits_of(got), bits_of(dev.decode(0)))


CASES = [
    # lengths, new-token counts, Hq, Hkv, D
    ([300, 77, 129, 16], [64, 77, 5, 1], 8, 2, 128),     # whole-sequence prefill, group 4
    ([1000, 33, 512], [7, 2, 16], 32, 8, 128),           # drafted tokens, group 4
    ([700, 48], [33, 17], 16, 1, 128),                   # group 16: one token per block
    ([257, 90], [40, 90], 8, 8, 64),                     # no grouping: 16 tokens per block
    ([400, 260], [200, 150], 8, 8, 64),                  # D = 64, eight-wave LDS units
    ([130, 64, 200], [12, 3, 0], 12, 4, 64),             # group 3 straddles blocks; q_len 0
    ([600, 100], [8, 5], 32, 8, 128),                    # two column blocks per wave
    ([2048 + 300], [300], 8, 1, 128),                    # chunked prefill on a long context
]


@pytest.mark.parametrize("lens,q_lens,Hq,Hkv,D", CASES)
def test_chunk_matches_oracle(lens, q_lens, Hq, Hkv, D):
    say(f"[chunk] {lens} q {q_lens} {Hq}/{Hkv}/{D}")
    wl = make_custom_workload(lens, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                              seed=sum(lens) + Hq)
    query, qs = make_chunk_queries(wl, q_lens, seed=len(lens) + D)
    ref = chunk_reference(wl, query, qs)
    dev = DeviceWorkload(wl)
    got = run_chunk(dev, query, qs)
    err = max_err(got, ref)
    say(f"    max abs err {err:.3e}")
    assert err <= TOL["bf16"]
    # A looser bound on q_len changes how many column blocks a wave carries
    # and adds units that exit at once; each column's arithmetic is the same
    # as long as the bound keeps the same kernel (past 64 columns per kv
    # head the LDS-staged kernel runs, with its own rounding order).
    loose = run_chunk(dev, query, qs, max_q=int(qs[-1]))
    G = Hq // Hkv
    if (max(q_lens) * G > LDS_MIN_COLUMNS) == (int(qs[-1]) * G > LDS_MIN_COLUMNS):
        assert np.array_equal(bits_of(loose), bits_of(got))
    else:
        assert max_err(loose, ref) <= TOL["bf16"]


def test_spec_decode_batch_at_config_2_shape():
    """Four new tokens for each of config 2's 64 sequences (the shape of a
    draft verification step), against the oracle."""
    say("[chunk] config 2 shape, 4 new tokens per sequence")
    wl = config_workload(2)
    query, qs = make_chunk_queries(wl, [4] * wl.num_seqs, seed=2)
    ref = chunk_reference(wl, query, qs)
    got = run_chunk(config_device(2), query, qs)
    assert max_err(got, ref) <= TOL["bf16"]


@pytest.mark.parametrize("B", [130, 1100])
def test_many_sequences_with_equal_lengths(B):
    """Units run longest sequence first: batches past one 64-sequence ballot
    chunk (130) and past the ordered range (1100, batch order), with many
    equal lengths and some new tokens preceding others' contexts; every row
    against the oracle, and a second call gives the same bits."""
    say(f"[chunk] {B} sequences, lengths from a few values")
    rng = np.random.default_rng(B)
    lens = rng.choice([3, 16, 17, 40, 97], size=B).tolist()
    wl = make_custom_workload(lens, num_q_heads=8, num_kv_heads=2, head_dim=64, seed=B)
    q_lens = [min(n, int(rng.integers(1, 6))) for n in lens]
    query, qs = make_chunk_queries(wl, q_lens, seed=B + 1)
    ref = chunk_reference(wl, query, qs)
    dev = DeviceWorkload(wl)
    got = run_chunk(dev, query, qs)
    assert max_err(got, ref) <= TOL["bf16"]
    assert np.array_equal(bits_of(run_chunk(dev, query, qs)), bits_of(got))


def test_lds_units_past_the_ordered_batch_sizes():
    """1100 sequences with 17-20 new tokens at a group of 4 (68-80 columns:
    four-wave LDS units), past the batch sizes whose units are ordered by
    length (they run in batch order); every row against the oracle."""
    say("[chunk] 1100 sequences, LDS units in batch order")
    rng = np.random.default_rng(1700)
    lens = rng.choice([20, 33, 40, 97], size=1100).tolist()
    wl = make_custom_workload(lens, num_q_heads=8, num_kv_heads=2, head_dim=64, seed=1701)
    q_lens = [min(n, int(rng.integers(17, 21))) for n in lens]
    query, qs = make_chunk_queries(wl, q_lens, seed=1702)
    ref = chunk_reference(wl, query, qs)
    got = run_chunk(DeviceWorkload(wl), query, qs)
    assert max(q_lens) * 4 > LDS_MIN_COLUMNS
    assert max_err(got, ref) <= TOL["bf16"]


@pytest.mark.parametrize("q", [16, 32, 64, 128])
def test_bench_shape_on_sampled_sequences(q):
    """q new tokens for each of config 2's 64 sequences, the single-pass launch
    that the multi-token bench times.  The GPU runs the whole batch;
    the oracle checks eight sequences (the longest, the shortest and six
    seeded picks), every row of each."""
    say(f"[chunk] config 2 shape, {q} new tokens per sequence, sampled oracle")
    wl = config_workload(2)
    query, qs = make_chunk_queries(wl, [q] * wl.num_seqs, seed=q)
    got = run_chunk(config_device(2), query, qs).float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    lens = np.asarray(wl.context_lens)
    rng = np.random.default_rng(q)
    pick = sorted({int(lens.argmax()), int(lens.argmin()),
                   *rng.choice(wl.num_seqs, 6, replace=False).tolist()})
    k, v = fill_pools(oracle, wl)
    for b in pick:
        lo, hi = int(qs[b]), int(qs[b + 1])
        ref = oracle.chunk_attention(query[lo:hi], k, v, wl.block_tables[b:b + 1],
                                     wl.context_lens[b:b + 1], np.array([0, hi - lo]),
                                     wl.scale, wl.page_size, wl.dtype)
        err = float(np.abs(got[lo:hi] - ref).max())
        assert err <= TOL["bf16"], (b, err)


@pytest.mark.parametrize("q", [4, 32])
def test_prefix_groups_on_sampled_sequences(q):
    """q new tokens for each of the prefix-reuse batch's 128 sequences (8
    groups of 16 sharing their first 128 pages): neighbours share a first
    page, so the single-pass units keep batch order and cached loads (the
    register kernel at q = 4, four-wave LDS units at q = 32).  Eight sampled
    sequences against the oracle, every row of each."""
    say(f"[chunk] prefix-reuse batch, {q} new tokens per sequence, sampled oracle")
    wl = config_workload(3)
    query, qs = make_chunk_queries(wl, [q] * wl.num_seqs, seed=300 + q)
    got = run_chunk(config_device(3), query, qs).float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    rng = np.random.default_rng(q)
    pick = sorted({0, 15, 16, wl.num_seqs - 1, *rng.choice(wl.num_seqs, 4, replace=False).tolist()})
    k, v = fill_pools(oracle, wl)
    for b in pick:
        lo, hi = int(qs[b]), int(qs[b + 1])
        ref = oracle.chunk_attention(query[lo:hi], k, v, wl.block_tables[b:b + 1],
                                     wl.context_lens[b:b + 1], np.array([0, hi - lo]),
                                     wl.scale, wl.page_size, wl.dtype)
        err = float(np.abs(got[lo:hi] - ref).max())
        assert err <= TOL["bf16"], (b, err)


@pytest.mark.parametrize("seed", range(8))
def test_chunk_random(seed):
    """Seeded random batches through both single-pass kernels: kv heads, group
    size, head dim, batch size (some contexts empty or one token long), new
    tokens per sequence up to 40 (so that max_query_len * group runs from a
    few columns to hundreds, across the register and LDS kernels), optional
    prefix groups (batch order, cached loads).  Every row against the oracle."""
    rng = np.random.default_rng(5000 + seed)
    B = int(rng.integers(1, 48))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    D = int(rng.choice([64, 128]))
    lens = np.where(rng.random(B) < 0.15, rng.integers(0, 2, B), rng.integers(2, 700, B))
    kw = {}
    if B >= 4 and rng.random() < 0.4:
        n_groups = int(rng.integers(1, 3))
        group_of = np.where(np.arange(B) < 2 * n_groups * 2, np.arange(B) // 4 % n_groups, -1)
        group_of = np.where(np.arange(B) < 4 * n_groups, group_of, -1)
        prefix = 16 * int(rng.integers(1, 8))
        lens = np.where(group_of >= 0, prefix + rng.integers(1, 100, B), lens)
        kw = dict(group_of=group_of.tolist(), prefix_tokens=prefix)
    q_cap = int(rng.choice([4, 16, 40]))
    q_lens = [int(min(n, rng.integers(1, q_cap + 1))) for n in lens]
    say(f"[chunk random {seed}] B={B} {Hkv * G}/{Hkv}/{D} q up to {max(q_lens)} "
        f"({max(q_lens) * G} columns) groups {bool(kw)}")
    wl = make_custom_workload([int(x) for x in lens], num_q_heads=Hkv * G, num_kv_heads=Hkv,
                              head_dim=D, seed=seed, placement_seed=seed + 7, **kw)
    query, qs = make_chunk_queries(wl, q_lens, seed=seed + 11)
    ref = chunk_reference(wl, query, qs)
    got = run_chunk(DeviceWorkload(wl), query, qs)
    assert max_err(got, ref) <= TOL["bf16"]


def test_later_tokens_never_reach_earlier_rows():
    say("[chunk] causality on the GPU")
    wl = make_custom_workload([200], num_q_heads=8, num_kv_heads=2, head_dim=128, seed=5)
    query, qs = make_chunk_queries(wl, [40], seed=6)               # positions 160..199
    dev = DeviceWorkload(wl)
    base = bits_of(run_chunk(dev, query, qs))
    p = 181                                                          # row p - 160 = 21
    page, slot = int(wl.block_tables[0, p // 16]), p % 16
    dev.k_cache[page, :, slot, :] *= -3
    dev.v_cache[page, :, :, slot] += 1
    moved = bits_of(run_chunk(dev, query, qs))
    assert np.array_equal(moved[:21], base[:21])
    assert not np.array_equal(moved[21], base[21])


def test_placement_and_repeats_do_not_change_bits():
    say("[chunk] placement invariance and determinism")
    lens, q_lens = [513, 40, 1000], [9, 40, 3]
    a = make_custom_workload(lens, num_q_heads=32, num_kv_heads=8, head_dim=128, seed=9)
    b = make_custom_workload(lens, num_q_heads=32, num_kv_heads=8, head_dim=128, seed=9,
                             placement_seed=3)
    query, qs = make_chunk_queries(a, q_lens, seed=10)
    ga = bits_of(run_chunk(DeviceWorkload(a), query, qs))
    db = DeviceWorkload(b)
    assert np.array_equal(ga, bits_of(run_chunk(db, query, qs)))
    assert np.array_equal(ga, bits_of(run_chunk(db, query, qs)))
