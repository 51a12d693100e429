"""Exact-output parity: inputs whose attention result is a ratio of small
integers, so every page that is dropped, read twice, read from the wrong
slot or masked wrongly moves the output by many bf16 ulps, and the library
must land within one bf16 ulp of the oracle's value rounded once to
nearest-even.

Value recipe (synthetic, seeded): V of the token at logical position p,
kv head g, is a row of zeros with a 1 at dim (p // 16 + 3g) mod (D - 16)
(its page, shifted per kv head) and a 1 at dim D - 16 + p % 16 (its slot in
the page).  Two query recipes:
  flat  q = 0: every score is 0 and every weight exactly 1, so the output
        is (tokens per page residue and per slot) / L, exact in fp32 and
        checking the whole V stream and the masking of partial pages;
  comb  q = e_0 and key dim 0 in [-1, 1], except one key per page (slot
        7 * page mod 16, so position 0 always) set to 2304: those scores
        are equal and exact, every other weight underflows to exactly 0 in
        fp32, and the output is the mean of the needles' V rows; a K tile
        dropped, misplaced or read from another page changes which needles
        count.
One bf16 ulp is the bound: the kernels' sums of these values are exact and
their final quotient carries a few fp32 roundings, which can move the bf16
result across at most one rounding boundary.

Lengths, head shapes and page scattering are those of the Llama-3-8B
batch (config 2), the long-context batch (4), the 70B share (5) and the
prefix-reuse batch (3), at single pass, each benchmarked partition and
2048 / 4096-token partitions (one wave then walks 128 or 256 pages, past the
64-id page-table refresh of its stream).
"""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_pa_amd as pa
from tests.gpu_helpers import (DEV, DeviceWorkload, bits_of, config_workload, say, tdtype,
                               to_dev)
from tests.oracle_pins import fill_pools
from tests.test_gpu_cascade import cascade
from tests.test_gpu_chunk import chunk_reference, run_chunk
from tests.test_gpu_chunk_split import run_split
from tests.test_gpu_decode_append import fused_step
from workloads import config_by_id, make_chunk_queries, make_custom_workload

pytestmark = pytest.mark.gpu

NEEDLE = 2304.0  # exact in bf16; scale * NEEDLE is about 204 (D = 128) or 288 (D = 64)


def needle_slot(page):
    return (7 * page) % 16


def indicator_values(mode):
    def fn(q, k, v, owners, lengths):
        pos = np.fromiter((p for _, p in owners), dtype=np.int64, count=len(owners))
        page, slot = pos // 16, pos % 16
        T, Hkv, D = v.shape
        rows = np.arange(T)
        v[:] = 0.0
        for g in range(Hkv):
            v[rows, g, (page + 3 * g) % (D - 16)] = 1.0
            v[rows, g, D - 16 + slot] = 1.0
        q[:] = 0.0
        if mode == "comb":
            q[:, :, 0] = 1.0
            k[:, :, 0] = np.clip(k[:, :, 0], -1.0, 1.0)
            k[slot == needle_slot(page), :, 0] = NEEDLE
        return q, k, v
    return fn


def chunk_query_values(mode):
    def fn(q32, query_start):
        q32[:] = 0.0
        if mode == "comb":
            q32[:, :, 0] = 1.0
        return q32
    return fn


@functools.lru_cache(maxsize=None)
def exact_workload(cid, mode):
    """Config cid's lengths, heads and scattering with the indicator values."""
    cfg = config_by_id(cid)
    base = config_workload(cid)
    kw = {}
    if cfg.prefix_group_size:
        kw = dict(group_size=cfg.prefix_group_size, prefix_tokens=cfg.prefix_tokens)
    return make_custom_workload(base.context_lens.tolist(), num_q_heads=cfg.num_q_heads,
                                num_kv_heads=cfg.num_kv_heads, head_dim=cfg.head_dim,
                                dtype=cfg.dtype, seed=500 + cid, value_fn=indicator_values(mode),
                                **kw)


@functools.lru_cache(maxsize=None)
def exact_reference_bits(cid, mode):
    wl = exact_workload(cid, mode)
    k, v = fill_pools(oracle, wl)
    ref = oracle.decode(wl.query, k, v, wl.block_tables, wl.context_lens, wl.scale,
                        wl.page_size, wl.dtype)
    return oracle.round_to_bf16_bits(ref)


@functools.lru_cache(maxsize=None)
def exact_device(cid, mode):
    return DeviceWorkload(exact_workload(cid, mode))


def check_exact(out, want_bits, what):
    got = bits_of(out)
    assert not np.isnan(out.float().cpu().numpy()).any(), f"{what}: NaN"
    ulp = oracle.bf16_ulp_distance(got, want_bits)
    worst = int(ulp.max())
    say(f"    {what}: max {worst} bf16 ulp, {int((ulp > 0).sum())} of {ulp.size} not equal")
    assert worst <= 1, (what, np.argwhere(ulp > 1)[:5].tolist())


def _partitions(cid):
    extra = {768} if cid == 2 else set()
    return sorted({0, config_by_id(cid).bench_partition_size, 2048, 4096} | extra)


DECODE_CASES = [(cid, mode, ps) for cid in (2, 4, 5) for mode in ("flat", "comb")
                for ps in _partitions(cid)]


@pytest.mark.parametrize("cid,mode,ps", DECODE_CASES,
                         ids=[f"cfg{c}-{m}-ps{p}" for c, m, p in DECODE_CASES])
def test_decode_exact(cid, mode, ps):
    say(f"[exact] pa_decode config {cid} {mode} partition {ps}")
    dev = exact_device(cid, mode)
    check_exact(dev.decode(ps), exact_reference_bits(cid, mode), "pa_decode")


@pytest.mark.parametrize("cid,mode", [(2, "flat"), (2, "comb"), (5, "comb")])
def test_decode_valu_exact(cid, mode):
    dev = exact_device(cid, mode)
    for ps in sorted({0, config_by_id(cid).bench_partition_size or 768}):
        say(f"[exact] pa_decode_valu config {cid} {mode} partition {ps}")
        check_exact(dev.decode(ps, "valu"), exact_reference_bits(cid, mode), "pa_decode_valu")


APPEND_CASES = [(cid, mode, ps) for cid in (2, 4, 5) for mode in ("flat", "comb")
                for ps in sorted({0, config_by_id(cid).bench_partition_size, 4096}
                                 | ({768} if cid == 2 else set()))]


@pytest.mark.parametrize("cid,mode,ps", APPEND_CASES,
                         ids=[f"cfg{c}-{m}-ps{p}" for c, m, p in APPEND_CASES])
def test_decode_append_exact(cid, mode, ps):
    """The one-call step on a pool holding only the cached tokens: the step's
    token (position L - 1, a needle when its slot is the page's) is written and
    attended in the same launch."""
    say(f"[exact] pa_decode_append config {cid} {mode} partition {ps}")
    wl = exact_workload(cid, mode)
    dev = DeviceWorkload(wl, fill=False)
    dev.prefill()
    check_exact(fused_step(dev, ps), exact_reference_bits(cid, mode), "pa_decode_append")


@pytest.mark.parametrize("mode", ["flat", "comb"])
@pytest.mark.parametrize("ps", [512, 2048])
@pytest.mark.parametrize("append", [False, True])
def test_cascade_exact(mode, ps, append):
    say(f"[exact] pa_decode_cascade prefix-reuse batch {mode} partition {ps} append {append}")
    wl = exact_workload(3, mode)
    groups = pa.prefix_groups(wl.block_tables, wl.context_lens, ps // 16)
    assert groups["num_groups"] == 8
    if append:
        dev = DeviceWorkload(wl, fill=False)
        dev.prefill()
    else:
        dev = exact_device(3, mode)
    check_exact(cascade(dev, ps, groups, append=append), exact_reference_bits(3, mode),
                "pa_decode_cascade")


@functools.lru_cache(maxsize=None)
def exact_chunk(mode, q_len):
    wl = exact_workload(2, mode)
    query, qs = make_chunk_queries(wl, [q_len] * wl.num_seqs, seed=q_len,
                                   value_fn=chunk_query_values(mode))
    return query, qs, oracle.round_to_bf16_bits(chunk_reference(wl, query, qs))


@pytest.mark.parametrize("mode", ["flat", "comb"])
@pytest.mark.parametrize("q_len", [1, 4, 8, 16])
def test_chunk_attention_exact(mode, q_len):
    say(f"[exact] pa_chunk_attention config 2 lengths, {q_len} new tokens, {mode}")
    query, qs, want = exact_chunk(mode, q_len)
    check_exact(run_chunk(exact_device(2, mode), query, qs), want, "pa_chunk_attention")


@pytest.mark.parametrize("mode", ["flat", "comb"])
@pytest.mark.parametrize("q_len", [32, 64])
def test_chunk_attention_lds_exact(mode, q_len):
    """32 or 64 new tokens per sequence (128 or 256 columns per kv head at
    group 4: the kernel that stages K/V in LDS, in four-wave units in the
    snake order with nontemporal loads, or eight-wave units longest first),
    on the eight longest of config 2's lengths (the oracle of all 64
    sequences takes about a minute)."""
    say(f"[exact] pa_chunk_attention, {q_len} new tokens, eight longest config 2 lengths, {mode}")
    cfg = config_by_id(2)
    lens = sorted(config_workload(2).context_lens.tolist(), reverse=True)[:8]
    wl = make_custom_workload(lens, num_q_heads=cfg.num_q_heads, num_kv_heads=cfg.num_kv_heads,
                              head_dim=cfg.head_dim, dtype=cfg.dtype, seed=640,
                              value_fn=indicator_values(mode))
    query, qs = make_chunk_queries(wl, [q_len] * wl.num_seqs, seed=q_len,
                                   value_fn=chunk_query_values(mode))
    want = oracle.round_to_bf16_bits(chunk_reference(wl, query, qs))
    check_exact(run_chunk(DeviceWorkload(wl), query, qs), want, "pa_chunk_attention (LDS)")


@pytest.mark.parametrize("mode", ["flat", "comb"])
@pytest.mark.parametrize("q_len,ps", [(4, 768), (4, 2048), (16, 768)])
def test_chunk_attention_split_exact(mode, q_len, ps):
    say(f"[exact] pa_chunk_attention_split config 2 lengths, {q_len} new tokens, {mode}, "
        f"partition {ps}")
    query, qs, want = exact_chunk(mode, q_len)
    check_exact(run_split(exact_device(2, mode), query, qs, ps), want,
                "pa_chunk_attention_split")


# --------------------------------------------------------------- stream ordinals
# A wave refreshes its page ids every 64 pages of its stream.  One needle per
# sequence at stream ordinal k of some wave: the output must be that token's V
# row, bit for bit (every other weight is exactly 0).
ORDINAL_CASES = [
    # (mode, partition size, ordinal k): the needle's logical page
    ("single", 0, 63), ("single", 0, 64), ("single", 0, 127), ("single", 0, 128),
    ("split", 2048, 63), ("split", 2048, 64), ("split", 2048, 127),
    ("split", 4096, 63), ("split", 4096, 64), ("split", 4096, 127), ("split", 4096, 128),
]


def _needle_page(mode, ps, k, b):
    if mode == "single":           # four waves per unit: wave w takes pages w, w + 4, ...
        return 4 * k + b % 4
    return (b % 2) * (ps // 16) + k  # ordinal k of partition 0 or 1


@pytest.mark.parametrize("mode,ps,k", ORDINAL_CASES,
                         ids=[f"{m}-ps{p}-ord{k}" for m, p, k in ORDINAL_CASES])
@pytest.mark.parametrize("entry", ["pa_decode", "pa_decode_append"])
def test_needle_at_stream_ordinal(mode, ps, k, entry):
    say(f"[exact] needle at stream ordinal {k}, {mode} partition {ps}, {entry}")
    lens = [8704, 9000, 17000, 12000, 8192 + 600, 16400]
    needle_pos = {b: 16 * _needle_page(mode, ps, k, b) + 5 for b in range(len(lens))}
    assert all(needle_pos[b] < lens[b] - 1 for b in needle_pos)

    def fn(q, kk, v, owners, lengths):
        q[:] = 0.0
        q[:, :, 0] = 1.0
        kk[:, :, 0] = np.clip(kk[:, :, 0], -1.0, 1.0)
        for i, (key, pos) in enumerate(owners):
            if key[0] == "s" and needle_pos[key[1]] == pos:
                kk[i, :, 0] = NEEDLE
        return q, kk, v

    wl = make_custom_workload(lens, num_q_heads=16, num_kv_heads=2, head_dim=128, seed=k + ps,
                              value_fn=fn)
    if entry == "pa_decode":
        dev = DeviceWorkload(wl)
        out = dev.decode(ps)
    else:
        dev = DeviceWorkload(wl, fill=False)
        dev.prefill()
        out = fused_step(dev, ps)
    k_pool, v_pool = fill_pools(oracle, wl)
    got = bits_of(out)
    for b in range(len(lens)):
        pos = needle_pos[b]
        page = int(wl.block_tables[b, pos // 16])
        for h in range(16):
            g = h // 8
            want = v_pool[page, g, :, pos % 16]
            assert np.array_equal(got[b, h], want), (b, h)
    ref = oracle.decode(wl.query, k_pool, v_pool, wl.block_tables, wl.context_lens, wl.scale, 16,
                        "bf16")
    assert np.array_equal(got, oracle.round_to_bf16_bits(ref))
