"""Lengths past what the caller's buffers cover, through the C ABI:

  - a context longer than max_num_partitions * partition_size: partitions at
    or past max_num_partitions are not computed and their rows are never
    written (a shared-prefix step's suffix units count partitions from the
    sequence's first, so with the "always enough" grid bound they used to
    reach past the row); the merge then covers the first
    max_num_partitions * partition_size tokens;
  - a context longer than the block table (16 * max_pages_per_seq tokens):
    it is clamped to the table, and split-KV partitions past the clamped
    context but below ceil(L / partition_size) get empty partials, so the
    merge of pa_decode_reduce (and the one inside pa_chunk_attention_split)
    gives the clamped context's attention instead of reading unwritten rows.

Partial buffers are views into larger NaN-filled allocations: the rows after
them must stay NaN.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_pa_amd as pa
from tests.gpu_helpers import (DEV, TOL, DeviceWorkload, max_err, oracle_reference, say, to_dev)
from tests.oracle_pins import fill_pools
from tests.test_gpu_cascade import dev_groups
from tests.test_gpu_chunk import chunk_reference
from workloads import make_chunk_queries, make_custom_workload

pytestmark = pytest.mark.gpu

CANARY_ROWS = 4096


def guarded_partials(B, Hq, NP, D):
    """Partial buffers [B][Hq][NP](x D) as the heads of larger NaN buffers."""
    rows = B * Hq * NP
    po_all = torch.full((rows + CANARY_ROWS, D), float("nan"), dtype=torch.float32, device=DEV)
    pm_all = torch.full((rows + CANARY_ROWS,), float("nan"), dtype=torch.float32, device=DEV)
    ps_all = torch.full((rows + CANARY_ROWS,), float("nan"), dtype=torch.float32, device=DEV)
    views = (po_all[:rows].view(B, Hq, NP, D), pm_all[:rows].view(B, Hq, NP),
             ps_all[:rows].view(B, Hq, NP))
    return views, (po_all[rows:], pm_all[rows:], ps_all[rows:])


def assert_canaries(tails):
    for t in tails:
        assert torch.isnan(t).all().item(), "a partial row past the buffer was written"


def clamped_reference(wl, limit):
    k, v = fill_pools(oracle, wl)
    lens = np.minimum(wl.context_lens, limit).astype(np.int32)
    return oracle.decode(wl.query, k, v, wl.block_tables, lens, wl.scale, 16, wl.dtype)


@pytest.mark.parametrize("suffix_bound", [0, 40])
def test_cascade_partitions_past_the_buffer(suffix_bound):
    """Groups share 128 tokens (two 64-token partitions); contexts reach 700
    tokens but the buffers hold 6 partitions (384 tokens).  A grid bound of
    0 ("always enough") or an overestimate must not let a suffix unit write
    partition 6 or later."""
    say(f"[bounds] cascade, contexts past max_num_partitions, suffix bound {suffix_bound}")
    rng = np.random.default_rng(3)
    B, ps, NP = 24, 64, 6
    group_of = np.where(np.arange(B) < 16, np.arange(B) // 8, -1)
    lens = np.where(group_of >= 0, 129 + rng.integers(0, 570, B), 1 + rng.integers(0, 699, B))
    wl = make_custom_workload(lens.tolist(), num_q_heads=16, num_kv_heads=2, head_dim=128,
                              seed=21, group_of=group_of.tolist(), prefix_tokens=128)
    g = pa.prefix_groups(wl.block_tables, wl.context_lens, ps // 16)
    assert g["num_groups"] == 2 and g["max_group_partitions"] == 2
    dev = DeviceWorkload(wl)
    (po, pm, psum), tails = guarded_partials(B, 16, NP, 128)
    pa.pa_decode_cascade(dev.query, dev.k_cache, dev.v_cache, dev.block_tables, dev.context_lens,
                         wl.scale, ps, po, pm, psum,
                         dev_groups(dict(g, max_suffix_partitions=suffix_bound)))
    out = torch.empty((B, 16, 128), dtype=torch.bfloat16, device=DEV)
    pa.pa_decode_reduce(out, po, pm, psum, dev.context_lens, ps)
    torch.cuda.synchronize()
    assert_canaries(tails)
    err = max_err(out, clamped_reference(wl, NP * ps))
    say(f"    max abs err {err:.3e} against the first {NP * ps} tokens")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("kernel", ["auto", "valu"])
@pytest.mark.parametrize("ps", [64, 256])
def test_decode_partitions_past_the_buffer(kernel, ps):
    say(f"[bounds] pa_decode {kernel}, contexts past max_num_partitions, partition {ps}")
    wl = make_custom_workload([900, 40, 1300, 257], num_q_heads=16, num_kv_heads=2, head_dim=128,
                              seed=22)
    NP = 3
    dev = DeviceWorkload(wl)
    (po, pm, psum), tails = guarded_partials(4, 16, NP, 128)
    fn = pa.pa_decode if kernel == "auto" else pa.pa_decode_valu
    fn(None, dev.query, dev.k_cache, dev.v_cache, dev.block_tables, dev.context_lens, wl.scale,
       ps, po, pm, psum)
    out = torch.empty((4, 16, 128), dtype=torch.bfloat16, device=DEV)
    pa.pa_decode_reduce(out, po, pm, psum, dev.context_lens, ps)
    torch.cuda.synchronize()
    assert_canaries(tails)
    assert max_err(out, clamped_reference(wl, NP * ps)) <= TOL["bf16"]


def table_width_workload():
    """Sequences 0 and 2 fill the 64-column table exactly (1024 tokens); the
    device lengths of those two are then raised past it."""
    wl = make_custom_workload([1024, 300, 1024, 77], num_q_heads=16, num_kv_heads=2,
                              head_dim=128, seed=23, max_pages_per_seq=64)
    dev = DeviceWorkload(wl)
    dev.context_lens[0] = 1024 + 300
    dev.context_lens[2] = 5000
    return wl, dev


@pytest.mark.parametrize("kernel", ["auto", "valu"])
@pytest.mark.parametrize("ps", [0, 64, 256, 768])
def test_decode_length_past_the_table_is_clamped(kernel, ps):
    say(f"[bounds] pa_decode {kernel}, lengths past the block table, partition {ps}")
    wl, dev = table_width_workload()
    ref = oracle_reference(wl)  # every length clamps back to what the table holds
    # Partition slots for the raw lengths: the ones past the table must be
    # written empty, or the merge reads the NaN fill.
    out = dev.decode(ps, kernel, max_parts=(-(-5000 // ps) if ps else None))
    assert max_err(out, ref) <= TOL["bf16"]


@pytest.mark.parametrize("ps", [64, 256])
def test_chunk_split_length_past_the_table_is_clamped(ps):
    say(f"[bounds] pa_chunk_attention_split, lengths past the block table, partition {ps}")
    wl, dev = table_width_workload()
    query, qs = make_chunk_queries(wl, [4, 4, 4, 4], seed=5)
    ref = chunk_reference(wl, query, qs)
    q = to_dev(query, wl.dtype)
    qst = torch.from_numpy(qs).to(DEV)
    T, Hq, D = q.shape
    NP = -(-5000 // ps)
    po = torch.full((T, Hq, NP, D), float("nan"), dtype=torch.float32, device=DEV)
    pm = torch.full((T, Hq, NP), float("nan"), dtype=torch.float32, device=DEV)
    psum = torch.full((T, Hq, NP), float("nan"), dtype=torch.float32, device=DEV)
    out = torch.full_like(q, float("nan"))
    # The queries of the raised sequences sit at the end of the clamped
    # context: the last four positions of the table.
    pa.pa_chunk_attention_split(out, q, dev.k_cache, dev.v_cache, dev.block_tables,
                                dev.context_lens, qst, 4, wl.scale, ps, po, pm, psum)
    single = torch.full_like(q, float("nan"))
    pa.pa_chunk_attention(single, q, dev.k_cache, dev.v_cache, dev.block_tables,
                          dev.context_lens, qst, 4, wl.scale)
    torch.cuda.synchronize()
    assert max_err(out, ref) <= TOL["bf16"]
    assert max_err(single, ref) <= TOL["bf16"]
