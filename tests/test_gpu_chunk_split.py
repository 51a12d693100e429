"""pa_chunk_attention_split (split-KV units and their merge, per new token)
against the fp64 oracle across partition sizes, including tokens that see
none of a partition's keys; one token per sequence reproduces the split
decode and its reduce bit for bit; results are deterministic."""
import numpy as np
import pytest
import torch

import paged_kv_decode_pa_amd as pa
from tests.gpu_helpers import (DEV, TOL, DeviceWorkload, bits_of, config_device, config_workload,
                               max_err, say, to_dev)
from tests.test_gpu_chunk import CASES, chunk_reference
from workloads import make_chunk_queries, make_custom_workload

pytestmark = pytest.mark.gpu


def run_split(dev, query, query_start, partition_size, max_q=None):
    wl = dev.wl
    q = to_dev(query, wl.dtype)
    qs = torch.from_numpy(np.asarray(query_start, dtype=np.int32)).to(DEV)
    T, Hq, D = q.shape
    P = max(1, -(-int(wl.context_lens.max()) // partition_size))
    po = torch.full((T, Hq, P, D), float("nan"), dtype=torch.float32, device=DEV)
    pm = torch.full((T, Hq, P), float("nan"), dtype=torch.float32, device=DEV)
    psum = torch.full((T, Hq, P), float("nan"), dtype=torch.float32, device=DEV)
    out = torch.full_like(q, float("nan"))
    mq = int(np.diff(np.asarray(query_start)).max()) if max_q is None else max_q
    pa.pa_chunk_attention_split(out, q, dev.k_cache, dev.v_cache, dev.block_tables,
                                dev.context_lens, qs, mq, wl.scale, partition_size, po, pm, psum)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("ps", [16, 64, 512])
@pytest.mark.parametrize("lens,q_lens,Hq,Hkv,D", CASES)
def test_split_matches_oracle(lens, q_lens, Hq, Hkv, D, ps):
    say(f"[chunk split] {lens} q {q_lens} {Hq}/{Hkv}/{D} partition {ps}")
    wl = make_custom_workload(lens, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                              seed=sum(lens) + Hq)
    query, qs = make_chunk_queries(wl, q_lens, seed=len(lens) + D)
    ref = chunk_reference(wl, query, qs)
    dev = DeviceWorkload(wl)
    got = run_split(dev, query, qs, ps)
    err = max_err(got, ref)
    say(f"    max abs err {err:.3e}")
    assert err <= TOL["bf16"]
    assert np.array_equal(bits_of(run_split(dev, query, qs, ps)), bits_of(got))  # deterministic


@pytest.mark.parametrize("cid,ps", [(2, 512), (2, 768), (5, 256), (4, 512)])
def test_one_token_per_sequence_is_split_decode(cid, ps):
    say(f"[chunk split] q_len = 1 equals split decode + reduce, config {cid}")
    dev = config_device(cid)
    wl = dev.wl
    qs = np.arange(wl.num_seqs + 1, dtype=np.int32)
    got = run_split(dev, wl.query, qs, ps)
    assert np.array_equal(bits_of(got), bits_of(dev.decode(ps)))


@pytest.mark.parametrize("q,ps", [(2, 512), (4, 512), (8, 512), (1, 768), (2, 768), (4, 768),
                                  (8, 768)])
def test_draft_verification_at_config_2_shape(q, ps):
    """q new tokens for each of config 2's 64 sequences; 768-token partitions
    are the split form's benchmarked size at this shape
    (bench.py --chunk Q --chunk-partition 768)."""
    say(f"[chunk split] config 2 shape, {q} new tokens per sequence, partition {ps}")
    wl = config_workload(2)
    query, qs = make_chunk_queries(wl, [q] * wl.num_seqs, seed=q)
    dev = config_device(2)
    got = run_split(dev, query, qs, ps)
    assert max_err(got, chunk_reference(wl, query, qs)) <= TOL["bf16"]


def test_tokens_that_precede_a_partition():
    """Contexts just past a partition boundary: the earlier new tokens see no
    key of the last partition (empty partials, weight 0 in the merge)."""
    say("[chunk split] tokens before the last partition")
    lens = [513, 514, 1025, 520, 64]
    q_lens = [4, 8, 6, 16, 3]
    wl = make_custom_workload(lens, num_q_heads=8, num_kv_heads=2, head_dim=128, seed=77)
    query, qs = make_chunk_queries(wl, q_lens, seed=78)
    dev = DeviceWorkload(wl)
    got = run_split(dev, query, qs, 512)
    assert max_err(got, chunk_reference(wl, query, qs)) <= TOL["bf16"]


def test_split_beyond_planned_batch_size():
    """More than 1024 sequences: the split kernel's plain grid (no unit plan,
    cached loads throughout)."""
    say("[chunk split] 1100-sequence batch")
    rng = np.random.default_rng(15)
    lens = rng.integers(1, 80, size=1100)
    q_lens = [int(rng.integers(0, min(int(L), 3) + 1)) for L in lens]
    wl = make_custom_workload(lens.tolist(), num_q_heads=8, num_kv_heads=1, head_dim=128, seed=16)
    query, qs = make_chunk_queries(wl, q_lens, seed=17)
    ref = chunk_reference(wl, query, qs)
    dev = DeviceWorkload(wl)
    for ps in (16, 32):
        assert max_err(run_split(dev, query, qs, ps), ref) <= TOL["bf16"], ps


@pytest.mark.parametrize("B", [48, 200])
def test_split_with_scattered_prefix_sharing(B):
    """Sequences sharing prefix pages anywhere in the batch: those stream their
    pages through the caches, the others with the nontemporal hint; shared and
    private copies of the same values give identical bits, and match the
    oracle."""
    say(f"[chunk split] scattered prefix sharing, batch {B}")
    rng = np.random.default_rng(B + 1)
    group_of = np.where(rng.random(B) < 0.4, rng.integers(0, 5, B), -1)
    prefix = 64
    lens = np.where(group_of >= 0, rng.integers(prefix + 4, 400, B), rng.integers(4, 400, B))
    q_lens = rng.integers(1, 4, B).tolist()
    kw = dict(num_q_heads=8, num_kv_heads=2, head_dim=128, seed=B, prefix_tokens=prefix,
              group_of=group_of.tolist())
    shared = make_custom_workload(lens.tolist(), **kw)
    private = make_custom_workload(lens.tolist(), share_prefix=False, **kw)
    query, qs = make_chunk_queries(shared, q_lens, seed=B)
    ref = chunk_reference(shared, query, qs)
    ds, dp = DeviceWorkload(shared), DeviceWorkload(private)
    for ps in (64, 256):
        a = run_split(ds, query, qs, ps)
        assert np.array_equal(bits_of(a), bits_of(run_split(dp, query, qs, ps))), ps
        assert max_err(a, ref) <= TOL["bf16"], ps
