"""pa_decode_cascade: shared prefix partitions read once per group and the
split-KV units of each sequence's own partitions, in one launch, merged by
pa_decode_reduce.  Checked against the oracle, against the plain split
decode, for determinism, with the step's token written in the same call, and
with groups that span several column groups or hold out-of-range members."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_pa_amd as pa
from tests.gpu_helpers import (DEV, TOL, DeviceWorkload, bits_of, config_workload, f64_of,
                               oracle_reference, parity_report, report_line, say, tdtype)
from workloads import config_by_id, make_custom_workload

pytestmark = pytest.mark.gpu


def dev_groups(g):
    out = dict(g)
    for k in ("group_start", "group_seqs", "group_partitions", "seq_first_partition"):
        out[k] = torch.from_numpy(np.ascontiguousarray(g[k], dtype=np.int32)).to(DEV)
    return out


def cascade(dev, ps, groups, append=False):
    wl = dev.wl
    B, Hq, D = wl.num_seqs, wl.num_q_heads, wl.head_dim
    n = dev.partition_count(ps)
    po = torch.full((B, Hq, n, D), float("nan"), dtype=torch.float32, device=DEV)
    pm = torch.full((B, Hq, n), float("nan"), dtype=torch.float32, device=DEV)
    psum = torch.full((B, Hq, n), float("nan"), dtype=torch.float32, device=DEV)
    extra = dict(key=dev.new_key, value=dev.new_value, slot_mapping=dev.new_slots) if append else {}
    pa.pa_decode_cascade(dev.query, dev.k_cache, dev.v_cache, dev.block_tables, dev.context_lens,
                         wl.scale, ps, po, pm, psum, dev_groups(groups), **extra)
    out = torch.empty((B, Hq, D), dtype=tdtype(wl.dtype), device=DEV)
    pa.pa_decode_reduce(out, po, pm, psum, dev.context_lens, ps)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("ps", sorted({256, 512, 1024, config_by_id(3).cascade_partition_size}))
def test_prefix_reuse_workload(ps):
    say(f"[cascade] prefix-reuse batch, partition {ps}")
    wl = config_workload(3)
    groups = pa.prefix_groups(wl.block_tables, wl.context_lens, ps // 16)
    assert groups["num_groups"] == 8 and groups["max_group_size"] == 16
    dev = DeviceWorkload(wl)
    got = cascade(dev, ps, groups)
    ref = oracle_reference(wl)
    err = float(np.abs(f64_of(got) - ref).max())
    say(f"    max abs err {err:.3e}; groups {groups['num_groups']}, partitions "
        f"{groups['max_group_partitions']}")
    assert err <= TOL["bf16"]
    plain = f64_of(dev.decode(ps))
    assert float(np.abs(f64_of(got) - plain).max()) <= TOL["bf16"]
    assert np.array_equal(bits_of(cascade(dev, ps, groups)), bits_of(got))  # deterministic


@pytest.mark.parametrize("ps", sorted({512, config_by_id(3).cascade_partition_size}))
def test_step_token_written_in_the_same_call(ps):
    """At the benchmarked 2048-token partitions too: pool and output bit for
    bit against the cascade on a pool that already holds the token, and the
    output against the oracle."""
    say(f"[cascade] with the step's token, partition {ps}")
    wl = config_workload(3)
    groups = pa.prefix_groups(wl.block_tables, wl.context_lens, ps // 16)
    ref_dev = DeviceWorkload(wl)
    dev = DeviceWorkload(wl, fill=False)
    dev.prefill()
    got = cascade(dev, ps, groups, append=True)
    assert np.array_equal(bits_of(dev.k_cache), bits_of(ref_dev.k_cache))
    assert np.array_equal(bits_of(dev.v_cache), bits_of(ref_dev.v_cache))
    assert np.array_equal(bits_of(got), bits_of(cascade(ref_dev, ps, groups)))
    rep = parity_report(got, oracle_reference(wl))
    say("    " + report_line(rep))
    assert rep["max_abs"] <= TOL["bf16"]


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (16, 2, 64), (8, 8, 128)])
def test_scattered_groups_and_wide_groups(Hq, Hkv, D):
    """Three groups (one of 20 members: more columns than one wave carries
    at a group of 4), members scattered through the batch, and sequences in
    no group."""
    say(f"[cascade] scattered groups {Hq}/{Hkv}/{D}")
    rng = np.random.default_rng(7)
    B = 40
    group_of = np.full(B, -1)
    idx = rng.permutation(B)
    group_of[idx[:20]] = 0
    group_of[idx[20:26]] = 1
    group_of[idx[26:29]] = 2
    lens = (300 + rng.integers(1, 200, B)).tolist()
    wl = make_custom_workload(lens, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, seed=8,
                              group_of=group_of.tolist(), prefix_tokens=256)
    groups = pa.prefix_groups(wl.block_tables, wl.context_lens, 4)
    assert groups["num_groups"] == 3 and groups["max_group_size"] == 20
    dev = DeviceWorkload(wl)
    got = cascade(dev, 64, groups)
    assert float(np.abs(f64_of(got) - oracle_reference(wl)).max()) <= TOL["bf16"]


def test_no_groups_is_the_split_decode():
    say("[cascade] no groups")
    wl = config_workload(2)
    dev = DeviceWorkload(wl)
    empty = {"num_groups": 0, "max_group_size": 0, "max_group_partitions": 0,
             "group_start": np.zeros(1, np.int32), "group_seqs": np.zeros(1, np.int32),
             "group_partitions": np.zeros(1, np.int32),
             "seq_first_partition": np.zeros(wl.num_seqs, np.int32)}
    assert np.array_equal(bits_of(cascade(dev, 512, empty)), bits_of(dev.decode(512)))


def test_out_of_range_members_are_skipped():
    say("[cascade] out-of-range members")
    wl = config_workload(3)
    g = pa.prefix_groups(wl.block_tables, wl.context_lens, 32)
    want = cascade(DeviceWorkload(wl), 512, g)
    # append two bogus members to group 0 (indices outside the batch)
    s = g["group_start"].copy()
    seqs = np.insert(g["group_seqs"], s[1], [-5, wl.num_seqs + 3])
    s[1:] += 2
    bad = dict(g, group_start=s, group_seqs=seqs, max_group_size=g["max_group_size"] + 2)
    got = cascade(DeviceWorkload(wl), 512, bad)
    assert np.array_equal(bits_of(got), bits_of(want))


@pytest.mark.parametrize("ps", [256, 1024])
def test_suffix_grid_bound(ps):
    """The suffix units' grid counts each sequence's partitions from its
    first: the tight bound from prefix_groups, a looser one and none (0) give
    the same bits."""
    say(f"[cascade] suffix grid bound, partition {ps}")
    wl = config_workload(3)
    g = pa.prefix_groups(wl.block_tables, wl.context_lens, ps // 16)
    dev = DeviceWorkload(wl)
    tight = bits_of(cascade(dev, ps, g))
    assert g["max_suffix_partitions"] >= 1
    for bound in (0, g["max_suffix_partitions"] + 2):
        assert np.array_equal(bits_of(cascade(dev, ps, dict(g, max_suffix_partitions=bound))), tight)
    assert float(np.abs(f64_of(cascade(dev, ps, g)) - oracle_reference(wl)).max()) <= TOL["bf16"]


@pytest.mark.parametrize("seed", range(10))
def test_cascade_random(seed):
    """Seeded random batches: kv heads, group size, head dim, partition size,
    prefix length, groups scattered through the batch with sequences in none
    (some empty or one token long), with or without the step's token written
    in the call.  Against the oracle, and bit for bit against the same call on
    a pool that already holds the token."""
    rng = np.random.default_rng(4000 + seed)
    B = int(rng.integers(2, 40))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    D = int(rng.choice([64, 128]))
    pp = int(rng.choice([1, 2, 4, 8]))
    prefix_tokens = 16 * int(rng.integers(pp, 6 * pp + 1))
    n_groups = int(rng.integers(1, 4))
    group_of = rng.integers(-1, n_groups, B)
    lens = np.where(group_of >= 0, prefix_tokens + rng.integers(1, 200, B),
                    np.where(rng.random(B) < 0.2, rng.integers(0, 2, B), rng.integers(2, 600, B)))
    append = bool(rng.integers(2))
    say(f"[cascade random {seed}] B={B} {Hkv * G}/{Hkv}/{D} partition {16 * pp} prefix "
        f"{prefix_tokens} groups {n_groups} append {append}")
    wl = make_custom_workload([int(x) for x in lens], num_q_heads=Hkv * G, num_kv_heads=Hkv,
                              head_dim=D, seed=seed, group_of=group_of.tolist(),
                              prefix_tokens=prefix_tokens, placement_seed=seed + 5)
    groups = pa.prefix_groups(wl.block_tables, wl.context_lens, pp)
    ref_dev = DeviceWorkload(wl)
    want = cascade(ref_dev, 16 * pp, groups)
    assert float(np.abs(f64_of(want) - oracle_reference(wl)).max()) <= TOL["bf16"]
    if append:
        dev = DeviceWorkload(wl, fill=False)
        dev.prefill()
        got = cascade(dev, 16 * pp, groups, append=True)
        assert np.array_equal(bits_of(dev.k_cache), bits_of(ref_dev.k_cache))
        assert np.array_equal(bits_of(dev.v_cache), bits_of(ref_dev.v_cache))
        assert np.array_equal(bits_of(got), bits_of(want))


def test_graph_replays_of_the_cascade_step():
    """The shared-prefix step (with the token write) captured once in a HIP
    graph and replayed three times, eager work between: every replay equals
    the eager step bit for bit (the write is idempotent)."""
    say("[cascade] graph replay")
    wl = config_workload(3)
    g0 = pa.prefix_groups(wl.block_tables, wl.context_lens, 64)
    groups = dev_groups(g0)
    dev = DeviceWorkload(wl, fill=False)
    dev.prefill()
    B, Hq, D = wl.num_seqs, wl.num_q_heads, wl.head_dim
    n = dev.partition_count(1024)
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=DEV)
    po = torch.empty((B, Hq, n, D), dtype=torch.float32, device=DEV)
    pm = torch.empty((B, Hq, n), dtype=torch.float32, device=DEV)
    psum = torch.empty((B, Hq, n), dtype=torch.float32, device=DEV)

    def step():
        pa.pa_decode_cascade(dev.query, dev.k_cache, dev.v_cache, dev.block_tables,
                             dev.context_lens, wl.scale, 1024, po, pm, psum, groups,
                             key=dev.new_key, value=dev.new_value, slot_mapping=dev.new_slots)
        pa.pa_decode_reduce(out, po, pm, psum, dev.context_lens, 1024)

    step()
    torch.cuda.synchronize()
    want = bits_of(out)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        out.zero_()
        po.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(out), want)
