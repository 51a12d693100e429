"""pa_decode (+ pa_decode_reduce) against the fp64 oracle, element by element.

Tolerances: 2e-2 max-abs for bf16 K/V with fp32 accumulation, 1e-5 for the
fp32 workload.  Structural properties that the loose bf16 tolerance could
hide are checked bit for bit on the GPU: repeatability, independence from
physical page placement and from prefix sharing, and one-token contexts.
"""
import math

import numpy as np
import pytest
import torch

from tests.gpu_helpers import (TOL, DeviceWorkload, bits_of, config_device, config_reference,
                               config_workload, f64_of, max_err, oracle_reference, parity_report,
                               report_line, say)
from workloads import config_by_id, make_custom_workload, make_workload

pytestmark = pytest.mark.gpu

KERNELS = ["auto", "valu"]


def _splits(cid):
    cfg = config_by_id(cid)
    s = {0, 512, cfg.bench_partition_size} | ({256, 1024} if cid > 1 else set())
    if cid == 2:
        s.add(768)  # the split partition size that single pass replaced in the benchmark
    return sorted(s)


CONFIG_CASES = [(cid, ps, kern) for cid in (1, 2, 3, 4, 5) for ps in _splits(cid)
                for kern in KERNELS if not (cid == 1 and kern == "valu")]


@pytest.mark.parametrize("cid,ps,kernel", CONFIG_CASES,
                         ids=[f"cfg{c}-ps{p}-{k}" for c, p, k in CONFIG_CASES])
def test_config_matches_oracle(cid, ps, kernel):
    say(f"[decode] config {cid} partition {ps} kernel {kernel}")
    wl = config_workload(cid)
    ref = config_reference(cid)
    dev = config_device(cid)
    out = dev.decode(ps, kernel)
    rep = parity_report(out, ref)
    say("    " + report_line(rep))
    assert rep["max_abs"] <= TOL[wl.dtype]


@pytest.mark.parametrize("cid", [2, 5])
def test_repeat_runs_bit_identical(cid):
    say(f"[decode] determinism config {cid}")
    dev = config_device(cid)
    ps = config_by_id(cid).bench_partition_size or 768
    a = bits_of(dev.decode(ps))
    b = bits_of(dev.decode(ps))
    c = bits_of(dev.decode(0))
    d = bits_of(dev.decode(0))
    assert np.array_equal(a, b) and np.array_equal(c, d)


@pytest.mark.parametrize("kernel", KERNELS)
def test_page_placement_does_not_change_bits(kernel):
    say(f"[decode] placement invariance {kernel}")
    lens = [1, 15, 16, 17, 200, 513, 1000, 33]
    a = make_custom_workload(lens, num_q_heads=32, num_kv_heads=8, head_dim=128, seed=12)
    b = make_custom_workload(lens, num_q_heads=32, num_kv_heads=8, head_dim=128, seed=12,
                             placement_seed=77)
    assert not np.array_equal(a.block_tables, b.block_tables)
    da, db = DeviceWorkload(a), DeviceWorkload(b)
    for ps in (0, 256):
        assert np.array_equal(bits_of(da.decode(ps, kernel)), bits_of(db.decode(ps, kernel)))


def test_prefix_sharing_does_not_change_bits():
    say("[decode] shared vs unshared prefix (config 3)")
    cfg = config_by_id(3)
    shared = config_device(3)
    unshared = DeviceWorkload(make_workload(cfg, share_prefix=False))
    for ps in (0, cfg.bench_partition_size):
        assert np.array_equal(bits_of(shared.decode(ps)), bits_of(unshared.decode(ps)))


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
@pytest.mark.parametrize("kernel", KERNELS)
def test_single_token_context_returns_v_exactly(dtype, D, kernel):
    say(f"[decode] L=1 {dtype} D={D} {kernel}")
    wl = make_custom_workload([1, 1, 1, 1], num_q_heads=8, num_kv_heads=2, head_dim=D,
                              dtype=dtype, seed=4)
    dev = DeviceWorkload(wl)
    for ps in (0, 16):
        out = bits_of(dev.decode(ps, kernel))
        want = np.repeat(wl.new_value, 4, axis=1)  # head h reads kv head h // 4
        assert np.array_equal(out, want)


@pytest.mark.parametrize(
    "lens,Hq,Hkv,D,dtype",
    [
        ([17, 64, 100, 255, 1, 15, 16, 31, 32, 33], 8, 2, 64, "f32"),
        ([17, 64, 100, 255, 1, 15, 16, 31, 32, 33], 8, 2, 128, "f32"),
        ([17, 64, 100, 255, 1, 15, 16, 31, 32, 33], 8, 2, 64, "bf16"),
        ([700, 3, 48, 129], 16, 1, 128, "bf16"),     # group of 16 fills the tile
        ([700, 3, 48, 129], 4, 4, 128, "bf16"),      # no grouping
        ([700, 3, 48, 129], 12, 4, 128, "bf16"),     # group of 3
        ([700, 3, 48, 129], 16, 1, 64, "f32"),
        ([700, 3, 48, 129], 12, 2, 128, "f32"),      # group of 6
        ([700, 3, 48, 129], 24, 2, 64, "bf16"),      # group of 12
        ([5000, 4097, 2], 8, 1, 128, "bf16"),        # more than 64 pages per wave
    ],
)
@pytest.mark.parametrize("kernel", KERNELS)
def test_shapes_and_ragged_tails(lens, Hq, Hkv, D, dtype, kernel):
    say(f"[decode] shapes {lens} {Hq}/{Hkv}/{D} {dtype} {kernel}")
    wl = make_custom_workload(lens, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, dtype=dtype,
                              seed=len(lens) + Hq + D)
    ref = oracle_reference(wl)
    dev = DeviceWorkload(wl)
    for ps in (0, 16, 48, 512):
        err = max_err(dev.decode(ps, kernel), ref)
        assert err <= TOL[dtype], (ps, err)


def _needle_fn(position, strength):
    def fn(q, k, v, owners, lengths):
        q[:] = 0.0
        q[:, :, 0] = 1.0
        k[:, :, 0] = np.clip(k[:, :, 0], -1.0, 1.0)
        for i, (key, pos) in enumerate(owners):
            if pos == position:
                k[i, :, 0] = strength
        return q, k, v
    return fn


@pytest.mark.parametrize("position", [0, 15, 16, 255, 256, 511, 512, 1000])
@pytest.mark.parametrize("kernel", KERNELS)
def test_needle_at_page_and_partition_boundaries(position, kernel):
    say(f"[decode] needle at {position} {kernel}")
    D = 128
    wl = make_custom_workload([1001, 1001], num_q_heads=8, num_kv_heads=2, head_dim=D,
                              seed=position, value_fn=_needle_fn(position, 60.0 * math.sqrt(D)))
    ref = oracle_reference(wl)
    dev = DeviceWorkload(wl)
    for ps in (0, 256, 512):
        out = dev.decode(ps, kernel)
        assert max_err(out, ref) <= TOL["bf16"], ps


@pytest.mark.parametrize("kernel", KERNELS)
def test_sharp_softmax_with_jumping_max(kernel):
    """q scaled x50: scores reach a few hundred, far past fp32 exp overflow,
    and the running max jumps many times along each context."""
    say(f"[decode] sharp softmax {kernel}")

    def fn(q, k, v, owners, lengths):
        for i, (key, pos) in enumerate(owners):
            k[i] *= 1.0 + pos / 400.0           # later keys tend to score higher
        return q * 50.0, k, v

    wl = make_custom_workload([900, 333, 64, 17], num_q_heads=32, num_kv_heads=8, head_dim=128,
                              seed=5, value_fn=fn)
    ref = oracle_reference(wl)
    dev = DeviceWorkload(wl)
    for ps in (0, 128):
        assert max_err(dev.decode(ps, kernel), ref) <= TOL["bf16"], ps


@pytest.mark.parametrize("kernel", KERNELS)
def test_empty_context_gives_zeros(kernel):
    say(f"[decode] L=0 {kernel}")
    wl = make_custom_workload([40, 17], num_q_heads=8, num_kv_heads=2, head_dim=128, seed=9)
    dev = DeviceWorkload(wl)
    dev.context_lens[1] = 0
    ref = oracle_reference(wl)
    for ps in (0, 32):
        out = f64_of(dev.decode(ps, kernel))
        assert (out[1] == 0).all()
        assert np.abs(out[0] - ref[0]).max() <= TOL["bf16"]


def test_matrix_core_and_vector_kernels_agree():
    say("[decode] mfma vs valu on config 2")
    dev = config_device(2)
    a = f64_of(dev.decode(256, "auto"))
    b = f64_of(dev.decode(256, "valu"))
    assert np.abs(a - b).max() <= 2 * TOL["bf16"]


@pytest.mark.parametrize("kernel", KERNELS)
def test_long_partitions_rotate_page_ids(kernel):
    """2048-token partitions: one wave walks 128 pages and refreshes its page ids."""
    say(f"[decode] 2048-token partitions {kernel}")
    wl = make_custom_workload([5000, 2048, 4111, 17], num_q_heads=16, num_kv_heads=2, head_dim=128,
                              seed=31)
    ref = oracle_reference(wl)
    dev = DeviceWorkload(wl)
    for ps in (2048, 4096):
        assert max_err(dev.decode(ps, kernel), ref) <= TOL["bf16"], ps


def test_split_plan_with_empty_and_ragged_contexts():
    """Zero-length contexts, one-page contexts and full partitions in one batch:
    every partition that holds tokens is computed exactly once."""
    say("[decode] split plan, ragged batch with empty contexts")
    lens = [0, 1, 256, 257, 0, 512, 31, 4096, 255, 16, 0, 1000]
    wl = make_custom_workload([max(x, 1) for x in lens], num_q_heads=8, num_kv_heads=2,
                              head_dim=128, seed=77)
    dev = DeviceWorkload(wl)
    for b, L in enumerate(lens):
        if L == 0:
            dev.context_lens[b] = 0
    ref = oracle_reference(wl)
    for ps in (16, 256, 512):
        out = f64_of(dev.decode(ps))
        for b, L in enumerate(lens):
            if L == 0:
                assert (out[b] == 0).all(), (ps, b)
            else:
                assert np.abs(out[b] - ref[b]).max() <= TOL["bf16"], (ps, b)


@pytest.mark.parametrize("kernel", KERNELS)
def test_split_beyond_planned_batch_size(kernel):
    """More than 1024 sequences: the split kernels fall back to the plain grid
    and the single passes to batch order."""
    say(f"[decode] 1100-sequence batch {kernel}")
    rng = np.random.default_rng(5)
    lens = rng.integers(1, 80, size=1100).tolist()
    wl = make_custom_workload(lens, num_q_heads=8, num_kv_heads=1, head_dim=128, seed=6)
    ref = oracle_reference(wl)
    dev = DeviceWorkload(wl)
    for ps in (0, 32):
        assert max_err(dev.decode(ps, kernel), ref) <= TOL["bf16"], ps


@pytest.mark.parametrize("n", [300, 1100])
def test_fp32_batches_in_length_order_and_past_the_plan(n):
    """fp32 (the vector kernel): a single pass with more units than compute
    units takes the length order; split partitions take the unit plan up to
    1024 sequences and the plain grid past it."""
    say(f"[decode] fp32 batch of {n}")
    rng = np.random.default_rng(n)
    lens = rng.integers(1, 300, size=n).tolist()
    wl = make_custom_workload(lens, num_q_heads=8, num_kv_heads=2, head_dim=64, dtype="f32",
                              seed=n)
    ref = oracle_reference(wl)
    dev = DeviceWorkload(wl)
    for ps in (0, 64):
        assert max_err(dev.decode(ps), ref) <= TOL["f32"], ps


@pytest.mark.parametrize("B", [48, 200, 300])
def test_scattered_prefix_sharing(B):
    """Sequences that share prefix pages sit anywhere in the batch, in each
    batch-size bucket of the device-side plan (up to 64, 256 and 1024
    sequences).  Sequences that share their first page are read through the
    caches and the others stream with the nontemporal hint; shared and private
    copies give identical bits, and both match the oracle."""
    say(f"[decode] scattered prefix sharing, batch {B}")
    rng = np.random.default_rng(B)
    group_of = np.where(rng.random(B) < 0.4, rng.integers(0, 5, B), -1)
    prefix = 64
    lens = np.where(group_of >= 0, rng.integers(prefix + 1, 400, B), rng.integers(1, 400, B))
    kw = dict(num_q_heads=8, num_kv_heads=2, head_dim=128, seed=B, prefix_tokens=prefix,
              group_of=group_of.tolist())
    shared = make_custom_workload(lens.tolist(), **kw)
    private = make_custom_workload(lens.tolist(), share_prefix=False, **kw)
    firsts = shared.block_tables[:, 0]
    assert len(np.unique(firsts)) < B  # some first pages are shared ...
    assert len(np.unique(private.block_tables[:, 0])) == B  # ... and none here
    ref = oracle_reference(shared)
    ds, dp = DeviceWorkload(shared), DeviceWorkload(private)
    for ps in (0, 64, 256):
        a = ds.decode(ps)
        assert np.array_equal(bits_of(a), bits_of(dp.decode(ps))), ps
        assert max_err(a, ref) <= TOL["bf16"], ps
