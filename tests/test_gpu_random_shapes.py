"""Seeded random shapes through every device entry point against the oracle:
batch sizes, context lengths (with ragged tails, empty and one-token
contexts), head counts and groups, head dims, dtypes, partition sizes, pool
slack and placement, and chunk lengths, drawn per case from its seed.  The
structured tests pin the edge cases one by one; these cover the space in
between, at sizes the oracle finishes in seconds."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_pa_amd as pa
from tests.gpu_helpers import DEV, TOL, DeviceWorkload, bits_of, f64_of, say, tdtype, to_dev
from tests.oracle_pins import fill_pools
from workloads import make_chunk_queries, make_custom_workload

pytestmark = pytest.mark.gpu


def draw(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 24))
    kind = rng.random(B)
    lens = np.where(kind < 0.1, rng.integers(0, 2, B),            # empty or one token
                    np.where(kind < 0.4, rng.integers(2, 64, B), rng.integers(64, 1500, B)))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 3, 4, 6, 8, 16]))
    D = int(rng.choice([64, 128]))
    dtype = "f32" if rng.random() < 0.2 else "bf16"
    ps = int(rng.choice([0, 16, 64, 256, 512]))
    return rng, [int(x) for x in lens], Hkv * G, Hkv, D, dtype, ps


@pytest.mark.parametrize("seed", range(16))
def test_decode_and_fused_step_random(seed):
    rng, lens, Hq, Hkv, D, dtype, ps = draw(1000 + seed)
    say(f"[random {seed}] B={len(lens)} {Hq}/{Hkv}/{D} {dtype} partition {ps} "
        f"lens {min(lens)}..{max(lens)}")
    wl = make_custom_workload(lens, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, dtype=dtype,
                              seed=seed, pool_factor=float(rng.uniform(1.0, 2.0)),
                              placement_seed=seed + 7)
    k, v = fill_pools(oracle, wl)
    ref = oracle.decode(wl.query, k, v, wl.block_tables, wl.context_lens, wl.scale, 16, dtype)
    dev = DeviceWorkload(wl)
    got = dev.decode(ps)
    assert float(np.abs(f64_of(got) - ref).max()) <= TOL[dtype]
    # the one-call step on a pool without the appended tokens gives the same bits
    fused = DeviceWorkload(wl, fill=False)
    fused.prefill()
    B = len(lens)
    out = torch.empty((B, Hq, D), dtype=tdtype(dtype), device=DEV)
    if ps:
        n = fused.partition_count(ps)
        po = torch.empty((B, Hq, n, D), dtype=torch.float32, device=DEV)
        pm = torch.empty((B, Hq, n), dtype=torch.float32, device=DEV)
        psum = torch.empty((B, Hq, n), dtype=torch.float32, device=DEV)
        pa.pa_decode_append(None, fused.query, fused.new_key, fused.new_value, fused.new_slots,
                            fused.k_cache, fused.v_cache, fused.block_tables, fused.context_lens,
                            wl.scale, ps, po, pm, psum)
        pa.pa_decode_reduce(out, po, pm, psum, fused.context_lens, ps)
    else:
        pa.pa_decode_append(out, fused.query, fused.new_key, fused.new_value, fused.new_slots,
                            fused.k_cache, fused.v_cache, fused.block_tables, fused.context_lens,
                            wl.scale)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(out).view(np.uint8), bits_of(got).view(np.uint8))
    assert np.array_equal(bits_of(fused.k_cache).view(np.uint8), bits_of(dev.k_cache).view(np.uint8))


@pytest.mark.parametrize("seed", range(10))
def test_chunk_random(seed):
    rng, lens, Hq, Hkv, D, _, _ = draw(2000 + seed)
    lens = [max(x, 1) for x in lens]
    q_lens = [int(rng.integers(0, min(L, 40) + 1)) for L in lens]
    say(f"[random chunk {seed}] B={len(lens)} {Hq}/{Hkv}/{D} q {min(q_lens)}..{max(q_lens)}")
    wl = make_custom_workload(lens, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, seed=seed,
                              placement_seed=seed + 3)
    query, qs = make_chunk_queries(wl, q_lens, seed=seed)
    k, v = fill_pools(oracle, wl)
    ref = oracle.chunk_attention(query, k, v, wl.block_tables, wl.context_lens, qs, wl.scale, 16,
                                 "bf16")
    if int(qs[-1]) == 0:
        return
    dev = DeviceWorkload(wl)
    q = to_dev(query, "bf16")
    out = torch.full_like(q, float("nan"))
    pa.pa_chunk_attention(out, q, dev.k_cache, dev.v_cache, dev.block_tables, dev.context_lens,
                          torch.from_numpy(qs).to(DEV), max(max(q_lens), 1), wl.scale)
    torch.cuda.synchronize()
    assert float(np.abs(f64_of(out) - ref).max()) <= TOL["bf16"]


@pytest.mark.parametrize("seed", range(6))
def test_transfer_random(seed):
    rng, lens, Hq, Hkv, D, dtype, _ = draw(3000 + seed)
    say(f"[random transfer {seed}] {Hkv} kv heads, D={D}, {dtype}")
    wl = make_custom_workload([max(x, 1) for x in lens], num_q_heads=Hq, num_kv_heads=Hkv,
                              head_dim=D, dtype=dtype, seed=seed)
    dev = DeviceWorkload(wl)
    n = int(rng.integers(1, wl.num_pages + 1))
    ids = rng.integers(-2, wl.num_pages + 2, size=n).astype(np.int32)
    block = Hkv * 16 * D
    buf = torch.zeros((2, n, block), dtype=tdtype(dtype), device=DEV)
    pa.pa_export_pages(buf, dev.k_cache, dev.v_cache, torch.from_numpy(ids).to(DEV))
    torch.cuda.synchronize()
    k, v = fill_pools(oracle, wl)
    store = np.float32 if dtype == "f32" else np.uint16
    want = oracle.export_pages(k, v, ids, np.zeros((2, n, block), dtype=store))
    assert np.array_equal(bits_of(buf).view(np.uint8), want.view(np.uint8))
