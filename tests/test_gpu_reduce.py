"""pa_decode_reduce on its own, fed the oracle's fp64 split-KV partials
(rounded to fp32), against the oracle's unsplit output."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_pa_amd as pa
from tests.gpu_helpers import DEV, TOL, f64_of, say, tdtype
from tests.oracle_pins import fill_pools
from workloads import make_custom_workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ps", [16, 64, 512])
def test_reduce_of_oracle_partials(dtype, ps):
    say(f"[reduce] {dtype} partition {ps}")
    lens = [1, 16, 17, 511, 512, 513, 1024, 1040, 3000]  # 64 and 65 partitions of 16
    wl = make_custom_workload(lens, num_q_heads=8, num_kv_heads=2, head_dim=128, dtype=dtype,
                              seed=ps)
    k, v = fill_pools(oracle, wl)
    full = oracle.decode(wl.query, k, v, wl.block_tables, wl.context_lens, wl.scale, 16, dtype)
    n = -(-max(lens) // ps)
    po, pm, psum = oracle.decode_partials(wl.query, k, v, wl.block_tables, wl.context_lens,
                                          wl.scale, 16, dtype, ps, n)
    out = torch.empty((len(lens), 8, 128), dtype=tdtype(dtype), device=DEV)
    f32 = lambda a: torch.from_numpy(a.astype(np.float32)).to(DEV)
    pa.pa_decode_reduce(out, f32(po), f32(pm), f32(psum),
                        torch.from_numpy(wl.context_lens).to(DEV), ps)
    torch.cuda.synchronize()
    err = np.abs(f64_of(out) - full).max()
    say(f"    max abs err {err:.3e}")
    assert err <= TOL[dtype]


def test_single_partition_is_identity_and_zero_length_is_zero():
    say("[reduce] identity / empty")
    rng = np.random.default_rng(1)
    B, Hq, D, n = 3, 4, 64, 5
    po = rng.standard_normal((B, Hq, n, D)).astype(np.float32)
    pm = rng.standard_normal((B, Hq, n)).astype(np.float32) * 10
    psum = rng.uniform(1, 50, (B, Hq, n)).astype(np.float32)
    lens = np.array([100, 0, 64], dtype=np.int32)           # partition 128: 1, 0, 1 partitions
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    t = lambda a: torch.from_numpy(a).to(DEV)
    pa.pa_decode_reduce(out, t(po), t(pm), t(psum), t(lens), 128)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got[1], np.zeros((Hq, D), np.float32))
    # one partition: w = l * exp(0) = l and out = l * o / l, within one rounding
    for b in (0, 2):
        assert np.allclose(got[b], po[b, :, 0], rtol=3e-7, atol=0)


def test_partitions_past_max_are_ignored():
    say("[reduce] clamp to max_num_partitions")
    B, Hq, D, n = 1, 2, 64, 2
    po = np.stack([np.full((Hq, D), 1.0), np.full((Hq, D), 3.0)], axis=1)[None].astype(np.float32)
    pm = np.zeros((B, Hq, n), np.float32)
    psum = np.ones((B, Hq, n), np.float32)
    lens = np.array([16 * 100], dtype=np.int32)             # 100 partitions of 16, only 2 stored
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    pa.pa_decode_reduce(out, t(po), t(pm), t(psum), t(lens), 16)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), np.full((B, Hq, D), 2.0, np.float32))
