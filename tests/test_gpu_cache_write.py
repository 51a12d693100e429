"""pa_reshape_and_cache against the oracle's cache write, bit for bit, over
the whole pool (so a stray write anywhere fails)."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import DEV, DeviceWorkload, bits_of, config_workload, say, to_dev
from tests.oracle_pins import fill_pools, nan_pools
from workloads import make_custom_workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_pool_bits_match_oracle(cid):
    say(f"[cache_write] config {cid}")
    wl = config_workload(cid)
    dev = DeviceWorkload(wl)
    k, v = fill_pools(oracle, wl)
    assert np.array_equal(bits_of(dev.k_cache).view(np.uint8), k.view(np.uint8))
    assert np.array_equal(bits_of(dev.v_cache).view(np.uint8), v.view(np.uint8))


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
def test_negative_and_out_of_pool_slots_write_nothing(dtype, D):
    say(f"[cache_write] skipped slots {dtype} D={D}")
    rng = np.random.default_rng(3)
    num_pages, Hkv, T = 6, 3, 40
    slots = rng.choice(num_pages * 16, size=T, replace=False).astype(np.int64)
    slots[::7] = -1
    slots[5] = num_pages * 16 + 3       # beyond the pool: skipped by the kernel
    key = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    val = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    if dtype == "bf16":
        from workloads import bf16_bits_from_f32
        key, val = bf16_bits_from_f32(key), bf16_bits_from_f32(val)
    k0, v0 = nan_pools(num_pages, Hkv, 16, D, dtype)
    oslots = slots.copy()
    oslots[5] = -1                      # the oracle's reading of an out-of-pool slot
    k, v = oracle.cache_write(k0, v0, key, val, oslots, 16)
    kc = to_dev(k0, dtype)
    vc = to_dev(v0, dtype)
    import paged_kv_decode_pa_amd as pa
    pa.pa_reshape_and_cache(to_dev(key, dtype), to_dev(val, dtype), kc, vc,
                            torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(kc).view(np.uint8), k.view(np.uint8))
    assert np.array_equal(bits_of(vc).view(np.uint8), v.view(np.uint8))


def test_append_after_prefill_only_touches_new_slots():
    say("[cache_write] append")
    wl = make_custom_workload([33, 16, 1, 70], num_q_heads=8, num_kv_heads=4, head_dim=128, seed=8)
    dev = DeviceWorkload(wl, fill=False)
    dev.prefill()
    torch.cuda.synchronize()
    before_k, before_v = bits_of(dev.k_cache).copy(), bits_of(dev.v_cache).copy()
    dev.append()
    torch.cuda.synchronize()
    after_k, after_v = bits_of(dev.k_cache), bits_of(dev.v_cache)
    changed = np.argwhere((before_k != after_k).reshape(wl.num_pages, 4, 16, 128).any(axis=(1, 3)))
    want = sorted((int(s) // 16, int(s) % 16) for s in wl.new_slots)
    assert sorted(map(tuple, changed.tolist())) == want
    changed_v = np.argwhere((before_v != after_v).reshape(wl.num_pages, 4, 128, 16).any(axis=(1, 2)))
    assert sorted(map(tuple, changed_v.tolist())) == want
