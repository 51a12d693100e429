"""pa_export_pages / pa_import_pages against the oracle, bit for bit, and the
hand-off property that matters: a batch moved into another pool at other
page ids decodes to the same bits."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_pa_amd as pa
from tests.gpu_helpers import DEV, DeviceWorkload, bits_of, config_device, say, tdtype, to_dev
from tests.oracle_pins import fill_pools, nan_pools
from workloads import make_custom_workload

pytestmark = pytest.mark.gpu


def seq_page_ids(wl, seqs):
    ids = [wl.block_tables[b, :-(-int(wl.context_lens[b]) // 16)] for b in seqs]
    return np.concatenate(ids).astype(np.int32)


def export_dev(dev, ids, prior=None):
    wl = dev.wl
    block = wl.num_kv_heads * 16 * wl.head_dim
    if prior is None:
        buf = torch.empty((2, len(ids), block), dtype=tdtype(wl.dtype), device=DEV)
    else:
        buf = to_dev(prior, wl.dtype).reshape(2, len(ids), block).contiguous()
    pa.pa_export_pages(buf, dev.k_cache, dev.v_cache, torch.from_numpy(ids).to(DEV))
    torch.cuda.synchronize()
    return buf


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_export_matches_oracle(dtype):
    say(f"[transfer] export, {dtype}")
    lens = [1, 16, 17, 300, 1000, 33]
    wl = make_custom_workload(lens, num_q_heads=8, num_kv_heads=4, head_dim=128, dtype=dtype,
                              seed=81)
    dev = DeviceWorkload(wl)
    ids = seq_page_ids(wl, [3, 0, 2, 5])
    ids = np.concatenate([ids, [-1, int(wl.num_pages), int(ids[0])]]).astype(np.int32)
    block = wl.num_kv_heads * 16 * wl.head_dim
    sentinel = 0x1234 if dtype == "bf16" else np.float32(3.25)
    store = np.uint16 if dtype == "bf16" else np.float32
    prior = np.full((2, len(ids), block), sentinel, dtype=store)
    got = bits_of(export_dev(dev, ids, prior))
    k, v = fill_pools(oracle, wl)
    want = oracle.export_pages(k, v, ids, prior)
    assert got.shape == want.shape
    assert np.array_equal(got.view(np.uint8), want.view(np.uint8))  # NaN poison included


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_import_matches_oracle_on_the_whole_pool(dtype):
    say(f"[transfer] import, {dtype}")
    num_pages, Hkv, D = 300, 8, 64
    rng = np.random.default_rng(82)
    ids = rng.permutation(num_pages)[:120].astype(np.int32)
    ids[[5, 77]] = [-3, num_pages + 4]  # skipped
    block = Hkv * 16 * D
    if dtype == "bf16":
        buf = rng.integers(0, 0x7F00, size=(2, len(ids), block), dtype=np.uint16)
    else:
        buf = rng.standard_normal((2, len(ids), block)).astype(np.float32)
    k0, v0 = nan_pools(num_pages, Hkv, 16, D, dtype)
    kd, vd = to_dev(k0, dtype), to_dev(v0, dtype)
    pa.pa_import_pages(to_dev(buf, dtype), kd, vd, torch.from_numpy(ids).to(DEV))
    torch.cuda.synchronize()
    k, v = oracle.import_pages(k0, v0, buf, ids)
    assert np.array_equal(bits_of(kd).view(np.uint8), k.view(np.uint8))
    assert np.array_equal(bits_of(vd).view(np.uint8), v.view(np.uint8))


@pytest.mark.parametrize("cid", [2, 3])
def test_handoff_decodes_to_the_same_bits(cid):
    """Every page of the batch exported, imported into a pool of another size
    at permuted page ids (config 3: its shared prefix pages once), block
    tables remapped: single-pass and split-KV decode give identical bits."""
    say(f"[transfer] hand-off, config {cid}")
    src = config_device(cid)
    wl = src.wl
    used = np.unique(seq_page_ids(wl, range(wl.num_seqs)))
    buf = export_dev(src, used.astype(np.int32))
    dest_pages = len(used) + 1000
    new_of = np.random.default_rng(83 + cid).permutation(dest_pages)[:len(used)].astype(np.int32)
    dst = DeviceWorkload(wl, fill=False)
    dst.k_cache = torch.full((dest_pages, wl.num_kv_heads, 16, wl.head_dim), float("nan"),
                             dtype=tdtype(wl.dtype), device=DEV)
    dst.v_cache = torch.full((dest_pages, wl.num_kv_heads, wl.head_dim, 16), float("nan"),
                             dtype=tdtype(wl.dtype), device=DEV)
    pa.pa_import_pages(buf, dst.k_cache, dst.v_cache, torch.from_numpy(new_of).to(DEV))
    remap = np.full(int(wl.num_pages), -1, dtype=np.int64)
    remap[used] = new_of
    tables = np.where(wl.block_tables >= 0, remap[np.maximum(wl.block_tables, 0)], -1)
    dst.block_tables = torch.from_numpy(tables.astype(np.int32)).to(DEV)
    torch.cuda.synchronize()
    for ps in (0, 512):
        assert np.array_equal(bits_of(dst.decode(ps)), bits_of(src.decode(ps))), ps


def test_empty_and_shape_checks():
    say("[transfer] empty call and binding checks")
    k = torch.zeros((4, 2, 16, 64), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros((4, 2, 64, 16), dtype=torch.bfloat16, device=DEV)
    buf = torch.zeros((2, 0, 2 * 16 * 64), dtype=torch.bfloat16, device=DEV)
    ids = torch.zeros((0,), dtype=torch.int32, device=DEV)
    pa.pa_export_pages(buf, k, v, ids)
    pa.pa_import_pages(buf, k, v, ids)
    short = torch.zeros((2, 1, 2 * 16 * 64 - 8), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(pa.PaError):
        pa.pa_export_pages(short, k, v, torch.zeros((1,), dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert not k.any() and not v.any()
