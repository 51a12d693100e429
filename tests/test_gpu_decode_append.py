"""pa_decode_append (cache write inside the decode launch) against the two
calls it replaces, pa_reshape_and_cache then pa_decode: the whole pool and
every output bit for bit, split-KV and single pass, on all five workloads;
plus sequences whose slot is negative (nothing written) and the fp32 path
(two launches behind the one call)."""
import numpy as np
import pytest
import torch

import paged_kv_decode_pa_amd as pa
from tests.gpu_helpers import (DEV, TOL, DeviceWorkload, bits_of, config_reference,
                               config_workload, parity_report, report_line, say, tdtype)
from workloads import config_by_id, make_custom_workload

pytestmark = pytest.mark.gpu


def raw(t):
    """The tensor's bytes (fp32 NaN poison compares equal to itself)."""
    return bits_of(t).view(np.uint8)


def fused_step(dev, partition_size, slots=None):
    wl = dev.wl
    B, Hq, D = wl.num_seqs, wl.num_q_heads, wl.head_dim
    out = torch.empty((B, Hq, D), dtype=tdtype(wl.dtype), device=DEV)
    slots = dev.new_slots if slots is None else slots
    if partition_size == 0:
        pa.pa_decode_append(out, dev.query, dev.new_key, dev.new_value, slots, dev.k_cache,
                            dev.v_cache, dev.block_tables, dev.context_lens, wl.scale)
    else:
        n = dev.partition_count(partition_size)
        po = torch.full((B, Hq, n, D), float("nan"), dtype=torch.float32, device=DEV)
        pm = torch.full((B, Hq, n), float("nan"), dtype=torch.float32, device=DEV)
        ps = torch.full((B, Hq, n), float("nan"), dtype=torch.float32, device=DEV)
        pa.pa_decode_append(None, dev.query, dev.new_key, dev.new_value, slots, dev.k_cache,
                            dev.v_cache, dev.block_tables, dev.context_lens, wl.scale,
                            partition_size, po, pm, ps)
        pa.pa_decode_reduce(out, po, pm, ps, dev.context_lens, partition_size)
    torch.cuda.synchronize()
    return out


FUSED_CASES = [(cid, ps) for cid in (1, 2, 3, 4, 5)
               for ps in sorted({0, 256, config_by_id(cid).bench_partition_size})]


@pytest.mark.parametrize("cid,ps", FUSED_CASES, ids=[f"cfg{c}-ps{p}" for c, p in FUSED_CASES])
def test_fused_step_equals_write_then_decode(cid, ps):
    """At each workload's benchmarked partition too (768, 512 and 256 tokens
    for configs 2, 4 and 5): the whole pool and the output bit for bit
    against the two calls, and the output against the oracle."""
    say(f"[decode_append] config {cid}, partition {ps}")
    wl = config_workload(cid)
    ref = DeviceWorkload(wl)                    # prefill + pa_reshape_and_cache
    want = ref.decode(ps)
    dev = DeviceWorkload(wl, fill=False)
    dev.prefill()
    got = fused_step(dev, ps)
    assert np.array_equal(raw(dev.k_cache), raw(ref.k_cache))
    assert np.array_equal(raw(dev.v_cache), raw(ref.v_cache))
    assert np.array_equal(raw(got), raw(want))
    rep = parity_report(got, config_reference(cid))
    say("    " + report_line(rep))
    assert rep["max_abs"] <= TOL[wl.dtype]


@pytest.mark.parametrize("ps", [0, 64])
def test_negative_slots_write_nothing(ps):
    say(f"[decode_append] negative slots, partition {ps}")
    lens = [1, 17, 300, 64, 33]
    wl = make_custom_workload(lens, num_q_heads=8, num_kv_heads=2, head_dim=128, seed=91)
    skip = torch.tensor([True, False, True, False, False], device=DEV)
    a = DeviceWorkload(wl)                      # every new token already in the pool
    want_pool = (bits_of(a.k_cache), bits_of(a.v_cache))
    slots = torch.where(skip, torch.full_like(a.new_slots, -1), a.new_slots)
    # Rewriting the written tokens with other values must leave the skipped
    # sequences' slots as they were.
    a.new_key = torch.randn_like(a.new_key)
    a.new_value = torch.randn_like(a.new_value)
    fused_step(a, ps, slots)
    k, v = bits_of(a.k_cache), bits_of(a.v_cache)
    s = a.new_slots.cpu().numpy()
    for b in range(len(lens)):
        page, off = s[b] // 16, s[b] % 16
        same = bool(skip[b])
        assert np.array_equal(k[page, :, off, :], want_pool[0][page, :, off, :]) == same
        assert np.array_equal(v[page, :, :, off], want_pool[1][page, :, :, off]) == same
    # every other slot untouched
    mask = np.ones(k.shape[0] * 16, dtype=bool)
    mask[s] = False
    kk = k.transpose(0, 2, 1, 3).reshape(-1, *k.shape[1:2], k.shape[3])
    wk = want_pool[0].transpose(0, 2, 1, 3).reshape(kk.shape)
    assert np.array_equal(kk[mask], wk[mask])


def test_fp32_runs_write_then_decode():
    say("[decode_append] fp32")
    wl = config_workload(1)
    ref = DeviceWorkload(wl)
    want = ref.decode(0)
    dev = DeviceWorkload(wl, fill=False)
    dev.prefill()
    got = fused_step(dev, 0)
    assert np.array_equal(raw(dev.k_cache), raw(ref.k_cache))
    assert np.array_equal(raw(got), raw(want))


def test_graph_replays_of_the_fused_step():
    """Captured once, replayed several times with eager work between: every
    replay equals the eager fused step (the write is idempotent)."""
    say("[decode_append] graph replay")
    wl = config_workload(2)
    dev = DeviceWorkload(wl, fill=False)
    dev.prefill()
    want = bits_of(fused_step(dev, 512))
    B, Hq, D = wl.num_seqs, wl.num_q_heads, wl.head_dim
    n = dev.partition_count(512)
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=DEV)
    po = torch.empty((B, Hq, n, D), dtype=torch.float32, device=DEV)
    pm = torch.empty((B, Hq, n), dtype=torch.float32, device=DEV)
    psum = torch.empty((B, Hq, n), dtype=torch.float32, device=DEV)

    def step():
        pa.pa_decode_append(None, dev.query, dev.new_key, dev.new_value, dev.new_slots,
                            dev.k_cache, dev.v_cache, dev.block_tables, dev.context_lens,
                            wl.scale, 512, po, pm, psum)
        pa.pa_decode_reduce(out, po, pm, psum, dev.context_lens, 512)

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
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(out), want)
