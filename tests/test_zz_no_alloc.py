"""pa_chunk_attention_split_noalloc (split partials in the library's fixed
per-GPU scratch array) against pa_chunk_attention_split (caller workspace),
through the C ABI, on two calls in a row, the second with a smaller batch:
the outputs must be identical bit for bit (same kernels, same arithmetic;
nothing left in the array by the first call may reach the second), and
within the bf16 tolerance of the fp64 oracle."""
import numpy as np
import pytest
import torch

import paged_kv_decode_pa_amd as pa
from tests.gpu_helpers import (DEV, TOL, DeviceWorkload, bits_of, config_device, max_err, say,
                               to_dev)
from tests.test_gpu_chunk import chunk_reference
from tests.test_gpu_chunk_split import run_split
from workloads import make_chunk_queries, make_custom_workload

pytestmark = pytest.mark.gpu


def run_noalloc(dev, query, query_start, partition_size):
    wl = dev.wl
    q = to_dev(query, wl.dtype)
    qs = torch.from_numpy(np.asarray(query_start, dtype=np.int32)).to(DEV)
    out = torch.full_like(q, float("nan"))
    n_parts = max(1, -(-int(wl.context_lens.max()) // partition_size))
    mq = int(np.diff(np.asarray(query_start)).max())
    pa.pa_chunk_attention_split_noalloc(out, q, dev.k_cache, dev.v_cache, dev.block_tables,
                                        dev.context_lens, qs, mq, wl.scale, partition_size,
                                        n_parts)
    torch.cuda.synchronize()
    return out


def test_noalloc_equals_workspace_on_two_calls():
    # Call 1: the Llama-3-8B-shaped batch, 4 drafted tokens per sequence,
    # 768-token partitions (64 x 4 tokens x 32 heads x 6 partitions: 26 MB of
    # partials).
    dev1 = config_device(2)
    q1, qs1 = make_chunk_queries(dev1.wl, [4] * dev1.wl.num_seqs, seed=81)
    # Call 2: a smaller batch with other lengths, 2 tokens, 256-token partitions.
    wl2 = make_custom_workload([300, 17, 900, 64, 1200, 5, 33, 700, 128, 2000, 16, 450],
                               num_q_heads=32, num_kv_heads=8, head_dim=128, seed=82)
    dev2 = DeviceWorkload(wl2)
    q2, qs2 = make_chunk_queries(wl2, [2] * wl2.num_seqs, seed=83)
    for name, dev, q, qs, ps in (("call 1", dev1, q1, qs1, 768), ("call 2", dev2, q2, qs2, 256)):
        say(f"[no-alloc] {name}: {dev.wl.num_seqs} sequences, partition {ps}")
        got = run_noalloc(dev, q, qs, ps)
        want = run_split(dev, q, qs, ps)
        assert np.array_equal(bits_of(got), bits_of(want)), name
        err = max_err(got, chunk_reference(dev.wl, q, qs))
        say(f"    bit-identical to the workspace call; max abs err {err:.3e}")
        assert err <= TOL["bf16"]


def test_noalloc_rejects_what_the_array_cannot_hold():
    dev = config_device(2)
    wl = dev.wl
    q, qs = make_chunk_queries(wl, [64] * wl.num_seqs, seed=84)
    # 4096 tokens x 32 heads x 256 partitions of 16 tokens: far past 64 MiB.
    with pytest.raises(pa.PaError) as e:
        run_noalloc(dev, q, qs, 16)
    assert e.value.status == 4
