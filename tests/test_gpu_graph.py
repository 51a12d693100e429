"""The decode step (cache write, decode, reduce) captured in a HIP graph.

The library only enqueues kernels on the caller's stream (no allocation, no
memset, no synchronization), so a serving loop may capture a whole step.
Every replay, with other eager work and synchronizations in between, must
reproduce the eager step bit for bit: the kernels are deterministic and the
appended token rewrites the same slot each time.
"""
import numpy as np
import pytest
import torch

import paged_kv_decode_pa_amd as pa
from tests.gpu_helpers import (DEV, TOL, bits_of, config_device, config_reference, max_err,
                               say, tdtype)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cid,ps", [(2, 512), (2, 0), (5, 256), (1, 0), (1, 64)])
def test_graph_replays_match_eager(cid, ps):
    say(f"[graph] config {cid} partition {ps}")
    dw = config_device(cid)
    wl = dw.wl
    B, Hq, D = wl.num_seqs, wl.num_q_heads, wl.head_dim
    out = torch.empty((B, Hq, D), dtype=tdtype(wl.dtype), device=DEV)
    n = dw.partition_count(ps) if ps else 0
    po = torch.empty((B, Hq, n, D), dtype=torch.float32, device=DEV) if ps else None
    pm = torch.empty((B, Hq, n), dtype=torch.float32, device=DEV) if ps else None
    psum = torch.empty((B, Hq, n), dtype=torch.float32, device=DEV) if ps else None

    def step():
        pa.pa_reshape_and_cache(dw.new_key, dw.new_value, dw.k_cache, dw.v_cache, dw.new_slots)
        if ps:
            pa.pa_decode(None, dw.query, dw.k_cache, dw.v_cache, dw.block_tables,
                         dw.context_lens, wl.scale, ps, po, pm, psum)
            pa.pa_decode_reduce(out, po, pm, psum, dw.context_lens, ps)
        else:
            pa.pa_decode(out, dw.query, dw.k_cache, dw.v_cache, dw.block_tables,
                         dw.context_lens, wl.scale)

    step()
    torch.cuda.synchronize()
    eager = bits_of(out).copy()
    assert max_err(out, config_reference(cid)) <= TOL[wl.dtype]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(4):
        out.fill_(float("nan"))
        if ps:
            po.fill_(float("nan"))
            pm.fill_(float("nan"))
            psum.fill_(float("nan"))
        noise = torch.randn(1 << 20, device=DEV)
        float(noise.sum())  # eager work and a synchronization between replays
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(out), eager), f"replay {rep} differs from the eager step"
    del graph
