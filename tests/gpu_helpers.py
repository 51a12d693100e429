"""Shared plumbing for the GPU parity tests: move a workload to the device,
run the library through its Python binding, and compare with the oracle."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import oracle
import paged_kv_decode_pa_amd as pa
from tests.oracle_pins import fill_pools
from workloads import config_by_id, make_workload

DEV = "cuda:0"
TOL = {"bf16": 2e-2, "f32": 1e-5}


def say(*msg):
    print(*msg, flush=True)
    sys.stdout.flush()


def tdtype(dtype):
    return torch.float32 if dtype == "f32" else torch.bfloat16


def to_dev(arr, dtype):
    """Host payload (float32 or bf16 bits) -> device tensor of the storage dtype."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(DEV)
    bits = np.ascontiguousarray(arr, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(bits).to(DEV).view(torch.bfloat16)


def bits_of(t):
    """Device tensor -> host uint16 (bf16) or float32 array with the same bits."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def f64_of(t):
    return t.float().cpu().numpy().astype(np.float64)


class DeviceWorkload:
    """A workload's tensors in GPU memory, pools NaN-poisoned before the fill."""

    def __init__(self, wl, fill=True):
        self.wl = wl
        dt = tdtype(wl.dtype)
        P, Hkv, D = wl.page_size, wl.num_kv_heads, wl.head_dim
        self.k_cache = torch.full((wl.num_pages, Hkv, P, D), float("nan"), dtype=dt, device=DEV)
        self.v_cache = torch.full((wl.num_pages, Hkv, D, P), float("nan"), dtype=dt, device=DEV)
        self.query = to_dev(wl.query, wl.dtype)
        self.block_tables = torch.from_numpy(wl.block_tables).to(DEV)
        self.context_lens = torch.from_numpy(wl.context_lens).to(DEV)
        self.new_key = to_dev(wl.new_key, wl.dtype)
        self.new_value = to_dev(wl.new_value, wl.dtype)
        self.new_slots = torch.from_numpy(wl.new_slots).to(DEV)
        if fill:
            self.prefill()
            self.append()
            torch.cuda.synchronize()

    def prefill(self):
        wl = self.wl
        if len(wl.prefill_slots):
            pa.pa_reshape_and_cache(to_dev(wl.prefill_key, wl.dtype),
                                    to_dev(wl.prefill_value, wl.dtype), self.k_cache,
                                    self.v_cache, torch.from_numpy(wl.prefill_slots).to(DEV))

    def append(self):
        pa.pa_reshape_and_cache(self.new_key, self.new_value, self.k_cache, self.v_cache,
                                self.new_slots)

    def partition_count(self, partition_size):
        return max(1, -(-int(self.wl.context_lens.max()) // partition_size))

    def decode(self, partition_size=0, kernel="auto", max_parts=None):
        wl = self.wl
        B, Hq, D = wl.num_seqs, wl.num_q_heads, wl.head_dim
        out = torch.empty((B, Hq, D), dtype=tdtype(wl.dtype), device=DEV)
        fn = pa.pa_decode if kernel == "auto" else pa.pa_decode_valu
        if partition_size == 0:
            fn(out, self.query, self.k_cache, self.v_cache, self.block_tables, self.context_lens,
               wl.scale)
        else:
            n = max_parts or self.partition_count(partition_size)
            # NaN-filled so a partition the kernel fails to write poisons the result
            po = torch.full((B, Hq, n, D), float("nan"), dtype=torch.float32, device=DEV)
            pm = torch.full((B, Hq, n), float("nan"), dtype=torch.float32, device=DEV)
            ps = torch.full((B, Hq, n), float("nan"), dtype=torch.float32, device=DEV)
            fn(None, self.query, self.k_cache, self.v_cache, self.block_tables,
               self.context_lens, wl.scale, partition_size, po, pm, ps)
            pa.pa_decode_reduce(out, po, pm, ps, self.context_lens, partition_size)
        torch.cuda.synchronize()
        return out


@functools.lru_cache(maxsize=None)
def config_workload(cid):
    return make_workload(config_by_id(cid))


@functools.lru_cache(maxsize=None)
def config_reference(cid):
    """The oracle's fp64 output for a fixed config (cached per session)."""
    return oracle_reference(config_workload(cid))


@functools.lru_cache(maxsize=None)
def config_device(cid):
    """The config's workload uploaded and cache-filled once per session."""
    return DeviceWorkload(config_workload(cid))


def oracle_reference(wl):
    k, v = fill_pools(oracle, wl)
    return oracle.decode(wl.query, k, v, wl.block_tables, wl.context_lens, wl.scale,
                         wl.page_size, wl.dtype)


def max_err(out, ref):
    got = f64_of(out)
    assert np.isfinite(got).all(), "non-finite output"
    return float(np.abs(got - ref).max())


def parity_report(out, ref):
    """Max-abs error, relative error max|err| / max|ref|, and (bf16) the
    largest distance in bf16 ulps from the oracle's value rounded once to
    nearest-even."""
    got = f64_of(out)
    assert np.isfinite(got).all(), "non-finite output"
    err = float(np.abs(got - ref).max())
    scale = float(np.abs(ref).max())
    rep = {"max_abs": err, "rel": err / scale if scale > 0 else err, "max_ulp": None}
    if out.dtype == torch.bfloat16:
        rep["max_ulp"] = int(oracle.bf16_ulp_distance(bits_of(out),
                                                      oracle.round_to_bf16_bits(ref)).max())
    return rep


def report_line(rep):
    ulp = "" if rep["max_ulp"] is None else f", max {rep['max_ulp']} bf16 ulp from RNE(oracle)"
    return f"max abs err {rep['max_abs']:.3e}, rel {rep['rel']:.3e}{ulp}"
