#!/usr/bin/env python3
"""Benchmark one paged-KV decode step on one MI355X.

A step is the whole hot path for one batch: pa_reshape_and_cache appends each
sequence's new token to the page pool, pa_decode attends over every cached
token, and pa_decode_reduce merges split-KV partitions.  Inputs are synthetic
(seeded, N(0,1) values cast to bf16) and resident in HBM before timing.  Before
each timed step a 1 GiB buffer is read on the same stream, outside the timed
events, so the KV pages come from HBM and not from L2 or the 256 MB MALL.  The
flush reads rather than writes: a write flush leaves up to 256 MB of dirty
lines in the MALL whose write-back would be charged to the timed kernels.

Prints ONE JSON line (the headline workload) on stdout; with --all, lines for
the other workloads go to stderr first.

    python bench.py [--steps K] [--warmup W] [--config 2] [--all]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention: achieved KV HBM GB/s (% of peak) + seqs/sec, 1 GPU"
PEAK_HBM_GBS = 8000.0   # MI355X HBM3E, vendor peak
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["paged_kv_decode_pa_amd/csrc/decode_mfma.hip",
                  "paged_kv_decode_pa_amd/csrc/split_plan.hpp",
                  "paged_kv_decode_pa_amd/csrc/wave_attn.hpp",
                  "paged_kv_decode_pa_amd/csrc/page_stream.hpp",
                  "paged_kv_decode_pa_amd/csrc/pa_device.hpp"]
CHUNK_KERNEL_SOURCES = ["paged_kv_decode_pa_amd/csrc/chunk_mfma.hip",
                        "paged_kv_decode_pa_amd/csrc/split_plan.hpp",
                        "paged_kv_decode_pa_amd/csrc/wave_attn.hpp",
                        "paged_kv_decode_pa_amd/csrc/page_stream.hpp",
                        "paged_kv_decode_pa_amd/csrc/pa_device.hpp"]
# The multi-token kernel that stages K/V in LDS (more than 64 columns per kv head).
CHUNK_LDS_KERNEL_SOURCES = ["paged_kv_decode_pa_amd/csrc/chunk_lds.hip",
                            "paged_kv_decode_pa_amd/csrc/split_plan.hpp",
                            "paged_kv_decode_pa_amd/csrc/page_stream.hpp",
                            "paged_kv_decode_pa_amd/csrc/pa_device.hpp"]
CHUNK_LDS_MIN_COLUMNS = 65  # max_query_len * (q heads per kv head) from which it runs
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
# --chunk default: the single pass (pa_chunk_attention) at every token count
# (on the Llama-3-8B batch it beats the split form at 768-token partitions from
# one new token up: 98 against 106 us at 1, 102 against 119 at 4).
# --chunk-partition PS times pa_chunk_attention_split instead.
TRANSFER_METRIC = ("KV page hand-off: export every page of the batch to one buffer, import it "
                   "into another pool; GB/s read + written, 1 GPU")
PAGER_METRIC = ("host page-pool owner: decode steps/s of bookkeeping (one append per "
                "sequence + the batch's block tables), 1 host thread")
CHUNK_METRIC = ("multi-token causal attention over the paged cache (draft verification / "
                "chunked prefill): query tokens/s, 1 GPU")

WORKLOAD_NAMES = {
    1: "tiny fp32 decode: 4 seqs, lengths {17,64,100,255}, 8 q / 2 kv heads, D=64, 16-token pages",
    2: "Llama-3-8B-shaped decode batch: 64 seqs, 32 q / 8 kv heads, D=128, bf16 KV, "
       "16-token pages, lengths U[512,4096], pages scattered in a 1.25x pool",
    3: "prefix-reuse decode: 128 seqs in 8 groups of 16 sharing a 2048-token prefix, suffixes "
       "U[64,512], 32 q / 8 kv heads, D=128, bf16 KV, 16-token pages",
    4: "long-context split-KV decode: 8 seqs, lengths U[16384,32768], 32 q / 8 kv heads, "
       "D=128, bf16 KV, 16-token pages, 512-token partitions",
    5: "70B tensor-parallel-8 per-GPU share: 256 seqs, 8 q / 1 kv head, D=128, bf16 KV, "
       "16-token pages, lengths log-uniform [128,8192] with 25% at <= 32",
}


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--all", action="store_true", help="also run the other four workloads")
    ap.add_argument("--partition-size", type=int, default=None,
                    help="split-KV partition in tokens (default: the workload's own)")
    ap.add_argument("--kernel", choices=["auto", "valu"], default="auto",
                    help="auto = pa_decode; valu = pa_decode_valu")
    ap.add_argument("--cascade", action="store_true",
                    help="read pages shared by a group of sequences once per group "
                         "(pa_decode_cascade; split-KV only; the prefix-reuse workload's "
                         "default)")
    ap.add_argument("--no-cascade", action="store_true",
                    help="the prefix-reuse workload without pa_decode_cascade (every "
                         "sequence reads its own block-table row)")
    ap.add_argument("--unfused", action="store_true",
                    help="time the step as three calls (pa_reshape_and_cache, pa_decode, reduce) "
                         "instead of pa_decode_append + reduce")
    ap.add_argument("--no-flush", action="store_true", help="keep caches warm between steps")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in a HIP graph (reported, not the value)")
    ap.add_argument("--unshared", action="store_true",
                    help="prefix-reuse workload with every sequence's prefix in private pages")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="time budget of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (counter calibration)")
    ap.add_argument("--transfer", action="store_true",
                    help="time pa_export_pages + pa_import_pages of every page of the batch "
                         "instead of the decode step")
    ap.add_argument("--pager", action="store_true",
                    help="time the host page-pool owner (no GPU): admitting the batch's "
                         "prompts, then decode-step appends and block tables")
    ap.add_argument("--chunk-partition", type=int, default=None, metavar="PS",
                    help="with --chunk: pa_chunk_attention_split at this partition size "
                         "(default 0 = the single-pass pa_chunk_attention)")
    ap.add_argument("--chunk", type=int, default=0, metavar="Q",
                    help="time pa_chunk_attention with Q new tokens per sequence instead of the "
                         "decode step (the cache write of the Q tokens, then the attention)")
    return ap.parse_args()


def stats(xs):
    a = np.asarray(xs, dtype=np.float64)
    return {"mean": float(a.mean()), "median": float(np.median(a)),
            "p10": float(np.percentile(a, 10)), "p90": float(np.percentile(a, 90))}


def byte_counts(wl, partition_size):
    """Algorithmic bytes of one step, from the workload's shapes."""
    esz = wl.elem_bytes
    B, Hq, Hkv, D = wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    L = wl.context_lens.astype(np.int64)
    per_token = 2 * Hkv * D * esz                      # K and V rows of one token
    unique_tokens = len(wl.prefill_slots) + int((wl.new_slots >= 0).sum())
    kv_unique = unique_tokens * per_token              # shared prefix pages counted once
    kv_logical = int(L.sum()) * per_token
    q_bytes = B * Hq * D * esz
    tables = int(((L + 15) // 16).sum()) * 4 + B * 4
    n_parts = (L + partition_size - 1) // partition_size if partition_size else np.zeros_like(L)
    partial = int(n_parts.sum()) * Hq * (D + 2) * 4
    decode = kv_unique + q_bytes + tables + (partial if partition_size else q_bytes)
    reduce = (partial + q_bytes + B * 4) if partition_size else 0
    cache_write = B * (2 * per_token + 8)              # read the new rows, write them, slots
    return {"kv_unique": kv_unique, "kv_logical": kv_logical, "decode_kernel": decode,
            "reduce_kernel": reduce, "cache_write": cache_write,
            "step": decode + reduce + cache_write}


def kernel_source_hash(sources=KERNEL_SOURCES):
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_profile_kv(name, sources):
    """key: value lines of a committed counter summary, or None when it is
    absent or the kernel's sources changed since the counters were taken."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash(sources):
        return None
    return kv


def read_traffic(cid, partition_size, cascade=False):
    """HBM bytes per decode launch from a committed counter summary, or None
    when the summary is absent or the kernel changed since it was taken."""
    kv = (read_profile_kv(f"traffic_cascade_cfg{cid}.txt", CHUNK_KERNEL_SOURCES) if cascade else
          read_profile_kv(f"traffic_decode_mfma_cfg{cid}.txt", KERNEL_SOURCES))
    if kv is None or int(kv.get("partition_size", -1)) != partition_size:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(dev):
    """Three 512 MiB device copies: the known sizes that scale the HBM counters."""
    import torch

    src = torch.empty(1 << 27, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def run_config(cid, args):
    import torch

    import paged_kv_decode_pa_amd as pa
    from workloads import config_by_id, make_workload

    cfg = config_by_id(cid)
    cascade = (args.cascade or cfg.bench_cascade) and not (args.no_cascade or args.unshared)
    default_ps = cfg.cascade_partition_size if cascade and cfg.bench_cascade else cfg.bench_partition_size
    ps = default_ps if args.partition_size is None else args.partition_size
    t0 = time.time()
    wl = make_workload(cfg, share_prefix=not args.unshared)
    print(f"[bench] config {cid} ({cfg.name}{', unshared' if args.unshared else ''}) drawn in {time.time() - t0:.1f}s; "
          f"partition {ps}", file=sys.stderr, flush=True)

    dev = torch.device("cuda:0")
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16

    def up(a):
        if wl.dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    P, Hkv, D, Hq, B = wl.page_size, wl.num_kv_heads, wl.head_dim, wl.num_q_heads, wl.num_seqs
    k_cache = torch.full((wl.num_pages, Hkv, P, D), float("nan"), dtype=dt, device=dev)
    v_cache = torch.full((wl.num_pages, Hkv, D, P), float("nan"), dtype=dt, device=dev)
    pa.pa_reshape_and_cache(up(wl.prefill_key), up(wl.prefill_value), k_cache, v_cache,
                            torch.from_numpy(wl.prefill_slots).to(dev))
    query = up(wl.query)
    new_key, new_value = up(wl.new_key), up(wl.new_value)
    new_slots = torch.from_numpy(wl.new_slots).to(dev)
    tables = torch.from_numpy(wl.block_tables).to(dev)
    lens = torch.from_numpy(wl.context_lens).to(dev)
    out = torch.empty((B, Hq, D), dtype=dt, device=dev)
    n_parts = max(1, -(-int(wl.context_lens.max()) // ps)) if ps else 0
    po = torch.empty((B, Hq, n_parts, D), dtype=torch.float32, device=dev) if ps else None
    pm = torch.empty((B, Hq, n_parts), dtype=torch.float32, device=dev) if ps else None
    psum = torch.empty((B, Hq, n_parts), dtype=torch.float32, device=dev) if ps else None
    decode_fn = pa.pa_decode if args.kernel == "auto" else pa.pa_decode_valu
    flush_buf = None if args.no_flush else torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def flush():
        if flush_buf is not None:
            flush_buf.sum()  # read 1 GiB: evicts L2 and MALL, leaves no dirty lines

    # The step's cache write runs inside the decode launch (pa_decode_append)
    # unless --unfused or the vector kernel is asked for.
    fused = args.kernel == "auto" and not args.unfused
    groups = None
    if cascade:
        if not ps or wl.dtype != "bf16" or args.kernel != "auto":
            raise SystemExit("--cascade needs a bf16 workload, the matrix-core kernels and a "
                             "partition size")
        t0 = time.perf_counter()
        g = pa.prefix_groups(wl.block_tables, wl.context_lens, ps // P)
        plan_us = (time.perf_counter() - t0) * 1e6
        groups = dict(g)
        for k in ("group_start", "group_seqs", "group_partitions", "seq_first_partition"):
            groups[k] = torch.from_numpy(np.ascontiguousarray(g[k], dtype=np.int32)).to(dev)

    def step(ev=None, marks=True):
        """One step; `ev` = events to record, at the step's ends only or (marks)
        also between its kernels."""
        if ev:
            ev[0].record()
        if not fused:
            pa.pa_reshape_and_cache(new_key, new_value, k_cache, v_cache, new_slots)
            if ev and marks:
                ev[1].record()
        elif ev and marks:
            ev[1] = ev[0]
        if groups is not None:
            pa.pa_decode_cascade(query, k_cache, v_cache, tables, lens, wl.scale, ps, po, pm,
                                 psum, groups, **({"key": new_key, "value": new_value,
                                                   "slot_mapping": new_slots} if fused else {}))
        elif fused and ps:
            pa.pa_decode_append(None, query, new_key, new_value, new_slots, k_cache, v_cache,
                                tables, lens, wl.scale, ps, po, pm, psum)
        elif fused:
            pa.pa_decode_append(out, query, new_key, new_value, new_slots, k_cache, v_cache,
                                tables, lens, wl.scale)
        elif ps:
            decode_fn(None, query, k_cache, v_cache, tables, lens, wl.scale, ps, po, pm, psum)
        else:
            decode_fn(out, query, k_cache, v_cache, tables, lens, wl.scale)
        if ev and marks and ps:
            ev[2].record()
        if ps:
            pa.pa_decode_reduce(out, po, pm, psum, lens, ps)
        if ev:
            ev[3].record()

    def timed(marks):
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
                  for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            flush()
            step(events[k], marks)
        torch.cuda.synchronize()
        return events, time.perf_counter() - t0

    for _ in range(args.warmup):
        flush()
        step()
    torch.cuda.synchronize()
    # Pass 1, the step as a whole: events only at its two ends (an event
    # recorded between kernels adds a few microseconds of its own).
    step_events, wall = timed(marks=False)
    # Pass 2, per kernel: events between the kernels, for the breakdown and the
    # decode launch time the roofline uses.
    events, _ = timed(marks=True)
    if not torch.isfinite(out.float()).all():
        raise RuntimeError("non-finite decode output")

    step_ms = [e[0].elapsed_time(e[3]) for e in step_events]
    marked_step_ms = [e[0].elapsed_time(e[3]) for e in events]
    cache_ms = None if fused else [e[0].elapsed_time(e[1]) for e in events]
    decode_ms = [e[1].elapsed_time(e[2] if ps else e[3]) for e in events]
    reduce_ms = [e[2].elapsed_time(e[3]) for e in events] if ps else None

    # Optionally the same step captured once in a HIP graph and replayed, as a
    # serving loop might run it: two events bracket each replay and the flush
    # stays outside them.  (On this stack a replay measured about 2 us slower
    # than the eager launches, so the value stays the eager step.)
    graph_ms = None
    if args.graph:
        cur = torch.cuda.current_stream()
        side = torch.cuda.Stream()
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            step()
        cur.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            flush()
            graph.replay()
        torch.cuda.synchronize()
        gev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for k in range(args.steps):
            flush()
            gev[k][0].record()
            graph.replay()
            gev[k][1].record()
        torch.cuda.synchronize()
        graph_ms = [a.elapsed_time(b) for a, b in gev]
        if not torch.isfinite(out.float()).all():
            raise RuntimeError("non-finite decode output (graph replay)")
        del graph

    if args.copy_calibration:
        copy_calibration(dev)

    nb = byte_counts(wl, ps)
    if groups is not None and int(groups["num_groups"]) > 0:
        # the prefix units carry one or two 16-column blocks per wave
        blocks = -(-int(groups["max_group_size"]) * (Hq // Hkv) // 16)
        roof_kernel = f"cascade_kernel<{D}, {min(max(blocks, 1), 2)}>"
        traffic = read_traffic(cid, ps, cascade=True)
    else:
        roof_kernel = ("decode_valu_kernel" if (wl.dtype != "bf16" or args.kernel != "auto")
                       else "decode_split_kernel" if ps else "decode_whole_kernel") + f"<{D}>"
        traffic = (read_traffic(cid, ps) if (wl.dtype == "bf16" and args.kernel == "auto")
                   else None)
    t_step = float(np.mean(step_ms)) * 1e-3
    t_dec = float(np.mean(decode_ms)) * 1e-3
    gbs = nb["kv_unique"] / t_step / 1e9
    launch_bytes = nb["decode_kernel"] + (nb["cache_write"] if fused else 0)
    achieved = launch_bytes / t_dec / 1e9
    line = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_NAMES[cid],
            "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "page_size": P,
            "partition_size": ps, "prefix_pages_shared": not args.unshared,
            "kernel": (("pa_decode_cascade (shared prefix pages read once per group"
                        + ("; the step's cache write inside the launch)" if fused else ")"))
                       if groups is not None else
                       "pa_decode_append (cache write inside the decode launch)" if fused else
                       "pa_decode" if args.kernel == "auto" else "pa_decode_valu"),
            "cache_flush_between_steps": flush_buf is not None,
            "parallelism": "none (1 GPU)",
            "shared_prefix_groups": (None if groups is None else
                                     {"groups": int(groups["num_groups"]),
                                      "max_members": int(groups["max_group_size"]),
                                      "shared_partitions": int(groups["max_group_partitions"]),
                                      "host_plan_us": round(plan_us, 1)}),
        },
        "pct_of_peak_hbm": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "seqs_per_s": round(B / t_step, 1),
        "effective_logical_kv_gbs": round(nb["kv_logical"] / t_step / 1e9, 1),
        "step_timing": "eager launches; HIP events on the library's stream at the step's ends",
        "kernels_ms": {"cache_write": stats(cache_ms) if cache_ms else None,
                       "decode": stats(decode_ms),
                       "reduce": stats(reduce_ms) if reduce_ms else None,
                       "step": stats(step_ms), "step_with_kernel_markers": stats(marked_step_ms)},
        "graph_step_ms": stats(graph_ms) if graph_ms else None,
        "wall_ms_per_step_incl_flush": round(wall / args.steps * 1e3, 4),
        "bytes": nb,
        "roofline": {
            "bound": "hbm",
            "kernel": roof_kernel,
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": launch_bytes,
            "mean_launch_us": round(t_dec * 1e6, 2),
        },
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, nb, t_step)
    return line


def chunk_counts(wl, q, partition_size=0):
    """Algorithmic bytes and flops of one multi-token call with q new tokens
    per sequence: every cached token's K/V read once (shared prefix pages
    once), the queries read and the outputs written once, and with split-KV
    partitions each partial written and read once; two products of D
    multiply-adds per (query token, head, attended position)."""
    esz, B, Hq, Hkv, D = wl.elem_bytes, wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    L = wl.context_lens.astype(np.int64)
    per_token = 2 * Hkv * D * esz
    unique_tokens = len(wl.prefill_slots) + int((wl.new_slots >= 0).sum())
    rows = B * q * Hq * D * esz
    tables = int(((L + 15) // 16).sum()) * 4 + B * 4 + (B + 1) * 4
    attended = int(sum(q * int(l) - q * (q - 1) // 2 for l in L))  # positions L-q .. L-1
    partials = 0
    if partition_size:
        n_parts = (L + partition_size - 1) // partition_size
        partials = 2 * int(n_parts.sum()) * q * Hq * (D + 2) * 4
    return {"kv_unique": unique_tokens * per_token, "query": rows, "out": rows, "tables": tables,
            "partials": partials,
            "kernel": unique_tokens * per_token + 2 * rows + tables + partials,
            "cache_write": B * q * (2 * per_token + 8),
            "flops": 4 * D * Hq * attended}


def run_chunk_config(cid, args):
    import torch

    import paged_kv_decode_pa_amd as pa
    from workloads import bf16_bits_from_f32, config_by_id, make_chunk_queries, make_workload

    cfg = config_by_id(cid)
    wl = make_workload(cfg, share_prefix=not args.unshared)
    if wl.dtype != "bf16":
        raise SystemExit("--chunk needs a bf16 workload")
    q = args.chunk
    if q > int(wl.context_lens.min()):
        raise SystemExit(f"--chunk {q} exceeds the shortest context")
    dev = torch.device("cuda:0")

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    P, Hkv, D, Hq, B = wl.page_size, wl.num_kv_heads, wl.head_dim, wl.num_q_heads, wl.num_seqs
    k_cache = torch.full((wl.num_pages, Hkv, P, D), float("nan"), dtype=torch.bfloat16, device=dev)
    v_cache = torch.full((wl.num_pages, Hkv, D, P), float("nan"), dtype=torch.bfloat16, device=dev)
    pa.pa_reshape_and_cache(up(wl.prefill_key), up(wl.prefill_value), k_cache, v_cache,
                            torch.from_numpy(wl.prefill_slots).to(dev))
    pa.pa_reshape_and_cache(up(wl.new_key), up(wl.new_value), k_cache, v_cache,
                            torch.from_numpy(wl.new_slots).to(dev))
    qpay, qs = make_chunk_queries(wl, [q] * B, seed=cid)
    query = up(qpay)
    query_start = torch.from_numpy(qs).to(dev)
    # The q new tokens' K/V rows (positions L-q .. L-1 of each sequence),
    # rewritten by every step as a verification step would append them.
    rng = np.random.default_rng(100 + cid)
    kv_shape = (B * q, Hkv, D)
    new_k = up(bf16_bits_from_f32(rng.standard_normal(kv_shape, dtype=np.float32)))
    new_v = up(bf16_bits_from_f32(rng.standard_normal(kv_shape, dtype=np.float32)))
    slots = np.empty(B * q, dtype=np.int64)
    for b in range(B):
        for i in range(q):
            pos = int(wl.context_lens[b]) - q + i
            slots[b * q + i] = int(wl.block_tables[b, pos // P]) * P + pos % P
    slots_d = torch.from_numpy(slots).to(dev)
    tables = torch.from_numpy(wl.block_tables).to(dev)
    lens = torch.from_numpy(wl.context_lens).to(dev)
    out = torch.empty_like(query)
    flush_buf = None if args.no_flush else torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    cps = args.chunk_partition or 0
    if cps:
        n_parts = max(1, -(-int(wl.context_lens.max()) // cps))
        T = B * q
        po = torch.empty((T, Hq, n_parts, D), dtype=torch.float32, device=dev)
        pm = torch.empty((T, Hq, n_parts), dtype=torch.float32, device=dev)
        psum = torch.empty((T, Hq, n_parts), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step(ev=None, marks=True):
        if ev:
            ev[0].record()
        pa.pa_reshape_and_cache(new_k, new_v, k_cache, v_cache, slots_d)
        if ev and marks:
            ev[1].record()
        if cps:
            pa.pa_chunk_attention_split(out, query, k_cache, v_cache, tables, lens, query_start, q,
                                        wl.scale, cps, po, pm, psum)
        else:
            pa.pa_chunk_attention(out, query, k_cache, v_cache, tables, lens, query_start, q,
                                  wl.scale)
        if ev:
            ev[2].record()

    def timed(marks):
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
                  for _ in range(args.steps)]
        torch.cuda.synchronize()
        for k in range(args.steps):
            if flush_buf is not None:
                flush_buf.sum()
            step(events[k], marks)
        torch.cuda.synchronize()
        return events

    for _ in range(args.warmup):
        if flush_buf is not None:
            flush_buf.sum()
        step()
    torch.cuda.synchronize()
    step_ev = timed(marks=False)
    ev = timed(marks=True)
    if not torch.isfinite(out.float()).all():
        raise RuntimeError("non-finite chunk attention output")
    if args.copy_calibration:
        copy_calibration(dev)
    step_ms = [e[0].elapsed_time(e[2]) for e in step_ev]
    cache_ms = [e[0].elapsed_time(e[1]) for e in ev]
    attn_ms = [e[1].elapsed_time(e[2]) for e in ev]
    nb = chunk_counts(wl, q, cps)
    t_step = float(np.mean(step_ms)) * 1e-3
    t_attn = float(np.mean(attn_ms)) * 1e-3
    gbs = nb["kernel"] / t_attn / 1e9
    tflops = nb["flops"] / t_attn / 1e12
    hbm_frac, mfma_frac = gbs / PEAK_HBM_GBS, tflops / PEAK_BF16_TFLOPS
    bound = "hbm" if hbm_frac >= mfma_frac else "mfma"
    roof = ({"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": round(hbm_frac, 4)} if bound == "hbm" else
            {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
             "unit": "TFLOP/s", "frac": round(mfma_frac, 4)})
    lds = not cps and q * (Hq // Hkv) >= CHUNK_LDS_MIN_COLUMNS
    lds_waves = 8 if q * (Hq // Hkv) > 128 else 4
    kv = read_profile_kv(f"traffic_chunk_attention_cfg{cid}_q{q}.txt",
                         CHUNK_LDS_KERNEL_SOURCES if lds else CHUNK_KERNEL_SOURCES)
    traffic = None
    if kv is not None and not args.unshared and int(kv.get("partition_size", 0)) == cps:
        try:
            traffic = float(kv["hbm_bytes_per_launch"])
        except (KeyError, ValueError):
            traffic = None
    roof.update({"traffic": traffic,
                 "kernel": (f"chunk_split_kernel<{D}> + decode_reduce_kernel (one call, "
                            f"{cps}-token partitions)" if cps else
                            f"chunk_lds_kernel<{D}, {lds_waves}>" if lds else
                            f"chunk_attention_kernel<{D}>"),
                 "algorithmic_bytes_per_launch": nb["kernel"], "flops_per_launch": nb["flops"],
                 "hbm_gbs": round(gbs, 1), "bf16_tflops": round(tflops, 2),
                 "mean_launch_us": round(t_attn * 1e6, 2)})
    return {
        "metric": CHUNK_METRIC,
        "value": round(B * q / t_step, 1),
        "unit": "query tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[cid] + f"; {q} new tokens per sequence",
                   "batch": B, "new_tokens_per_seq": q, "partition_size": cps,
                   "entry_point": "pa_chunk_attention_split" if cps else "pa_chunk_attention",
                   "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": D, "page_size": P, "prefix_pages_shared": not args.unshared,
                   "cache_flush_between_steps": flush_buf is not None,
                   "parallelism": "none (1 GPU)"},
        "kernels_ms": {"cache_write": stats(cache_ms), "chunk_attention": stats(attn_ms),
                       "step": stats(step_ms)},
        "bytes": nb,
        "roofline": roof,
    }


def run_transfer_config(cid, args):
    import torch

    import paged_kv_decode_pa_amd as pa
    from workloads import config_by_id, make_workload

    cfg = config_by_id(cid)
    wl = make_workload(cfg, share_prefix=not args.unshared)
    dev = torch.device("cuda:0")
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16

    def up(a):
        if wl.dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    P, Hkv, D = wl.page_size, wl.num_kv_heads, wl.head_dim
    k_cache = torch.full((wl.num_pages, Hkv, P, D), float("nan"), dtype=dt, device=dev)
    v_cache = torch.full((wl.num_pages, Hkv, D, P), float("nan"), dtype=dt, device=dev)
    pa.pa_reshape_and_cache(up(wl.prefill_key), up(wl.prefill_value), k_cache, v_cache,
                            torch.from_numpy(wl.prefill_slots).to(dev))
    pa.pa_reshape_and_cache(up(wl.new_key), up(wl.new_value), k_cache, v_cache,
                            torch.from_numpy(wl.new_slots).to(dev))
    n_of = (wl.context_lens.astype(np.int64) + P - 1) // P
    used = np.unique(np.concatenate([wl.block_tables[b, :n_of[b]] for b in range(wl.num_seqs)]))
    n = len(used)
    ids = torch.from_numpy(used.astype(np.int32)).to(dev)
    dest = torch.from_numpy(np.random.default_rng(200 + cid).permutation(wl.num_pages)[:n]
                            .astype(np.int32)).to(dev)
    block = Hkv * P * D
    buf = torch.empty((2, n, block), dtype=dt, device=dev)
    k2 = torch.full_like(k_cache, float("nan"))
    v2 = torch.full_like(v_cache, float("nan"))
    flush_buf = None if args.no_flush else torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev:
            ev[0].record()
        pa.pa_export_pages(buf, k_cache, v_cache, ids)
        if ev:
            ev[1].record()
        pa.pa_import_pages(buf, k2, v2, dest)
        if ev:
            ev[2].record()

    for _ in range(args.warmup):
        if flush_buf is not None:
            flush_buf.sum()
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for k in range(args.steps):
        if flush_buf is not None:
            flush_buf.sum()
        step(ev[k])
    torch.cuda.synchronize()
    if args.copy_calibration:
        copy_calibration(dev)
    if not torch.equal(k2[dest.long()].view(torch.int16), k_cache[ids.long()].view(torch.int16)):
        raise RuntimeError("imported K pages differ from the exported ones")
    exp_ms = [e[0].elapsed_time(e[1]) for e in ev]
    imp_ms = [e[1].elapsed_time(e[2]) for e in ev]
    step_ms = [e[0].elapsed_time(e[2]) for e in ev]
    moved = 2 * n * block * wl.elem_bytes          # K and V blocks, one direction
    t_exp = float(np.mean(exp_ms)) * 1e-3
    t_step = float(np.mean(step_ms)) * 1e-3
    achieved = 2 * moved / t_exp / 1e9             # read + written by the export
    return {
        "metric": TRANSFER_METRIC,
        "value": round(4 * moved / t_step / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[cid] + f"; all {n} pages in use exported and "
                   "imported at permuted ids", "pages": n, "bytes_per_page_kv": 2 * block * wl.elem_bytes,
                   "cache_flush_between_steps": flush_buf is not None,
                   "parallelism": "none (1 GPU)"},
        "kernels_ms": {"export": stats(exp_ms), "import": stats(imp_ms), "step": stats(step_ms)},
        "roofline": {"bound": "hbm", "kernel": "page_copy_kernel<true> (export)",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": 2 * moved,
                     "mean_launch_us": round(t_exp * 1e6, 2)},
    }


def run_pager_config(cid, args):
    """The native pager on the workload's shapes: every sequence's prompt
    (its cached tokens) admitted with synthetic token ids (sequences of a
    prefix group share their prefix ids, so the prefix pages are reused),
    then decode steps of one append per sequence plus the block tables; the
    policy model in oracle.pager timed on a bounded sample beside it."""
    import oracle.pager as opager

    import paged_kv_decode_pa_amd as pa
    from workloads import config_by_id, make_workload

    cfg = config_by_id(cid)
    wl = make_workload(cfg, share_prefix=not args.unshared)
    rng = np.random.default_rng(300 + cid)
    B, P = wl.num_seqs, wl.page_size
    lens = wl.context_lens.astype(np.int64) - 1   # prompt = the cached tokens
    shared = cfg.prefix_group_size > 0 and not args.unshared
    prefix_len = cfg.prefix_tokens if shared else 0
    stems = {}
    prompts = []
    for b in range(B):
        g = b // cfg.prefix_group_size if shared else -1 - b
        if g not in stems:
            stems[g] = rng.integers(0, 128000, size=prefix_len).astype(np.int32)
        tail = rng.integers(0, 128000, size=int(lens[b]) - len(stems[g])).astype(np.int32)
        prompts.append(np.concatenate([stems[g], tail]))
    steps = max(args.steps, 1) * 4
    grow = 2 * steps // P + 2  # pages each sequence gains over the two timed loops
    max_pages = int(wl.block_tables.shape[1]) + grow
    num_pages = int(wl.num_pages) + B * grow

    def native():
        pg = pa.Pager(num_pages, P, max_pages)
        t0 = time.perf_counter()
        for b in range(B):
            pg.add_sequence(b, prompts[b])
        t_admit = time.perf_counter() - t0
        ids = np.arange(B, dtype=np.int64)
        toks = rng.integers(0, 128000, size=(steps, B)).astype(np.int32)
        app = tuple(np.empty(B, dtype=np.int64) for _ in range(3))
        tab = (np.empty((B, max_pages), dtype=np.int32), np.empty(B, dtype=np.int32))
        # The engine's path: the library entry points called with the step's
        # buffers' addresses computed once.
        lib, h = pg._lib, pg._h
        a_ids, a_tok, a_tab, a_len = ids.ctypes.data, toks.ctypes.data, tab[0].ctypes.data, \
            tab[1].ctypes.data
        a_out = [x.ctypes.data for x in app]
        done = ctypes.c_int64()
        t0 = time.perf_counter()
        for k in range(steps):
            if lib.pa_pager_append_batch(h, a_ids, a_tok + 4 * B * k, B, *a_out,
                                         ctypes.byref(done)):
                raise RuntimeError("append_batch failed")
            if lib.pa_pager_block_tables(h, a_ids, B, a_tab, a_len):
                raise RuntimeError("block_tables failed")
        t_dec = (time.perf_counter() - t0) / steps
        # The same through the convenience binding (per-call marshalling).
        t0 = time.perf_counter()
        for k in range(steps):
            pg.append_batch(ids, toks[k], out=app)
            pg.block_tables(ids, out=tab)
        t_py = (time.perf_counter() - t0) / steps
        return t_admit, t_dec, t_py, pg.stats()

    def model(n_seqs, n_steps):
        m = opager.PagerModel(num_pages, P, max_pages)
        t0 = time.perf_counter()
        for b in range(n_seqs):
            m.add_sequence(b, prompts[b].tolist())
        t_admit = time.perf_counter() - t0
        ids = list(range(n_seqs))
        t0 = time.perf_counter()
        for k in range(n_steps):
            for b in ids:
                m.append(b, 1)
            m.block_tables(ids)
        return t_admit, (time.perf_counter() - t0) / n_steps

    native()  # warm-up (page faults, allocator)
    t_admit, t_dec, t_py, st = native()
    n_m = min(B, 8)
    m_admit, m_dec = model(n_m, 3)
    admitted = int(lens.sum())
    return {
        "metric": PAGER_METRIC,
        "value": round(1.0 / t_dec, 1),
        "unit": "steps/s",
        "n_gpus": 0, "steps": steps, "warmup": 1,
        "ms_per_step": round(t_dec * 1e3, 4),
        "higher_is_better": True, "scaling": "none", "vs_baseline": None,
        "dtype": "int32", "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[cid] + "; prompts = the cached tokens, token ids "
                   "synthetic, shared prefix ids per group", "batch": B, "page_size": P,
                   "num_pages": num_pages, "parallelism": "none (host)"},
        "admission": {"tokens": admitted, "seconds": round(t_admit, 6),
                      "tokens_per_s": round(admitted / t_admit, 1),
                      "prefix_hit_tokens": st["prefix_hit_tokens"]},
        "decode_step_us": round(t_dec * 1e6, 2),
        "decode_step_us_via_python_binding": round(t_py * 1e6, 2),
        "stats_after": st,
        "cpu_baseline": {"value": round(1.0 / (m_dec * B / n_m), 2), "unit": "steps/s",
                         "cores": 1, "kind": "oracle",
                         "sample": f"the policy model (oracle.pager) on the first {n_m} "
                                   f"sequences, 3 decode steps, scaled to {B} sequences; "
                                   f"admission {int(lens[:n_m].sum()) / m_admit:.0f} tokens/s"},
    }


def cpu_baseline(wl, budget_s, nb, t_step_gpu):
    """The fp64 oracle, as it stands, on a bounded sample of the same batch:
    whole sequences in batch order until the time budget is spent."""
    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
    store = np.float32 if wl.dtype == "f32" else np.uint16
    nan = np.float32("nan") if wl.dtype == "f32" else 0x7FC0
    P, Hkv, D = wl.page_size, wl.num_kv_heads, wl.head_dim
    k = np.full((wl.num_pages, Hkv, P, D), nan, dtype=store)
    v = np.full((wl.num_pages, Hkv, D, P), nan, dtype=store)
    k, v = oracle.cache_write(k, v, wl.prefill_key, wl.prefill_value, wl.prefill_slots, P)
    k, v = oracle.cache_write(k, v, wl.new_key, wl.new_value, wl.new_slots, P)
    per_token = 2 * wl.num_kv_heads * wl.head_dim * wl.elem_bytes
    done, tokens, t = 0, 0, 0.0
    while t < budget_s and done < 50 * wl.num_seqs:
        b = done % wl.num_seqs
        t0 = time.perf_counter()
        oracle.decode(wl.query[b:b + 1], k, v, wl.block_tables[b:b + 1],
                      wl.context_lens[b:b + 1], wl.scale, wl.page_size, wl.dtype)
        t += time.perf_counter() - t0
        tokens += int(wl.context_lens[b])
        done += 1
    gbs = tokens * per_token / t / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} sequence decodes cycling through the same {wl.num_seqs}-sequence "
                      f"batch in order ({tokens} cached tokens attended), fp64 NumPy, "
                      f"{t:.1f}s of CPU time",
            "seqs_per_s": round(done / t, 2),
            "host_cpus_visible": len(os.sched_getaffinity(0))}


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(decode attention shards by sequence or kv head with no exchange)",
              file=sys.stderr)
        sys.exit(2)
    if args.pager:
        print(json.dumps(run_pager_config(args.config, args)), flush=True)
        return
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import paged_kv_decode_pa_amd as pa

    pa.load()
    if args.chunk:
        print(json.dumps(run_chunk_config(args.config, args)), flush=True)
        return
    if args.transfer:
        print(json.dumps(run_transfer_config(args.config, args)), flush=True)
        return
    others = [c for c in (1, 2, 3, 4, 5) if c != args.config] if args.all else []
    for cid in others:
        print(json.dumps(run_config(cid, args)), file=sys.stderr, flush=True)
    print(json.dumps(run_config(args.config, args)), flush=True)


if __name__ == "__main__":
    main()
