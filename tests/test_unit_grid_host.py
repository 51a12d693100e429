"""The four-wave decode units' grid (unit_of / unit_pages, pa_device.hpp),
compiled for the host and enumerated on the CPU.

With a shared prefix, a sequence's suffix units count partitions from its
first_partition and the grid holds a bound on how many follow.  A bound of
max_num_partitions ("always enough") or an overestimate must never give a
unit whose partition index reaches max_num_partitions: its partial row would
be another head's (or past the buffer).  Every partition that the merge
counts for a sequence (ceil(L / partition size), at most max_num_partitions)
and that is not a shared one must have exactly one unit per kv head.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import numpy as np
import pytest

from paged_kv_decode_pa_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def grid_exe(tmp_path_factory):
    if shutil.which(B.hipcc()) is None and not os.path.exists(B.hipcc()):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("grid") / "host_unit_grid")
    cmd = [B.hipcc(), "-x", "hip", f"--offload-arch={B.ARCH}", "-O1", "-std=c++17",
           f"-I{B.INCLUDE}", f"-I{B.CSRC}", os.path.join(HERE, "host_unit_grid.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return exe


def enumerate_grid(exe, lens, Hkv, G, NP, GP, PP, MP, first=None):
    head = f"{len(lens)} {Hkv} {G} {NP} {GP} {PP} {MP} {int(first is not None)}\n"
    body = " ".join(map(str, lens)) + "\n"
    if first is not None:
        body += " ".join(map(str, first)) + "\n"
    res = subprocess.run([exe], input=head + body, capture_output=True, text=True, check=True)
    units, skipped = [], 0
    for line in res.stdout.splitlines():
        f = line.split()
        if f[0] == "skip":
            skipped += 1
        else:
            units.append(tuple(int(x) for x in f[1:]))
    return units, skipped


CASES = [
    # lens, first partitions, NP, grid bound, PP, max pages per seq
    ([1000, 700, 40, 2047], [2, 2, 0, 3], 4, 4, 16, 64),     # bound 0 -> max_num_partitions
    ([1000, 700, 40, 2047], [2, 2, 0, 3], 4, 6, 16, 64),     # an overestimate
    ([5000, 300], [1, 1], 3, 3, 16, 400),                   # L far past NP partitions
    ([256, 257, 0, 16], None, 2, 2, 8, 64),                  # no shared prefix
    ([9000, 100], [2, 0], 4, 4, 16, 200),                    # L past the table's width
]


@pytest.mark.parametrize("lens,first,NP,GP,PP,MP", CASES)
def test_suffix_units_stay_inside_the_partial_rows(grid_exe, lens, first, NP, GP, PP, MP):
    Hkv, G = 2, 4
    units, skipped = enumerate_grid(grid_exe, lens, Hkv, G, NP, GP, PP, MP, first)
    assert len(units) + skipped == len(lens) * Hkv * GP
    seen = {}
    for u, seq, kvh, part, has, lo, hi, merged in units:
        assert 0 <= part < NP, (u, seq, part)
        f = 0 if first is None else min(max(first[seq], 0), NP)
        assert part >= f
        seen.setdefault((seq, kvh), []).append(part)
        n_pages = min(-(-lens[seq] // 16), MP)
        if has:
            assert lo == part * PP and hi == min(lo + PP, n_pages) and lo < hi
        ps = 16 * PP
        assert merged == min(-(-lens[seq] // ps), NP)
    for seq, L in enumerate(lens):
        f = 0 if first is None else min(max(first[seq], 0), NP)
        want = set(range(f, min(-(-L // (16 * PP)), NP)))
        for kvh in range(Hkv):
            got = seen.get((seq, kvh), [])
            assert len(got) == len(set(got))
            assert want <= set(got), (seq, kvh, sorted(want - set(got)))
