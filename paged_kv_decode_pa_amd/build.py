"""Build libpa.so (gfx950) in-tree with hipcc.

    python -m paged_kv_decode_pa_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpa.so")
PAGER_LIB = os.path.join(PKG, "libpa_pager.so")
PAGER_SOURCES = ["pager.cpp"]
SOURCES = ["pa_api.hip", "reshape_and_cache.hip", "decode_mfma.hip", "decode_valu.hip",
           "decode_reduce.hip", "chunk_mfma.hip", "chunk_lds.hip", "page_transfer.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


OBJ_DIR = os.path.join(PKG, "_build")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 vector ops stay off: the kernels are written for scalar fp32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs: the online-softmax rescale
    # multiplies them in place instead of copying through AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def command(out: str = LIB) -> list:
    """One hipcc line that compiles every source and links libpa.so."""
    return [hipcc(), *FLAGS, "-shared", *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]


def object_command(source: str) -> list:
    obj = os.path.join(OBJ_DIR, os.path.splitext(source)[0] + ".o")
    return [hipcc(), *FLAGS, "-c", os.path.join(CSRC, source), "-o", obj]


def link_command(out: str) -> list:
    objs = [os.path.join(OBJ_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    return [hipcc(), f"--offload-arch={ARCH}", "-fPIC", "-shared", *objs, "-o", out]


def device_asm_command(source: str, out: str) -> list:
    """hipcc line that writes the gfx950 assembly of one source, compiled with
    the same flags as the library."""
    flags = [c for c in FLAGS if c != "-fPIC"]
    return [hipcc(), *flags, "--cuda-device-only", "-S", os.path.join(CSRC, source), "-o", out]


def pager_command(out: str = PAGER_LIB) -> list:
    """The host-only page pool owner: plain C++17, no HIP."""
    cxx = os.environ.get("CXX", "g++")
    return [cxx, "-std=c++17", "-O2", "-Wall", "-Wextra", "-fPIC", "-shared", f"-I{INCLUDE}",
            *[os.path.join(CSRC, s) for s in PAGER_SOURCES], "-o", out]


def build_pager(verbose: bool = False) -> str:
    tmp = PAGER_LIB + ".tmp"
    cmd = pager_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"pager build failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, PAGER_LIB)
    return PAGER_LIB


def _run(cmd: list, verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")


def build(verbose: bool = False) -> str:
    """Compile every source into libpa.so and libpa_pager.so (always
    recompiles): one object per source, compiled in parallel, then linked."""
    from concurrent.futures import ThreadPoolExecutor

    build_pager(verbose)
    os.makedirs(OBJ_DIR, exist_ok=True)
    jobs = max(1, min(len(SOURCES), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(jobs) as pool:
        for f in [pool.submit(_run, object_command(s), verbose) for s in SOURCES]:
            f.result()
    tmp = LIB + ".tmp"
    _run(link_command(tmp), verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
