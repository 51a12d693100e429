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
           "decode_reduce.hip", "chunk_mfma.hip", "page_transfer.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def command(out: str = LIB) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed fp32 vector ops stay off: the kernels are written for scalar fp32
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # matrix-core accumulators in ordinary VGPRs: the online-softmax rescale
        # multiplies them in place instead of copying through AGPRs
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-Wno-unused-command-line-argument",
        f"-I{INCLUDE}", f"-I{CSRC}",
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out,
    ]


def device_asm_command(source: str, out: str) -> list:
    """hipcc line that writes the gfx950 assembly of one source, compiled with
    the same flags as the library."""
    lib = command(out)
    flags = [c for c in lib if not c.endswith(".hip") and c not in ("-shared", "-fPIC")]
    return [*flags, "--cuda-device-only", "-S", os.path.join(CSRC, source)]


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


def build(verbose: bool = False) -> str:
    """Compile every source into libpa.so and libpa_pager.so (always recompiles)."""
    build_pager(verbose)
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
