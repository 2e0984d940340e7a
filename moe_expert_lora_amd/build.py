"""Build libmlora.so in-tree with hipcc for gfx950.

Usage: ``python -m moe_expert_lora_amd.build`` (or ``build()`` from Python).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmlora.so")
SOURCES = [os.path.join(CSRC, "mlora_host.cpp"), os.path.join(CSRC, "mlora_fold.hip")]
# measurement probes for bench.py (launch and read-pattern floors), a library of their own
PROBE_LIB = os.path.join(PKG, "libmlora_probe.so")
PROBE_SOURCES = [os.path.join(CSRC, "mlora_probe.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # keep hipcc from forming packed fp32 VALU ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # kernel arguments that lead with plain pointers / ints arrive in SGPRs
    # (the kernel keeps a prologue that loads them where firmware does not)
    "-mllvm", "-amdgpu-kernarg-preload-count=10",
    "-I", INCLUDE,
]


def _compile(sources, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [HIPCC, *FLAGS, *sources, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile moe_expert_lora_amd/libmlora.so (the fold) and libmlora_probe.so
    (bench.py's measurement probes); returns the fold library's path."""
    _compile(SOURCES, LIB, verbose)
    _compile(PROBE_SOURCES, PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
