"""Build libfsa.so in-tree with hipcc for gfx950.

    python -m frame_windowed_block_amd.build [--asm]

The library is one shared object: the host-side plan and argument checks
(plain C++) and the HIP kernels, compiled for gfx950 only. Packed-fp32 VALU
instructions are disabled on the device (``-packed-fp32-ops``); hipcc's host
pass warns that it does not know that feature, which is harmless.
``--asm`` also writes the gfx950 assembly of the kernels next to the sources
(``csrc/fsa_kernels-gfx950.s``, not committed) for inspection.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfsa.so")
SOURCES = ["fsa_plan.cpp", "fsa_api.cpp", "fsa_kernels.hip", "fsa_preattn.hip"]
ARCH = "gfx950"

DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
                "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfsa)")


def build(verbose: bool = False, asm: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *COMMON_FLAGS, *DEVICE_FLAGS, "-shared", "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(x for x in (res.stdout, res.stderr) if x)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    if asm:
        s_out = os.path.join(CSRC, f"fsa_kernels-{ARCH}.s")
        cmd = [hipcc(), *COMMON_FLAGS, *DEVICE_FLAGS, "--cuda-device-only", "-S", "-o", s_out,
               os.path.join(CSRC, "fsa_kernels.hip")]
        subprocess.run(cmd, check=True, capture_output=not verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, asm="--asm" in sys.argv))
