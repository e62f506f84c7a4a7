"""Build step of the HIP library: hipcc for gfx950, in-tree.

``python -m attention_forward_amd.build`` compiles ``csrc/`` into
``attention_forward_amd/libfa_mi355x.so``.  gfx950 is the only target.
Packed-fp32 instruction selection is switched off on purpose (the library
writes no packed fp32 code and lets the compiler emit none).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_NAME = "libfa_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["fa_api.cpp", "fa_kernels.hip"]  # the library; csrc/intake_probe.hip is a separate executable

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the softmax rescales O in place every few
    # tiles, which costs two extra moves per element when O lives in AGPRs.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is needed to build the attention library")


PROBE_SRC = os.path.join(CSRC, "intake_probe.hip")
PROBE_PATH = os.path.join(PKG, "intake_probe")


def build_probe(verbose: bool = False) -> str:
    """Compile the compute-unit intake probe (a standalone executable that
    bench.py --intake-probe runs); returns its path."""
    tmp = PROBE_PATH + ".tmp"
    flags = [f for f in HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    cmd = [hipcc(), *flags, PROBE_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed on the intake probe:\n" + "\n".join(msgs))
    os.replace(tmp, PROBE_PATH)
    return PROBE_PATH


def build(verbose: bool = False) -> str:
    """Compile every source into the shared library; returns its path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass of hipcc does not know the packed-fp32 feature; that
    # warning is expected and dropped.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB_PATH)
    build_probe(verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
