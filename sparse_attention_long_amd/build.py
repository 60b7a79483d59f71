"""Build the HIP libraries in-tree with hipcc for gfx950.

  sparse_attention_long_amd/libdsa.so   the DSA kernels and their C ABI
  synth/libdsa_synth.so                 the device-side input generator

Usage: python -m sparse_attention_long_amd.build [-v]
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed fp32 instructions are kept out of every code object.
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

DSA_SOURCES = ["dsa_api.hip", "indexer.hip", "topk.hip", "sparse_mla.hip", "quant.hip", "paged.hip", "masked_mha.hip", "validate.hip"]
LIB_DSA = os.path.join(HERE, "libdsa.so")
LIB_SYNTH = os.path.join(ROOT, "synth", "libdsa_synth.so")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed ({r.returncode}):\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err)


def build(verbose: bool = False, extra=()):
    csrc = os.path.join(HERE, "csrc")
    tmp = LIB_DSA + ".tmp"
    _run([HIPCC, *COMMON, *extra, *[os.path.join(csrc, s) for s in DSA_SOURCES], "-o", tmp], verbose)
    os.replace(tmp, LIB_DSA)
    tmp = LIB_SYNTH + ".tmp"
    _run([HIPCC, *COMMON, *extra, os.path.join(ROOT, "synth", "gen_device.hip"), "-o", tmp], verbose)
    os.replace(tmp, LIB_SYNTH)
    return LIB_DSA, LIB_SYNTH


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
