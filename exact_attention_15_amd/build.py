"""Build libattn.so (hipcc, gfx950) in-tree.

Usage: ``python -m exact_attention_15_amd.build`` or ``build_library()``.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_PATH = os.path.join(PKG, "libattn.so")

SOURCES = ["attn_api.hip", "fwd_mfma16.hip", "fwd_f32.hip", "bwd_mfma16.hip", "bwd_f32.hip",
           "unfused.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # Packed fp32 VALU forms are kept out of every kernel.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-Wno-inline-asm",
]


# The race-check build: the same sources with timing probes compiled in
# (ATTN_DELAY_PROBE), loaded only by the race tests, which compare its
# outputs with the library's bit for bit.
PROBE_LIB_PATH = os.path.join(PKG, "libattn_probe.so")


def build_library(verbose: bool = False, extra_flags=None) -> str:
    """Build libattn.so and the race-check libattn_probe.so (two hipcc runs
    in parallel)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    jobs = []
    for path, defs in ((LIB_PATH, []), (PROBE_LIB_PATH, ["-DATTN_DELAY_PROBE=1"])):
        tmp = path + ".tmp"
        cmd = [HIPCC, *FLAGS, *defs, *(extra_flags or []), "-I", os.path.join(ROOT, "include"),
               *srcs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((subprocess.Popen(cmd), tmp, path))
    failed = [path for proc, _, path in jobs if proc.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, f"hipcc for {failed}")
    for _, tmp, path in jobs:
        os.replace(tmp, path)
    return LIB_PATH


if __name__ == "__main__":
    build_library(verbose=True, extra_flags=sys.argv[1:])
