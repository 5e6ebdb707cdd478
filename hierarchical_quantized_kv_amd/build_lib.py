"""Builds libquantspec.so (the HIP library behind include/quantspec.h) for gfx950 in-tree.

Usage: python -m hierarchical_quantized_kv_amd.build_lib
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libquantspec.so")
SOURCES = [os.path.join(CSRC, "qs_kernels.hip"), os.path.join(CSRC, "qs_sample.hip"),
           os.path.join(CSRC, "qs_api.cpp")]
# Measurement helper for bench.py (the device's streaming-read ceiling); not part of the library.
PROBE_LIB = os.path.join(HERE, "libqs_readprobe.so")
PROBE_SOURCES = [os.path.join(CSRC, "read_probe.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 instructions are disabled for all device code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False, extra: list[str] | None = None, out: str = LIB,
          sources: list[str] | None = None) -> str:
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra or []), *(sources or SOURCES), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host compilation pass does not know the device-only feature name: drop that warning
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


def build_probe(verbose: bool = False) -> str:
    return build(verbose=verbose, out=PROBE_LIB, sources=PROBE_SOURCES)


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_probe(verbose=True))
