"""Builds libquantspec.so (the HIP library behind include/quantspec.h) for gfx950 in-tree.

Each source is compiled to an object of its own, in parallel (the attention kernels are split
over one translation unit per call variant), then the objects are linked into the library.

Usage: python -m hierarchical_quantized_kv_amd.build_lib
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libquantspec.so")
SOURCES = [os.path.join(CSRC, f) for f in (
    "qs_attn_host.hip", "qs_attn_app.hip", "qs_attn_dev.hip", "qs_attn_gqa.hip",
    "qs_attn_split_host.hip", "qs_attn_split_app.hip", "qs_quant.hip", "qs_sample.hip",
    "qs_api.cpp")]
# Measurement helper for bench.py (the device's streaming-read ceiling); not part of the library.
PROBE_LIB = os.path.join(HERE, "libqs_readprobe.so")
PROBE_SOURCES = [os.path.join(CSRC, "read_probe.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
OBJ_DIR = os.path.join(HERE, "_build")

# Packed fp32 instructions are disabled for all device code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# the host compilation pass does not know the device-only feature name: that warning is dropped
NOISE = "'-packed-fp32-ops' is not a recognized feature for this target"


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if NOISE not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def _jobs() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16, int(os.environ.get("MAX_JOBS", "16"))))


def build(verbose: bool = False, extra: list[str] | None = None, out: str = LIB,
          sources: list[str] | None = None) -> str:
    srcs = sources or SOURCES
    tag = os.path.splitext(os.path.basename(out))[0]
    odir = os.path.join(OBJ_DIR, tag)
    os.makedirs(odir, exist_ok=True)
    objs = [os.path.join(odir, os.path.basename(s) + ".o") for s in srcs]
    cmds = [[HIPCC, *FLAGS, *(extra or []), "-c", s, "-o", o] for s, o in zip(srcs, objs)]
    with ThreadPoolExecutor(max_workers=_jobs()) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = out + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


def build_probe(verbose: bool = False) -> str:
    return build(verbose=verbose, out=PROBE_LIB, sources=PROBE_SOURCES)


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_probe(verbose=True))
