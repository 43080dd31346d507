"""Build libmlafa.so (gfx950 only) in-tree with hipcc, and libmlapeaks.so beside it.

libmlafa.so is the attention library (include/mla_fa.h).  libmlapeaks.so holds the
achievable-peak micro-benchmarks (include/mla_peaks.h) that benchmarks use to state
roofline fractions against measured peaks; it is a library of its own so the attention
library exports only the path.

Every HIP source is compiled with packed-FP32 instructions disabled: hipcc -O3 would
otherwise fuse scalar float code into v_pk_{add,mul,fma}_f32.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libmlafa.so")
PEAKS_LIB = os.path.join(HERE, "libmlapeaks.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["attn.hip", "mha.hip", "proj.hip", "compact.hip", "api.hip"]
PEAKS_SOURCES = ["peaks.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
    cmd = [HIPCC, *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(noise))
    if verbose and noise:
        print("\n".join(noise), flush=True)
    return obj


def _link(objs: list, out: str, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every source and link both libraries; returns the attention library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PEAKS_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in SOURCES], LIB, verbose)
    _link([objs[s] for s in PEAKS_SOURCES], PEAKS_LIB, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
