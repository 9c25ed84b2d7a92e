"""Build libbgg.so (the C-ABI library) and libbgg_probe.so (the benchmark's
streaming probe kernels) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbgg.so")
PROBE_LIB = os.path.join(HERE, "libbgg_probe.so")
PROBE_SOURCES = ["probe_stream.hip"]
SOURCES = ["bgg_host.cpp", "bgg_rotate.hip", "bgg_gemv.hip", "bgg_gemv_noalloc.hip", "bgg_mxv.hip", "bgg_unpack.hip", "bgg_gemm.hip",
           "bgg_ternarize.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 VALU forms are kept out of the generated code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    """Compile every source and link libbgg.so and libbgg_probe.so; always
    rebuilds."""
    _link(SOURCES, LIB, verbose)
    _link(PROBE_SOURCES, PROBE_LIB, verbose)
    return LIB


def _link(sources, lib, verbose):
    objs = []
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    for src in sources:
        obj = os.path.join(build_dir, src + ".o")
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
               "-Wall", "-Wno-unused-function", *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
        objs.append(obj)
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs, "-lpthread"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, lib)


if __name__ == "__main__":
    print(build(verbose=True))
