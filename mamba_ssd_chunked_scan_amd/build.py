"""Builds libssd.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m mamba_ssd_chunked_scan_amd.build

Objects go to _build/ at the repository root; the library lands next to this
file so that the binding finds it.  Every HIP source is compiled with packed
fp32 instructions disabled.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libssd.so")
# plain copy / read / write kernels for the benchmark's HBM ceiling (not part of libssd)
BW_LIB = os.path.join(HERE, "libssd_bw.so")
BW_SOURCES = ["bw_probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["ssd_api.cpp", "generic.hip", "mfma.hip", "fused.hip", "backward.hip", "noalloc.hip"]
FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
# hipcc's host pass does not know the gfx feature name above and says so.
_NOISE = "'-packed-fp32-ops' is not a recognized feature"


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if _NOISE not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def _compile(src):
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    out = _run([HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
    return obj, out


def build(verbose: bool = False) -> str:
    """Builds libssd.so and the benchmark's bandwidth helper libssd_bw.so."""
    os.makedirs(OBJDIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        results = list(ex.map(_compile, SOURCES + BW_SOURCES))
    for _, out in results:
        if out.strip() and verbose:
            print(out)
    objs = [o for o, _ in results]
    for lib, srcs in ((LIB, SOURCES), (BW_LIB, BW_SOURCES)):
        tmp = lib + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp,
              *[objs[(SOURCES + BW_SOURCES).index(s)] for s in srcs]])
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
