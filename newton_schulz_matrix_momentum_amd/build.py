"""Build libmuon.so (HIP for gfx950) in-tree with hipcc.

Usage: ``python -m newton_schulz_matrix_momentum_amd.build`` or ``build()``.
Objects go to ``_build/`` next to this file; the shared library is written to
``libmuon.so`` in this package directory.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmuon.so")
SOURCES = ["muon_host.cpp", "elementwise.hip", "ns_gemm.hip", "limuon.hip", "muon_static.hip"]
ARCH = "gfx950"

# Packed fp32 VALU ops are disabled for all device code.
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I" + INCLUDE, "-I" + CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; libmuon needs ROCm's hipcc to build")


def _compile(src: str, verbose: bool, defines=(), tag: str = "") -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + tag + ".o")
    cmd = [hipcc()] + HIPCC_FLAGS + ["-D" + d for d in defines]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, out))
    if verbose and out.strip():
        print(out, flush=True)
    return obj


def build(verbose: bool = False, defines=(), out: str = LIB) -> str:
    """Compile every source for gfx950 and link libmuon.so; returns its path.

    ``defines`` (``NAME=VALUE`` strings) and ``out`` build a tuning variant
    of the library elsewhere; the defaults build the shipped library."""
    os.makedirs(BUILD, exist_ok=True)
    tag = "" if out == LIB else "_" + str(abs(hash((tuple(defines), out))))
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, defines, tag), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
