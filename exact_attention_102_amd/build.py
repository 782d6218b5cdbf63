"""Builds libfa.so (the gfx950 kernels plus the C ABI of include/fa.h) in-tree.

    python -m exact_attention_102_amd.build        # or __graft_entry__.build()

Each translation unit is compiled by hipcc for gfx950 in parallel, then linked
into exact_attention_102_amd/libfa.so; the stand-alone measurement probes
(csrc/probe_atomic_dq.hip, csrc/probe_rates.hip) are built next to it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libfa.so")

SOURCES = ["fa_fwd.hip", "fa_bwd.hip", "fa_pad.hip", "fa_api.cpp"]
# measurement tools (stand-alone programs), not part of libfa.so
PROBES = ["probe_atomic_dq", "probe_rates"]
ARCH = "gfx950"
# Packed-fp32 instructions are disabled: the compiler must not emit v_pk_{add,mul,fma}_f32.
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfa.so)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compiling %s failed:\n%s" % (src, r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    """Compiles every source (always) and links libfa.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("linking libfa.so failed:\n%s" % r.stderr)
    os.replace(tmp, LIB_PATH)
    build_probe(verbose)
    return LIB_PATH


def build_probe(verbose: bool = False) -> None:
    """Builds the stand-alone measurement probes (csrc/probe_*.hip) next to the library."""
    for name in PROBES:
        cmd = [hipcc()] + FLAGS + ["-I" + CSRC, "-x", "hip", os.path.join(CSRC, name + ".hip"), "-o",
                                   os.path.join(PKG, name)]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("building %s failed:\n%s" % (name, r.stderr))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
