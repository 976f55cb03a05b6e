"""Build libiq.so (HIP kernels for gfx950 + the C-ABI host code) in-tree, and the measurement
library libiq_probe.so (a read-only streaming kernel, include/iq_probe.h) beside it.

Usage: python -m compressed_space_decode_amd.build   (or via __graft_entry__.build()).
Always recompiles.  Objects go to compressed_space_decode_amd/_build/, the
library to compressed_space_decode_amd/libiq.so.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libiq.so")
SOURCES = ["iq_api.hip", "iq_quantize.hip", "iq_decode.hip", "iq_diag.hip", "iq_formats.hip", "iq_noalloc.hip",
           "iq_rotation.cpp"]
PROBE_LIB = os.path.join(PKG, "libiq_probe.so")
PROBE_SOURCES = ["iq_probe.hip"]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            # packed fp32 VALU ops are kept out of the generated code on purpose
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # no NaN semantics needed (infinities still are): lets min/max skip canonicalisation
            "-fno-honor-nans",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s%s" % (" ".join(cmd), res.stdout, res.stderr))
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed: %s\n%s%s" % (" ".join(cmd), res.stdout, res.stderr))
    os.replace(tmp, lib)


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print("built", LIB)
        print("built", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
