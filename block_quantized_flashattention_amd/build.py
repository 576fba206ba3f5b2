"""Build libqfa.so (HIP, gfx950) in-tree with hipcc, and libqfa_ixcheck.so, a
host-only library that checks the forward kernel's address arithmetic (the
same index functions, compiled for the host) for the CPU tests.

Usage: python -m block_quantized_flashattention_amd.build  (or build() from Python).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqfa.so")
IXCHECK_LIB = os.path.join(PKG, "libqfa_ixcheck.so")
IXCHECK_SRC = "index_check.hip"

SOURCES = ["api.hip", "quant.hip", "prefill.hip", "decode.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    # Packed fp32 VALU ops stay off: the compiler otherwise forms them on its own.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build_ixcheck(verbose: bool = False) -> str:
    """Compile the host-only index checker into libqfa_ixcheck.so."""
    tmp = IXCHECK_LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, os.path.join(CSRC, IXCHECK_SRC),
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    pr = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    lines = [ln for ln in pr.stdout.decode(errors="replace").splitlines()
             if "packed-fp32-ops" not in ln]
    if lines and (verbose or pr.returncode):
        print("\n".join(lines), file=sys.stderr)
    if pr.returncode:
        raise RuntimeError(f"hipcc failed for {IXCHECK_SRC}")
    os.replace(tmp, IXCHECK_LIB)
    return IXCHECK_LIB


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source into libqfa.so next to this file, and the index
    checker. Always recompiles."""
    objs = []
    procs = []
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [hipcc(), *[f for f in HIPCC_FLAGS if f != "-shared"], "-c",
               "-I", INCLUDE, "-I", CSRC, os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, pr in procs:
        out, _ = pr.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the fp32 packing feature; that note is harmless.
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
        if lines and (verbose or pr.returncode):
            print("\n".join(lines), file=sys.stderr)
        if pr.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    build_ixcheck(verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
