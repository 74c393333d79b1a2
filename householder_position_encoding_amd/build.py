"""Build libpath_attn.so (HIP, gfx950) in-tree with hipcc.

Every .hip file under csrc/ is compiled for gfx950 and linked into
``householder_position_encoding_amd/libpath_attn.so``.  Packed-fp32 VALU
instructions are disabled for all device code.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libpath_attn.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # gfx950 matrix instructions read and write ordinary VGPRs; without this
    # the accumulators are kept in AGPRs and copied to VGPRs for every
    # vector-unit use (the softmax, the bf16 repacking of the running tile).
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-result",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


# Per-file extra flags.  prep.hip: with packed-fp32 instructions disabled the
# gfx950 backend cannot select the <2 x float> bitcasts that the SLP vectoriser
# forms from pairs of bf16 -> float conversions, so SLP is turned off there.
EXTRA = {"prep.hip": ["-fno-slp-vectorize"]}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build_library(verbose: bool = False) -> str:
    """Compile every HIP source (in parallel) and link the shared library."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    procs = []
    objs = []
    for src in sources():
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src,
               "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT, text=True)))
    failed = False
    for src, p in procs:
        out, _ = p.communicate()
        msgs = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
        if msgs and (verbose or p.returncode != 0):
            print("\n".join(msgs), file=sys.stderr)
        if p.returncode != 0:
            failed = True
            print(f"hipcc failed on {src}", file=sys.stderr)
    if failed:
        raise RuntimeError("libpath_attn build failed")
    tmp = LIB_PATH + ".tmp"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs,
                    "-o", tmp], check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
