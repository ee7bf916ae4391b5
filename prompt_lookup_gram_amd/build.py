"""Build libpld.so (HIP kernels + C-ABI) for gfx950 with hipcc, in-tree.

Usage: python -m prompt_lookup_gram_amd.build
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpld.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-FP32 instruction selection is switched off for all device code.
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
             # the scan's leading kernel arguments arrive in SGPRs
             "-mllvm", "-amdgpu-kernarg-preload-count=8",
             "-Wall", "-Wextra", "-Werror", "-Wno-unused-command-line-argument",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", INCLUDE, "-I", CSRC]


# The scan's atomics are issued by one lane (a workgroup's merge, a
# wavefront's error bit): the compiler's atomic optimizer would wrap each in a
# wavefront-wide scan loop that only lengthens the merge on the critical path.
SOURCE_FLAGS = {"pld_kernels.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def sources():
    return [os.path.join(CSRC, "pld_kernels.hip"), os.path.join(CSRC, "pld_index.hip"),
            os.path.join(CSRC, "pld_control.hip"), os.path.join(CSRC, "pld_ngram.hip"),
            os.path.join(CSRC, "pld_api.cpp")]


def build(verbose: bool = False) -> str:
    """Compile every source and link libpld.so; returns its path."""
    objs = []
    for src in sources():
        obj = os.path.join(CSRC, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC, *HIP_FLAGS, *SOURCE_FLAGS.get(os.path.basename(src), []), *lang,
               "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
