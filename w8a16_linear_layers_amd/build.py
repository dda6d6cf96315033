"""Build libfp8lin.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Usage: python -m w8a16_linear_layers_amd.build [-v]
Each source compiles to an object under ``_build/``; the objects link into
``libfp8lin.so`` next to this file. Cross-compiles without a GPU.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIBRARY = os.path.join(PKG, "libfp8lin.so")

SOURCES = ["api.hip", "quantize.hip", "gemm.hip", "swiglu.hip", "split.hip", "qknorm.hip"]
ARCH = "gfx950"

COMPILE_FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # keep float code off the packed-FP32 VALU ops
    "-Xclang",
    "-target-feature",
    "-Xclang",
    "-packed-fp32-ops",
    "-I" + INCLUDE,
    "-I" + CSRC,
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libfp8lin")
    return path


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("packed-fp32-ops", "not a recognized feature", "warning: argument unused")
    lines = [l for l in (r.stdout + r.stderr).splitlines() if not any(n in l for n in noise)]
    if r.returncode != 0:
        raise RuntimeError("command failed (%d): %s\n%s" % (r.returncode, " ".join(cmd), "\n".join(lines)))
    if verbose and lines:
        print("\n".join(lines))


def build(verbose=False, jobs=4):
    """Compile every source and link libfp8lin.so; always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([cc] + COMPILE_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIBRARY + ".tmp"
    _run([cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
