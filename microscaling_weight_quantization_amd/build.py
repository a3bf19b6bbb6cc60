"""Build the gfx950 library (hipcc, in-tree).

``python -m microscaling_weight_quantization_amd.build`` writes
``libmxq.so`` next to this file, plus three variants of the same source used by
the build-variant tests: ``libmxq_fastmath.so`` (fast-math, denormals flushed),
``libmxq_o1.so`` (-O1) and ``libmxq_o0.so`` (-O0, no optimisation).  Every
step of the path is integer arithmetic, so all four builds must produce
identical bits.  ``libmxq_shapes.so`` holds the access-shape reference kernels
(``csrc/shapes.hip``) that bench.py times beside the library's kernels.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "mxq.hip")
INCLUDE = os.path.join(ROOT, "include")
ARCH = "gfx950"

# Packed fp32 instructions are kept out of every build; the library has no fp32 math anyway.
COMMON = ["--offload-arch=" + ARCH, "-std=c++17", "-fPIC", "-shared", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I" + INCLUDE]

VARIANTS = {
    "libmxq.so": ["-O3"],
    "libmxq_fastmath.so": ["-O3", "-ffast-math", "-fgpu-flush-denormals-to-zero"],
    "libmxq_o1.so": ["-O1"],
    "libmxq_o0.so": ["-O0"],
    "libmxq_shapes.so": ["-O3"],
}
SOURCES = {"libmxq_shapes.so": os.path.join(HERE, "csrc", "shapes.hip")}   # the others: SRC


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build_one(name: str, flags, verbose: bool = False) -> str:
    out = os.path.join(HERE, name)
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc()] + COMMON + flags + [SOURCES.get(name, SRC), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def build(variants=None, verbose: bool = False):
    names = list(VARIANTS) if variants is None else list(variants)
    with ThreadPoolExecutor(len(names)) as ex:
        return list(ex.map(lambda n: build_one(n, VARIANTS[n], verbose), names))


def library_path(name: str = "libmxq.so") -> str:
    return os.path.join(HERE, name)


def stale(name: str = "libmxq.so") -> bool:
    lib = library_path(name)
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    srcs = (SOURCES[name], os.path.join(INCLUDE, "mxq_shapes.h")) if name in SOURCES else (SRC, os.path.join(INCLUDE, "mxq.h"))
    return any(os.path.getmtime(p) > t for p in srcs)


if __name__ == "__main__":
    for p in build(sys.argv[1:] or None, verbose=True):
        print(p)
