"""Build tests/c/c_caller, the plain C caller of the library used by
tests/test_gpu_c_caller.py.  gcc with the HIP runtime's C headers; the program
finds libmxq.so next to the package through its run path."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "microscaling_weight_quantization_amd")
EXE = os.path.join(HERE, "c_caller")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-Wall", "-std=c99", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(HERE, "c_caller.c"), "-L", PKG, "-lmxq", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../microscaling_weight_quantization_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-o", EXE + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    build(verbose=True)
