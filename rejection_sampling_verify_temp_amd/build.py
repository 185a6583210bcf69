"""Build the verify-step HIP library (libspecverify.so) for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIB_DIR, "libspecverify.so")
SOURCES = ["sv_kernels.hip", "sv_api.hip", "sv_ngram.hip", "sv_tree.hip"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def command(out: str = LIB, extra=()) -> list[str]:
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    return [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
            "-shared", "-Wall", "-Wno-unused-function",
            # no packed fp32 instructions in device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC,
            *[os.path.join(CSRC, s) for s in SOURCES],
            "-o", out, f"-Wl,-rpath,{ROCM}/lib", *extra]


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile every source into `out`; `defines` are extra -D flags."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = command(tmp, extra=[f"-D{d}" for d in defines])
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
