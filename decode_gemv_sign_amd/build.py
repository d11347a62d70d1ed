"""Build libwc.so (gfx950) from csrc/*.hip with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 instructions
disabled, into objects under _build/, then linked into libwc.so next to
this file.  `python -m decode_gemv_sign_amd.build` rebuilds.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libwc.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-I" + os.path.join(ROOT, "include"),
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str, build_dir: str, defines) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    subprocess.check_call([HIPCC, *FLAGS, *["-D" + d for d in defines], "-c", src, "-o", obj])
    return obj


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile and link; `defines` (NAME=VALUE) override compile-time tuning
    constants, `out` places the library elsewhere (for tuning sweeps)."""
    build_dir = BUILD if out == LIB else out + ".build"
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, defines), srcs))
    tmp = out + ".tmp"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, out)
    LIB_OUT = out
    if verbose:
        print("built", LIB_OUT)
    return LIB_OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
