"""Builds libzf.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libzf.so")
SOURCES = ["zf_api.hip", "zf_codec.hip", "zf_attention.hip", "zf_probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         # packed fp32 ops (v_pk_*_f32) stay off: ordinary float code only
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str) -> str:
    obj = os.path.join(CSRC, "_obj_" + os.path.splitext(src)[0] + ".o")
    subprocess.check_call([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    return obj


def build(verbose: bool = False) -> str:
    with concurrent.futures.ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
