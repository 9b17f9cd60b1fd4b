"""AddressSanitizer + UndefinedBehaviorSanitizer build of the host-side code, and the CPU test
suite run against it.

Builds, under _build/sanitize/ (not committed):
  libzf.so      the library with its host code (argument checks, sizing, the capacity model,
                launch set-up) instrumented; the gfx950 device code is built as usual
  liboracle.so  the C oracle, instrumented
  libsynth.so   the input generator, instrumented
then runs `pytest -m "not gpu"` with the three loaded in their place (ZF_LIB, ZF_ORACLE_LIB,
ZF_SYNTH_LIB) and clang's ASan runtime preloaded into the interpreter.  Any report fails the
run (UBSan findings abort).  Usage:  python -m decode_attention_encode_amd.sanitize
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

from . import build as hip_build

ROOT = os.path.dirname(hip_build.HERE)
OUT = os.path.join(ROOT, "_build", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-shared-libasan"]
C_SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-shared-libasan"]


def asan_runtime() -> str:
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise SystemExit("no clang ASan runtime under /opt/rocm/llvm")
    return found[-1]


def build_all() -> dict:
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for src in hip_build.SOURCES:
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        subprocess.check_call([hip_build.HIPCC, *hip_build.FLAGS, *HOST_SAN, "-g", "-c",
                               os.path.join(hip_build.CSRC, src), "-o", obj])
        objs.append(obj)
    libs = {"ZF_LIB": os.path.join(OUT, "libzf.so"),
            "ZF_ORACLE_LIB": os.path.join(OUT, "liboracle.so"),
            "ZF_SYNTH_LIB": os.path.join(OUT, "libsynth.so")}
    subprocess.check_call([hip_build.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SAN,
                           "-o", libs["ZF_LIB"], *objs])
    subprocess.check_call([CLANG, "-O1", "-g", "-fPIC", "-shared", "-std=c11", *C_SAN,
                           "-o", libs["ZF_ORACLE_LIB"], os.path.join(ROOT, "oracle", "zf_oracle.c"), "-lm"])
    subprocess.check_call([CLANG, "-O1", "-g", "-fPIC", "-shared", "-std=c11", *C_SAN,
                           "-o", libs["ZF_SYNTH_LIB"], os.path.join(ROOT, "synth", "synth.c"), "-lm"])
    return libs


def main() -> int:
    libs = build_all()
    env = dict(os.environ, **libs)
    env["LD_PRELOAD"] = asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-m", "not gpu",
           "-p", "no:cacheprovider"]
    return subprocess.call(cmd, env=env, cwd=ROOT)


if __name__ == "__main__":
    sys.exit(main())
