"""Host-side AddressSanitizer and UndefinedBehaviorSanitizer run of the C ABI and the oracle.

Builds, beside the normal artefacts (under _build/san, not shipped):
  * the C ABI's host code (glu_api.hip: argument validation and every launch planner, and
    glu_noalloc.hip) compiled with -fsanitize=address,undefined for the host pass only (each
    -fsanitize= after -Xarch_host; the GPU code is built exactly as usual), linked with the
    other, unchanged objects of the library into libglu_gemv_san.so;
  * the oracle (oracle/glu_oracle.c) with the same sanitizers, single-threaded;
then runs the CPU tests that exercise them (the boundary and planner tests and the oracle's pins)
in a child process with the sanitizer runtime preloaded and every report fatal.  Host only: the
GPU is never touched (the tests it runs never launch a kernel).

    python -m glu_mlp_gemv_amd.sanitize          # exit status 0 when clean
"""
from __future__ import annotations

import os
import subprocess
import sys

from . import build as hip_build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN_DIR = os.path.join(hip_build.BUILD_DIR, "san")
LLVM = "/opt/rocm/llvm/bin"
SAN_SOURCES = ("glu_api.hip", "glu_noalloc.hip")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
TESTS = ["tests/test_boundary.py", "tests/test_plan_sweep.py", "tests/test_oracle_pins.py"]


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    if res.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd[:3])} ... failed:\n{res.stdout[-4000:]}\n{res.stderr[-4000:]}")
    return res


def asan_runtime() -> str:
    return _run([os.path.join(LLVM, "clang"), "-print-file-name=libclang_rt.asan-x86_64.so"]).stdout.strip()


def build_sanitized() -> tuple:
    os.makedirs(SAN_DIR, exist_ok=True)
    # the library's other objects as the normal build makes them
    objs = []
    for src in hip_build.sources():
        name = os.path.basename(src)
        if name in SAN_SOURCES:
            obj = os.path.join(SAN_DIR, name + ".o")
            flags = [f for f in hip_build.HIP_FLAGS if f != "-O3"] + ["-O1", "-g"] + HOST_SAN
            _run([hip_build.HIPCC, *flags, "-c", src, "-o", obj])
        else:
            obj = os.path.join(hip_build.BUILD_DIR, name + ".o")
            if not os.path.exists(obj):
                hip_build._compile(src, False)
        objs.append(obj)
    lib = os.path.join(SAN_DIR, "libglu_gemv_san.so")
    _run([hip_build.HIPCC, f"--offload-arch={hip_build.ARCH}", "-shared", "-fPIC", "-shared-libsan",
          "-fsanitize=address,undefined", "-o", lib, *objs])
    oracle_src = os.path.join(ROOT, "oracle", "glu_oracle.c")
    olib = os.path.join(SAN_DIR, "liboracle_san.so")
    _run([os.path.join(LLVM, "clang"), "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
          "-shared", "-shared-libsan", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-Wall", "-Wextra", "-Werror", "-o", olib, oracle_src, "-lm"])
    return lib, olib


def main() -> int:
    lib, olib = build_sanitized()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": asan_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "GLU_GEMV_LIBRARY": lib,
        "GLU_ORACLE_LIBRARY": olib,
        "HIP_VISIBLE_DEVICES": "",
    })
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider", *TESTS]
    print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True)
    sys.stdout.write(res.stdout[-3000:])
    sys.stderr.write(res.stderr[-3000:])
    return res.returncode


if __name__ == "__main__":
    sys.exit(main())
