"""CPU-only sanitizer build of the host layer and of the oracle (for the CPU test tier).

The host layer (argument checks, FLOP model, per-stream state, planner: api.cpp and plan.cpp) is
compiled with g++ -fsanitize=address,undefined and linked, unsanitized, with the kernels' objects
from the regular hipcc build; the oracle's C source is compiled with gcc and the same
sanitizers.  Nothing here runs on a GPU: the CPU tests load these builds through HDP_LIB_PATH and
HDP_ORACLE_LIB_PATH with the sanitizer runtimes preloaded (see sanitizer_env).
"""
from __future__ import annotations

import os
import subprocess

from . import build as hip_build

SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-g", "-O1"]
OUT = os.path.join(hip_build.BUILD, "sanitized")
ROCM = "/opt/rocm"
HOST_SOURCES = ("api.cpp", "plan.cpp")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("%s failed:\n%s%s" % (cmd[0], r.stdout, r.stderr))


def runtime_libs():
    """The gcc sanitizer runtimes, which must be loaded before anything else in the process."""
    libs = []
    for name in ("libasan.so", "libubsan.so"):
        p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
        libs.append(p)
    return libs


def build() -> tuple:
    """Returns (host library, oracle library) paths of the sanitized builds."""
    os.makedirs(OUT, exist_ok=True)
    kernel_objs = [os.path.join(hip_build.BUILD, os.path.basename(s) + ".o") for s in hip_build.sources()
                   if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in kernel_objs):
        hip_build.build()
    host_objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(OUT, src + ".o")
        _run(["g++", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I", ROCM + "/include",
              "-I", hip_build.INCLUDE, "-I", hip_build.CSRC] + SAN + ["-c", os.path.join(hip_build.CSRC, src), "-o", obj])
        host_objs.append(obj)
    host = os.path.join(OUT, "libhdpattn_sanitized.so")
    _run(["g++", "-shared", "-o", host] + host_objs + kernel_objs + SAN[:1] +
         ["-L", ROCM + "/lib", "-Wl,-rpath," + ROCM + "/lib", "-lamdhip64"])
    root = os.path.dirname(hip_build.PKG)
    orc = os.path.join(OUT, "libhdp_oracle_sanitized.so")
    _run(["gcc", "-std=c11", "-fPIC", "-shared", "-fopenmp"] + SAN +
         ["-o", orc, os.path.join(root, "oracle", "hdp_oracle.c"), "-lm"])
    return host, orc


def sanitizer_env(host: str, orc: str) -> dict:
    env = dict(os.environ)
    env["LD_PRELOAD"] = " ".join(runtime_libs())
    # the interpreter itself is not instrumented and keeps memory until exit
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["HDP_LIB_PATH"] = host
    env["HDP_ORACLE_LIB_PATH"] = orc
    return env
