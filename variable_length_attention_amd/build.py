"""Builds libhdpattn.so in-tree with hipcc for gfx950 (no JIT, no torch extension machinery)."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libhdpattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU instructions are kept out of the device code on purpose.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                # MFMA accumulators in VGPRs: the online-softmax rescale touches the output
                # accumulator with VALU ops, and AGPR accumulators would be copied every step.
                "-mllvm", "-amdgpu-mfma-vgpr-form",
                # Work-queue pops are single-lane atomics whose result is needed only at the end
                # of an item; the atomic optimizer would rewrite them into a form that waits for
                # the result right after the atomic.
                "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
                "-I", INCLUDE, "-I", CSRC]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + DEVICE_FLAGS + ["-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-x", "hip"] + DEVICE_FLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int = 8) -> str:
    """Compile every HIP/C++ source under csrc/ and link variable_length_attention_amd/libhdpattn.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
