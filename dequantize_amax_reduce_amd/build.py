"""Build the HIP library libfp8q.so in-tree with hipcc for gfx950.

    python dequantize_amax_reduce_amd/build.py

(run by path: importing the package loads libfp8q.so, which may be missing
or stale before the build).

Flags that matter for the numerics:
  -ffp-contract=off   no FMA contraction of the binary32 products
  -Xclang -target-feature -Xclang -packed-fp32-ops
                      no v_pk_{add,mul,fma}_f32 (scalar VALU fp32 only)
  no -ffast-math / -fgpu-flush-denormals-to-zero: IEEE division and fp32
  denormals stay on (correctly rounded scale = fp8_max / amax).

A flag that matters for speed only:
  -mllvm -amdgpu-kernarg-preload-count=16
                      gfx950 preloads the first kernel arguments into SGPRs at
                      dispatch, so a wave starts without the kernarg-segment
                      load round trip (3-6 % on the 10-25 us launches, nothing
                      measurable on the long ones).  The code object keeps a
                      prologue that loads them the old way for firmware that
                      does not preload.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfp8q.so")
SOURCES = [os.path.join(CSRC, f) for f in ("fp8q_kernels.hip", "fp8q_shift.hip", "fp8q_abi.cpp")]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libfp8q.so)")


def build(verbose: bool = False) -> str:
    """Compile every source to an object, in parallel (one hipcc per
    translation unit), then link libfp8q.so."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor
    flags = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
             "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-kernarg-preload-count=16",
             "-Wall", "-I", INCLUDE, "-I", CSRC]
    # the host pass does not know the device-only feature name; that warning is expected
    noise = "'-packed-fp32-ops' is not a recognized feature"

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(cmd)}\n{msgs}")
        if msgs.strip() and verbose:
            print(msgs)

    with tempfile.TemporaryDirectory(prefix="fp8q_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in SOURCES]
        with ThreadPoolExecutor(len(SOURCES)) as ex:
            for f in [ex.submit(run, [hipcc(), *flags, "-c", src, "-o", obj]) for src, obj in zip(SOURCES, objs)]:
                f.result()
        tmp = LIB + ".tmp%d" % os.getpid()
        run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    build_example(verbose)
    return LIB


EXAMPLE_SRC = os.path.join(PKG, "examples", "c_abi_example.c")
EXAMPLE = os.path.join(PKG, "fp8q_c_example")


def build_example(verbose: bool = False) -> str:
    """A plain C program that calls the library through include/fp8q.h and
    the HIP runtime API only (no torch, no C++), linked next to libfp8q.so."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cmd = [os.environ.get("CC", "gcc"), "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", INCLUDE, EXAMPLE_SRC, "-o", EXAMPLE,
           "-L", PKG, "-lfp8q", "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the C example failed ({r.returncode}):\n{r.stdout}{r.stderr}")
    return EXAMPLE


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
