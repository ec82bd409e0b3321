"""CPU: the oracle (oracle/fp8_oracle.c) and the C ABI layer
(dequantize_amax_reduce_amd/csrc/fp8q_abi.cpp) built with
-fsanitize=address,undefined, each driven by its existing tests in a child
process with the AddressSanitizer runtime preloaded:

- every fast oracle pin (test_oracle_pins.py) on the sanitizer build of the
  oracle: an out-of-bounds access, a use of uninitialised shift or an integer
  overflow in the reference arithmetic aborts the child;
- every host ABI case (test_abi_host.py) on the sanitizer build of the ABI
  layer over host-only launcher stubs (tests/sanitize/fp8q_launch_stubs.cpp),
  including the valid calls that reach the launchers.

No GPU and no HIP runtime are involved; the stubs stand in for the kernels.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _asan_runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not path or not os.path.exists(path):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return os.path.realpath(path)


def _run(test_file, extra_env):
    env = dict(os.environ)
    env.update(extra_env)
    env["LD_PRELOAD"] = _asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=86"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=87"
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", test_file],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, f"{test_file} under ASan/UBSan (rc {r.returncode}):\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r.stdout


def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "libfp8_oracle_san.so")
    subprocess.run(["gcc", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall",
                    *SAN, "-I", os.path.join(ROOT, "oracle"), os.path.join(ROOT, "oracle", "fp8_oracle.c"),
                    "-o", lib, "-lm"], check=True)
    out = _run("tests/test_oracle_pins.py", {"ORACLE_LIB": lib})
    assert " passed" in out


def test_abi_host_under_asan_ubsan(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("g++ is not installed")
    lib = str(tmp_path / "libfp8q_abi_san.so")
    subprocess.run(["g++", "-std=c++17", "-fPIC", "-shared", "-Wall", *SAN, "-D__HIP_PLATFORM_AMD__",
                    "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "dequantize_amax_reduce_amd", "csrc"),
                    os.path.join(ROOT, "dequantize_amax_reduce_amd", "csrc", "fp8q_abi.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "fp8q_launch_stubs.cpp"), "-o", lib], check=True)
    out = _run("tests/test_abi_host.py", {"FP8Q_ABI_LIB": lib})
    assert " passed" in out and "skipped" not in out
