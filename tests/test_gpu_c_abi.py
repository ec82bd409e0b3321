"""GPU: a plain C caller (dequantize_amax_reduce_amd/examples/c_abi_example.c,
built next to libfp8q.so) uses the library through include/fp8q.h and the
HIP runtime API alone -- no torch, no Python -- and checks the results
against properties fixed by the definitions."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu
EXE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "dequantize_amax_reduce_amd",
                   "fp8q_c_example")


def test_plain_c_caller():
    assert os.path.exists(EXE), "build first: python dequantize_amax_reduce_amd/build.py"
    print("[case] plain C caller", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c_abi_example: OK" in r.stdout
