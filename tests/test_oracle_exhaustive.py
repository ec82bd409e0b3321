"""The oracle's binary32 -> e4m3fn / e5m2 / bf16 / fp16 conversions checked
on all 2^32 binary32 inputs against an independent nearest-value rule
(tests/exhaustive/conv_exhaustive.c: grid rounding in binary64 from the
formats' definitions, outputs decoded from their bit fields).  About half a
minute on 8 threads."""
import os
import subprocess

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "exhaustive", "conv_exhaustive.c")


def test_all_binary32_inputs(tmp_path):
    exe = str(tmp_path / "conv_exhaustive")
    subprocess.run(["gcc", "-O2", "-std=c11", "-D_POSIX_C_SOURCE=200809L", "-ffp-contract=off", "-fno-fast-math",
                    SRC, "-o", exe, "-ldl", "-lpthread", "-lm"], check=True)
    lib = oracle.default().path
    threads = max(1, min(8, os.cpu_count() or 1))
    r = subprocess.run([exe, lib, str(threads)], capture_output=True, text=True, timeout=900)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count("4294967296 inputs, 0 mismatches") == 4, r.stdout
