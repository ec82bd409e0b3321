"""GPU: the hardware fp8 encode, through the C ABI, on every one of the 2^32
binary32 bit patterns.  fp8q_cast_with_amax with amax = fp8_max makes the
scale exactly 1, so q = fp8(x) by the saturating rule; the codes must equal
the oracle's (NaN compared by class).  Inputs are built on the device from
their indices, in chunks of 2^28; the oracle runs on the host in parallel
ctypes calls."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import dequantize_amax_reduce_amd as fq
import oracle
from gpu_util import G, FP8_NAN_CLASS

pytestmark = pytest.mark.gpu
FP8_MAX = {"e4m3fn": 448.0, "e5m2": 57344.0}
CHUNK = 1 << 28


def _oracle_encode(v, fmt, pool, parts):
    out = np.empty(v.size, np.uint8)
    step = (v.size + parts - 1) // parts

    def one(i):
        out[i:i + step] = oracle.fp8_encode(v[i:i + step], fmt)
    list(pool.map(one, range(0, v.size, step)))
    return out


@pytest.mark.parametrize("fmt", ["e4m3fn", "e5m2"])
def test_every_binary32_input(fmt):
    L = oracle.default()
    assert L is not None
    threads = max(1, min(16, os.cpu_count() or 1))
    amax = torch.tensor([FP8_MAX[fmt]], dtype=torch.float32, device="cuda:0")
    scale = G.empty(1, dtype=torch.float32, device="cuda:0")
    q = G.empty(CHUNK, dtype=torch.uint8, device="cuda:0")
    with ThreadPoolExecutor(threads) as pool:
        for c0 in range(0, 1 << 32, CHUNK):
            print(f"[case] {fmt} inputs 0x{c0:08X}..0x{c0 + CHUNK - 1:08X}", flush=True)
            x = torch.arange(c0, c0 + CHUNK, dtype=torch.int64, device="cuda:0").to(torch.int32).view(torch.float32)
            fq.fp8q_cast_with_amax(x, amax, q, scale, fmt)
            got = q.cpu().numpy()
            del x
            v = np.arange(c0, c0 + CHUNK, dtype=np.uint32).view(np.float32)
            want = _oracle_encode(v, fmt, pool, threads * 4)
            assert float(scale.item()) == 1.0
            nan = FP8_NAN_CLASS[fmt](want) & FP8_NAN_CLASS[fmt](got)
            bad = np.nonzero((got != want) & ~nan)[0]
            assert bad.size == 0, (fmt, hex(c0 + int(bad[0])), int(got[bad[0]]), int(want[bad[0]]), bad.size)
