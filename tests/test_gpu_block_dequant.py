"""GPU parity: 128x128 block weight dequant, through the C ABI, against the
CPU oracle, bit-exact.  The full-size case is the block-dequant workload:
e4m3fn [18432, 7168] with uniformly random non-NaN codes and float32 block
scales [144, 56] = 10**U(-4, -1), output bf16 (and fp32 for the fp32 path)."""
import numpy as np
import pytest
import torch

import dequantize_amax_reduce_amd as fq
import oracle
from dequantize_amax_reduce_amd import workloads as W
from gpu_util import G, assert_hp_equal, dev, empty_hp, host

pytestmark = pytest.mark.gpu


def _run(q, s, fmt, ydtype, q_offset=0, y_offset=0):
    M, N = q.shape
    qb = G.empty(M * N + q_offset, dtype=torch.uint8, device="cuda:0")
    qb[q_offset:] = dev(q.reshape(-1))
    yb = empty_hp(M * N + y_offset, ydtype)
    y = yb[y_offset:].view(M, N)
    print(f"[case] block128 dequant {fmt}->{ydtype} {M}x{N} q_off={q_offset} y_off={y_offset}", flush=True)
    fq.fp8q_weight_dequant_block128(qb[q_offset:].view(M, N), dev(s), y, fmt)
    torch.cuda.synchronize()
    return host(y)


def _check(M, N, fmt, ydtype, seed, **kw):
    q = W.fp8_codes_finite((M, N), fmt, seed=seed)
    rng = np.random.Generator(np.random.PCG64(seed + 1))
    s = (10.0 ** rng.uniform(-4, -1, size=((M + 127) // 128, (N + 127) // 128))).astype(np.float32)
    assert_hp_equal(_run(q, s, fmt, ydtype, **kw), oracle.weight_dequant_block128(q, fmt, s, ydtype), ydtype,
                    f"block dequant {M}x{N} {fmt} {ydtype}")


def test_block_weight_config_full_size():
    q, s = W.block_weight()
    assert s.shape == (144, 56)
    for ydtype in ("bf16", "f32"):
        assert_hp_equal(_run(q, s, "e4m3fn", ydtype), oracle.weight_dequant_block128(q, "e4m3fn", s, ydtype),
                        ydtype, f"block weight config -> {ydtype}")


@pytest.mark.parametrize("ydtype", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("fmt", ["e4m3fn", "e5m2"])
@pytest.mark.parametrize("M,N", [(1, 16), (128, 128), (300, 200), (257, 1040), (129, 17), (5, 1), (1000, 333)])
def test_block_dequant_shapes(M, N, fmt, ydtype):
    _check(M, N, fmt, ydtype, seed=M * 3 + N)


@pytest.mark.parametrize("q_offset,y_offset", [(1, 0), (0, 1), (8, 3)])
def test_block_dequant_unaligned(q_offset, y_offset):
    _check(256, 384, "e4m3fn", "bf16", seed=77, q_offset=q_offset, y_offset=y_offset)


def test_block_dequant_all_codes_extreme_scales():
    """every code (NaN included) against scales from 2^-149 to 2^127, so products
    cover binary32 subnormals, overflow to inf and bf16/fp16 rounding limits."""
    fmt_codes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))  # [256, 256]: 2x2 tiles
    s = np.array([[2.0 ** -149, 3.0e38], [1e-30, 0.7]], dtype=np.float32)
    for fmt in ("e4m3fn", "e5m2"):
        for ydtype in ("bf16", "f32", "f16"):
            got = _run(fmt_codes, s, fmt, ydtype)
            assert_hp_equal(got, oracle.weight_dequant_block128(fmt_codes, fmt, s, ydtype), ydtype,
                            f"all codes {fmt} {ydtype}")


def test_block_dequant_empty():
    for M, N in [(0, 128), (128, 0)]:
        q = G.empty((M, N), dtype=torch.uint8, device="cuda:0")
        s = G.empty(((M + 127) // 128, (N + 127) // 128), dtype=torch.float32, device="cuda:0")
        y = G.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
        fq.fp8q_weight_dequant_block128(q, s, y)
        torch.cuda.synchronize()
