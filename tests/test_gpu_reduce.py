"""GPU parity: the reduce step of the fp8-compressed reduce-scatter /
all-reduce (fp8q_dequant_sum, fp8q_dequant_sum_requant) against the CPU
oracle, bit-exact (NaN by class).  Chunks are seeded synthetic received
chunks (finite fp8 codes, one scale_inv per chunk)."""
import numpy as np
import pytest
import torch

import dequantize_amax_reduce_amd as fq
import oracle
from dequantize_amax_reduce_amd import workloads as W
from gpu_util import G, assert_f32_equal, assert_fp8_equal, assert_hp_equal, dev, empty_hp, host

pytestmark = pytest.mark.gpu


def _sum(q, s, fmt, ydtype, average, requant, q_offset=0, y_offset=0, qo_offset=0):
    Wn, n = q.shape
    qb = G.empty(Wn * n + q_offset, dtype=torch.uint8, device="cuda:0")
    qb[q_offset:] = dev(q.reshape(-1))
    qd = qb[q_offset:].view(Wn, n)
    y = empty_hp(n + y_offset, ydtype)[y_offset:]
    print(f"[case] dequant_sum W={Wn} n={n} {fmt}->{ydtype} avg={average} requant={requant} q_off={q_offset} "
          f"y_off={y_offset} qo_off={qo_offset}", flush=True)
    if not requant:
        fq.fp8q_dequant_sum(qd, dev(s), y, fmt, average)
        torch.cuda.synchronize()
        return host(y), None, None
    qo = G.empty(n + qo_offset, dtype=torch.uint8, device="cuda:0")[qo_offset:]
    so = G.full((1,), -3.0, dtype=torch.float32, device="cuda:0")
    ws = G.full((fq.fp8q_per_tensor_workspace_bytes() // 4,), 12345, dtype=torch.int32, device="cuda:0")
    fq.fp8q_dequant_sum_requant(qd, dev(s), y, qo, so, ws, fmt, average)
    torch.cuda.synchronize()
    return host(y), host(qo), host(so)


def _check(q, s, fmt, ydtype, average, requant, **kw):
    y, qo, so = _sum(q, s, fmt, ydtype, average, requant, **kw)
    wy, wq, ws = oracle.dequant_sum_requant(q, fmt, s, ydtype, average)
    assert_hp_equal(y, wy, ydtype, f"sum {fmt} {ydtype} avg={average}")
    if requant:
        assert_fp8_equal(qo, wq, fmt, "requant q")
        assert_f32_equal(so, ws, "requant scale_inv")


@pytest.mark.parametrize("ydtype", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("fmt", ["e5m2", "e4m3fn"])
@pytest.mark.parametrize("Wn,n", [(1, 1), (2, 7), (3, 8), (5, 1000), (8, 4099), (4, 1 << 16), (8, (1 << 20) + 3)])
def test_dequant_sum_shapes(Wn, n, fmt, ydtype):
    q, s = W.received_chunks(Wn, n, fmt, seed=Wn * 31 + n % 97)
    for average in (False, True):
        _check(q, s, fmt, ydtype, average, requant=False)
    _check(q, s, fmt, ydtype, True, requant=True)


@pytest.mark.parametrize("q_offset", [1, 4])
def test_dequant_sum_unaligned(q_offset):
    q, s = W.received_chunks(3, 1000, "e5m2", seed=3)
    _check(q, s, "e5m2", "bf16", True, requant=True, q_offset=q_offset)


@pytest.mark.parametrize("ydtype,y_offset,qo_offset", [("bf16", 1, 0), ("bf16", 3, 2), ("f32", 1, 1), ("f16", 2, 3)])
def test_dequant_sum_requant_unaligned_outputs(ydtype, y_offset, qo_offset):
    """y (the sum, which the re-cast reads) and the re-cast's codes as views
    part-way into their buffers: the re-cast then takes the shifted cast
    kernel, which folds the 64 amax slots (128 bytes apart) the sum left in
    the workspace.  Sizes span several chunks of that kernel and a ragged
    tail."""
    for n in (1000, 300007):
        q, s = W.received_chunks(4, n, "e5m2", seed=n % 101 + y_offset)
        _check(q, s, "e5m2", ydtype, True, requant=True, y_offset=y_offset, qo_offset=qo_offset)


def test_dequant_sum_special_values():
    """-0 chunks sum to +0; NaN and inf codes propagate; huge scales overflow
    to inf in the type; an all-zero sum re-casts with the zero-tensor scale."""
    for fmt in ("e4m3fn", "e5m2"):
        q = np.full((3, 64), 0x80, np.uint8)
        q[1, 5] = 0x7F                            # NaN (both formats)
        if fmt == "e5m2":
            q[2, 9] = 0x7C                        # +inf
        q[0, 20:30] = 0x38
        s = np.array([1.0, 2.0, 3.0e38], np.float32)
        for ydtype in ("bf16", "f32", "f16"):
            _check(q, s, fmt, ydtype, False, requant=False)
            _check(q, s, fmt, ydtype, True, requant=True)
        z = np.full((2, 40), 0x80, np.uint8)
        _check(z, np.ones(2, np.float32), fmt, "bf16", True, requant=True)


def test_dequant_sum_empty():
    q = G.empty((3, 0), dtype=torch.uint8, device="cuda:0")
    s = G.ones(3, dtype=torch.float32, device="cuda:0")
    y = G.empty(0, dtype=torch.bfloat16, device="cuda:0")
    qo = G.empty(0, dtype=torch.uint8, device="cuda:0")
    so = G.zeros(1, dtype=torch.float32, device="cuda:0")
    ws = G.empty(fq.fp8q_per_tensor_workspace_bytes() // 4, dtype=torch.int32, device="cuda:0")
    fq.fp8q_dequant_sum(q, s, y, "e5m2")
    fq.fp8q_dequant_sum_requant(q, s, y, qo, so, ws, "e5m2", True)
    torch.cuda.synchronize()
    assert host(so)[0] == 1.0


def test_gradient_bucket_reduce_full_size():
    """One rank's reduce step of the DDP hook on a 2^28-element bf16 bucket
    over 8 ranks: 8 received e5m2 chunks of 2^25 -> bf16 sum / 8 -> e5m2."""
    q, s = W.received_chunks(8, 1 << 25, "e5m2", seed=6)
    _check(q, s, "e5m2", "bf16", True, requant=True)


def test_reduce_helper():
    q, s = W.received_chunks(4, 5000, "e4m3fn", seed=8)
    qd = dev(q).view(torch.float8_e4m3fn)
    y = fq.reduce_fp8_chunks(qd, dev(s), torch.bfloat16)
    torch.cuda.synchronize()
    assert_hp_equal(host(y), oracle.dequant_sum(q, "e4m3fn", s, "bf16"), "bf16")
    y, qo, so = fq.reduce_fp8_chunks(qd, dev(s), torch.float32, average=True, requant=True)
    torch.cuda.synchronize()
    wy, wq, ws = oracle.dequant_sum_requant(q, "e4m3fn", s, "f32", True)
    assert_hp_equal(host(y), wy, "f32")
    assert_fp8_equal(host(qo), wq, "e4m3fn")
    assert_f32_equal(host(so), ws)
