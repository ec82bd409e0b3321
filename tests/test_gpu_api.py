"""GPU: the page-level helpers of the Python binding (allocation wrappers over
the C ABI) against the oracle, and stream ordering on a non-default stream."""
import numpy as np
import pytest
import torch

import dequantize_amax_reduce_amd as fq
import oracle
from dequantize_amax_reduce_amd import workloads as W
from gpu_util import G, assert_f32_equal, assert_fp8_equal, assert_hp_equal, dev, host

pytestmark = pytest.mark.gpu


def test_cast_to_from_fp8_helpers():
    xf, xb, _ = W.tensor_rows_scaled(rows=64, cols=320, seed=31)
    for fmt, tfmt in (("e4m3", "e4m3fn"), ("e5m2", "e5m2")):
        for per_channel in (False, True):
            x = dev(xb, "bf16")
            q, s = fq.cast_to_fp8(x, fmt, per_channel_scale=per_channel)
            assert q.dtype == (torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2)
            op = oracle.cast_per_channel if per_channel else oracle.cast_per_tensor
            wq, ws = op(xb, "bf16", tfmt)
            assert_fp8_equal(host(q), wq, tfmt)
            assert_f32_equal(host(s), ws)
            y = fq.cast_from_fp8(q, s, torch.bfloat16, per_channel_scale=per_channel)
            deq = oracle.dequant_per_channel if per_channel else oracle.dequant_per_tensor
            assert_hp_equal(host(y), deq(wq, tfmt, ws, "bf16"), "bf16")
            # the out= forms write into the caller's tensors and return them;
            # cast_from_fp8 takes out's dtype (fp32 here), as torch.mul(..., out=out) does
            qo = G.full(x.shape, 0x55, dtype=torch.uint8, device="cuda:0")
            r, s2 = fq.cast_to_fp8(x, fmt, per_channel_scale=per_channel, out=qo)
            assert r is qo
            assert_fp8_equal(host(qo), wq, tfmt)
            assert_f32_equal(host(s2), ws)
            yo = G.full(x.shape, 7.0, dtype=torch.float32, device="cuda:0")
            r = fq.cast_from_fp8(q, s, torch.bfloat16, per_channel_scale=per_channel, out=yo)
            assert r is yo
            assert_f32_equal(host(yo), deq(wq, tfmt, ws, "f32"))
    with pytest.raises(TypeError):   # out of the other fp8 format
        fq.cast_to_fp8(dev(xb, "bf16"), "e4m3", out=G.empty(xb.shape, dtype=torch.float8_e5m2, device="cuda:0"))
    with pytest.raises(ValueError):  # out of the wrong size
        fq.cast_from_fp8(q, s, torch.bfloat16, out=G.empty(5, dtype=torch.float32, device="cuda:0"))


def test_per_token_and_weight_dequant_helpers():
    x, _ = W.group_cast_small()
    q, s = fq.per_token_cast_to_fp8(dev(x, "bf16"))
    wq, ws = oracle.cast_per_group128(x, "bf16", "e4m3fn")
    assert q.dtype == torch.float8_e4m3fn and tuple(s.shape) == (128, 4)
    assert_fp8_equal(host(q), wq, "e4m3fn")
    assert_f32_equal(host(s), ws)
    y = fq.per_token_cast_back(q, s)
    assert_hp_equal(host(y), oracle.dequant_per_group128(wq, "e4m3fn", ws, "bf16"), "bf16")
    c, sb = W.block_weight(M=300, N=640, seed=4)
    yw = fq.weight_dequant(dev(c).view(torch.float8_e4m3fn), dev(sb))
    assert yw.dtype == torch.bfloat16
    assert_hp_equal(host(yw), oracle.weight_dequant_block128(c, "e4m3fn", sb, "bf16"), "bf16")


def test_errors_surface_as_python_exceptions():
    x = G.zeros((4, 100), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(ValueError):
        fq.per_token_cast_to_fp8(x)
    with pytest.raises(TypeError):
        fq.cast_to_fp8(G.zeros(4, dtype=torch.int32, device="cuda:0"))
    with pytest.raises(ValueError):
        fq.fp8q_cast_per_group128(x.t(), G.empty((100, 4), dtype=torch.uint8, device="cuda:0"),
                                  G.empty(0, dtype=torch.float32, device="cuda:0"))


def test_non_default_stream_ordering():
    """Work enqueued on a side stream is ordered on that stream: the cast, the
    dequant and a dependent torch op all run on it with no host sync between."""
    x, _ = W.activation_outlier_channels(rows=256, cols=7168, seed=3)
    xd = dev(x, "bf16")
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        q, s = fq.per_token_cast_to_fp8(xd)
        y = fq.per_token_cast_back(q, s, torch.float32)
        ysum = y.double().sum()
    st.synchronize()
    wq, ws = oracle.cast_per_group128(x, "bf16", "e4m3fn")
    assert_fp8_equal(host(q), wq, "e4m3fn")
    wy = oracle.dequant_per_group128(wq, "e4m3fn", ws, "f32")
    assert_f32_equal(host(y), wy)
    assert float(ysum.cpu()) == pytest.approx(float(wy.astype(np.float64).sum()), rel=1e-12)
