"""GPU: the stated round-trip tolerance at full size.  For every element whose
scaled value lies in the fp8 normal range, |dequant(quant(x)) - x| / |x| is at
most half an fp8 ulp, 2^-(mantissa bits + 1) -- 2^-4 for e4m3fn, 2^-3 for
e5m2 -- up to the binary32 rounding of the scale and the product (a 2^-20
relative slack covers it).  Checked on the device's own outputs (fp32
dequant, so no output-type rounding enters) over the whole tensor: a property
that holds at any size, beside the bit-exact comparisons with the oracle."""
import pytest
import torch

import dequantize_amax_reduce_amd as fq
from dequantize_amax_reduce_amd import workloads as W
from gpu_util import G, dev

pytestmark = pytest.mark.gpu

MIN_NORMAL = {"e4m3fn": 2.0 ** -6, "e5m2": 2.0 ** -14}
TOL = {"e4m3fn": 2.0 ** -4, "e5m2": 2.0 ** -3}


def _max_rel(x, y, sinv_elem, fmt):
    xd, yd = x.reshape(-1).double(), y.reshape(-1).double()
    m = (xd.abs() / sinv_elem.reshape(-1).double()) >= MIN_NORMAL[fmt]
    rel = ((yd - xd).abs() / xd.abs())[m]
    return float(rel.max().item()), int(m.sum().item())


def test_group128_activation_roundtrip_bound():
    xh, _ = W.activation_outlier_channels()
    x = dev(xh, "bf16")
    R, C = x.shape
    q = G.empty((R, C), dtype=torch.uint8, device="cuda:0")
    s = G.empty((R, C // 128), dtype=torch.float32, device="cuda:0")
    y = G.empty((R, C), dtype=torch.float32, device="cuda:0")
    print("[case] group128 activation round-trip bound", flush=True)
    fq.fp8q_cast_per_group128(x, q, s, "e4m3fn")
    fq.fp8q_dequant_per_group128(q, s, y)
    torch.cuda.synchronize()
    worst, checked = _max_rel(x, y, s.repeat_interleave(128, dim=1), "e4m3fn")
    assert checked > 0.9 * R * C
    assert worst <= TOL["e4m3fn"] * (1 + 2.0 ** -20), worst


def test_per_tensor_gradient_roundtrip_bound():
    x = dev(W.gradient_payload(), "bf16")
    n = x.numel()
    q = G.empty(n, dtype=torch.uint8, device="cuda:0")
    s = G.empty(1, dtype=torch.float32, device="cuda:0")
    ws = G.empty(fq.fp8q_per_tensor_workspace_bytes() // 4, dtype=torch.int32, device="cuda:0")
    y = G.empty(n, dtype=torch.float32, device="cuda:0")
    print("[case] per-tensor gradient round-trip bound", flush=True)
    fq.fp8q_cast_per_tensor(x, q, s, ws, "e5m2")
    fq.fp8q_dequant_per_tensor(q, s, y, "e5m2")
    torch.cuda.synchronize()
    worst, checked = _max_rel(x, y, s, "e5m2")
    assert checked > 0.99 * n
    assert worst <= TOL["e5m2"] * (1 + 2.0 ** -20), worst
