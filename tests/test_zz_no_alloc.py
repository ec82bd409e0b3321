"""GPU: fp8q_cast_per_tensor_noalloc (library-held device scratch, no
workspace argument) against fp8q_cast_per_tensor (caller workspace) through
the C ABI, bit-exactly, on calls in a row on one stream where each later call
has a smaller input than the one before.  The first call plants a large
maximum, so a later call that folded partials left in the shared scratch by
an earlier one would get a different scale.  The oracle checks both."""
import ctypes

import numpy as np
import pytest
import torch

import dequantize_amax_reduce_amd as fq
import oracle
from dequantize_amax_reduce_amd import workloads as W
from gpu_util import G, assert_f32_equal, assert_fp8_equal, dev, host

pytestmark = pytest.mark.gpu

# (n, element type, format, planted maximum or None, seed): each n smaller than the one before
CALLS = [
    ((1 << 24) + 3, "bf16", "e4m3fn", 30000.0, 71),
    (5000, "bf16", "e4m3fn", None, 72),
    (4099, "f32", "e5m2", None, 73),
    (1, "f16", "e4m3fn", None, 74),
]


def _input(n, dtype, peak, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    v = rng.standard_normal(n).astype(np.float32)
    if peak is not None:
        v[n - 1] = peak
    if dtype == "f32":
        return v
    if dtype == "bf16":
        return W.to_bf16_bits(v)
    return v.astype(np.float16).view(np.uint16)


def test_noalloc_matches_workspace_entry_point():
    st = torch.cuda.current_stream().cuda_stream
    ws = G.empty(fq.fp8q_per_tensor_workspace_bytes() // 4, dtype=torch.int32)
    for n, dtype, fmt, peak, seed in CALLS:
        print(f"[case] noalloc per-tensor n={n} {dtype} {fmt}", flush=True)
        xh = _input(n, dtype, peak, seed)
        x = dev(xh, dtype)
        q_ref, s_ref = G.empty(n, dtype=torch.uint8), G.empty(1, dtype=torch.float32)
        q_new, s_new = G.empty(n, dtype=torch.uint8), G.empty(1, dtype=torch.float32)
        f = fq.E4M3FN if fmt == "e4m3fn" else fq.E5M2
        dt = {"f32": fq.F32, "bf16": fq.BF16, "f16": fq.F16}[dtype]
        assert fq.lib.fp8q_cast_per_tensor(x.data_ptr(), dt, n, f, q_ref.data_ptr(), s_ref.data_ptr(),
                                           ws.data_ptr(), ctypes.c_void_p(st)) == fq.OK
        assert fq.lib.fp8q_cast_per_tensor_noalloc(x.data_ptr(), dt, n, f, q_new.data_ptr(), s_new.data_ptr(),
                                                   ctypes.c_void_p(st)) == fq.OK
        torch.cuda.synchronize()
        assert_fp8_equal(host(q_new), host(q_ref), fmt, f"q, n={n}")
        assert_f32_equal(host(s_new), host(s_ref), f"scale_inv, n={n}")
        wq, wsi = oracle.cast_per_tensor(xh, dtype, fmt)
        assert_fp8_equal(host(q_new), wq, fmt, f"q vs oracle, n={n}")
        assert_f32_equal(host(s_new), wsi, f"scale_inv vs oracle, n={n}")


def test_noalloc_empty_and_binding():
    s = G.full((1,), 7.0, dtype=torch.float32)
    fq.fp8q_cast_per_tensor_noalloc(G.empty(0, dtype=torch.bfloat16), G.empty(0, dtype=torch.uint8), s)
    torch.cuda.synchronize()
    assert float(host(s)[0]) == 1.0                       # cast_to_fp8's empty-tensor branch
    xh = _input(1000, "bf16", None, 75)
    q, si = G.empty(1000, dtype=torch.float8_e5m2), G.empty(1, dtype=torch.float32)
    fq.fp8q_cast_per_tensor_noalloc(dev(xh, "bf16"), q, si, "e5m2")
    torch.cuda.synchronize()
    wq, wsi = oracle.cast_per_tensor(xh, "bf16", "e5m2")
    assert_fp8_equal(host(q), wq, "e5m2", "binding q")
    assert_f32_equal(host(si), wsi, "binding scale_inv")


def test_noalloc_under_graph_capture():
    """The callers this entry point exists for include code under HIP graph
    capture: capture it (no allocation inside the capture), replay the graph
    four times with eager work that scribbles over the outputs in between, and
    check every replay against an eager call."""
    n = 3_000_005
    xh = _input(n, "bf16", None, 76)
    x = dev(xh, "bf16")
    q, si = G.empty(n, dtype=torch.uint8), G.empty(1, dtype=torch.float32)
    fq.fp8q_cast_per_tensor_noalloc(x, q, si, "e4m3fn")          # eager call (also warms the lookup)
    torch.cuda.synchronize()
    want_q, want_s = host(q).copy(), host(si).copy()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fq.fp8q_cast_per_tensor_noalloc(x, q, si, "e4m3fn", stream=s)
    torch.cuda.synchronize()
    for rep in range(4):
        q.fill_(0xA5)
        si.fill_(-1.0)
        torch.cuda.synchronize()
        print(f"[case] noalloc graph replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(q), want_q), rep
        assert np.array_equal(host(si).view(np.uint32), want_s.view(np.uint32)), rep
    wq, wsi = oracle.cast_per_tensor(xh, "bf16", "e4m3fn")
    assert_fp8_equal(want_q, wq, "e4m3fn", "graph q vs oracle")
    assert_f32_equal(want_s, wsi, "graph scale_inv vs oracle")
