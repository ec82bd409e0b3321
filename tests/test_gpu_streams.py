"""GPU: the library keeps no global state, so calls on two streams that run
at the same time (each per-tensor call with its own workspace) give the same
bits as the oracle.  Both streams are ordinary default-priority streams."""
import numpy as np
import pytest
import torch

import dequantize_amax_reduce_amd as fq
import oracle
from dequantize_amax_reduce_amd import workloads as W
from gpu_util import G, assert_f32_equal, assert_fp8_equal, assert_hp_equal, dev, host

pytestmark = pytest.mark.gpu


def test_two_streams_interleaved():
    xa, _, _ = W.tensor_rows_scaled(rows=512, cols=2048, seed=91)
    xb, _, _ = W.tensor_rows_scaled(rows=384, cols=2048, seed=92)
    ga, _ = W.activation_outlier_channels(rows=256, cols=7168, seed=93)
    want = {}
    for name, x in (("a", xa), ("b", xb)):
        q, s = oracle.cast_per_tensor(x, "f32", "e4m3fn")
        want[name] = (q, s, oracle.dequant_per_tensor(q, "e4m3fn", s, "bf16"))
    wg_q, wg_s = oracle.cast_per_group128(ga, "bf16", "e5m2")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    bufs = []
    for x in (xa, xb):
        n = x.size
        bufs.append(dict(x=dev(x), q=G.empty(n, dtype=torch.uint8, device="cuda:0"),
                         s=G.empty(1, dtype=torch.float32, device="cuda:0"),
                         y=G.empty(n, dtype=torch.bfloat16, device="cuda:0"),
                         ws=G.empty(fq.fp8q_per_tensor_workspace_bytes() // 4, dtype=torch.int32,
                                        device="cuda:0"),
                         g=dev(ga, "bf16"), gq=G.empty(ga.shape, dtype=torch.uint8, device="cuda:0"),
                         gs=G.empty((ga.shape[0], ga.shape[1] // 128), dtype=torch.float32, device="cuda:0")))
    torch.cuda.synchronize()
    print("[case] two streams, 6 interleaved rounds", flush=True)
    for _ in range(6):
        for st, b in zip(streams, bufs):
            fq.fp8q_cast_per_tensor(b["x"], b["q"], b["s"], b["ws"], "e4m3fn", stream=st)
            fq.fp8q_cast_per_group128(b["g"], b["gq"], b["gs"], "e5m2", stream=st)
            fq.fp8q_dequant_per_tensor(b["q"], b["s"], b["y"], "e4m3fn", stream=st)
    torch.cuda.synchronize()
    for name, b in zip(("a", "b"), bufs):
        q, s, y = want[name]
        assert_fp8_equal(host(b["q"]), q, "e4m3fn", f"stream {name} q")
        assert_f32_equal(host(b["s"]), s, f"stream {name} scale_inv")
        assert_hp_equal(host(b["y"]), y, "bf16", f"stream {name} y")
        assert_fp8_equal(host(b["gq"]), wg_q, "e5m2", f"stream {name} group q")
        assert_f32_equal(host(b["gs"]), wg_s, f"stream {name} group scale_inv")


def test_host_threads_concurrent():
    """Four host threads call the entry points at the same time, each on its
    own stream with its own buffers and workspace (ctypes releases the GIL
    around every call), eight rounds each: the per-tensor cast, the
    per-channel cast, and the per-tensor dequant back to fp32."""
    from concurrent.futures import ThreadPoolExecutor
    T, rounds = 4, 8
    xs = [W.tensor_rows_scaled(rows=256, cols=1024, seed=100 + t)[0] for t in range(T)]
    want = []
    for x in xs:
        q, s = oracle.cast_per_tensor(x, "f32", "e5m2")
        qc, sc = oracle.cast_per_channel(x, "f32", "e5m2")
        want.append((q, s, oracle.dequant_per_tensor(q, "e5m2", s, "f32"), qc, sc))
    bufs = []
    for x in xs:
        n = x.size
        bufs.append(dict(st=torch.cuda.Stream(), x=dev(x), q=G.empty(n, dtype=torch.uint8, device="cuda:0"),
                         s=G.empty(1, dtype=torch.float32, device="cuda:0"),
                         y=G.empty(n, dtype=torch.float32, device="cuda:0"),
                         qc=G.empty(x.shape, dtype=torch.uint8, device="cuda:0"),
                         sc=G.empty(x.shape[0], dtype=torch.float32, device="cuda:0"),
                         ws=G.empty(fq.fp8q_per_tensor_workspace_bytes() // 4, dtype=torch.int32,
                                        device="cuda:0")))
    torch.cuda.synchronize()

    def work(b):
        for _ in range(rounds):
            fq.fp8q_cast_per_tensor(b["x"], b["q"], b["s"], b["ws"], "e5m2", stream=b["st"])
            fq.fp8q_cast_per_channel(b["x"], b["qc"], b["sc"], "e5m2", stream=b["st"])
            fq.fp8q_dequant_per_tensor(b["q"], b["s"], b["y"], "e5m2", stream=b["st"])
        b["st"].synchronize()

    print(f"[case] {T} host threads x {rounds} rounds, one stream each", flush=True)
    with ThreadPoolExecutor(T) as pool:
        list(pool.map(work, bufs))
    torch.cuda.synchronize()
    for t, (b, (q, s, y, qc, sc)) in enumerate(zip(bufs, want)):
        assert_fp8_equal(host(b["q"]), q, "e5m2", f"thread {t} q")
        assert_f32_equal(host(b["s"]), s, f"thread {t} scale_inv")
        assert_f32_equal(host(b["y"]), y, f"thread {t} y")
        assert_fp8_equal(host(b["qc"]), qc, "e5m2", f"thread {t} per-channel q")
        assert_f32_equal(host(b["sc"]), sc, f"thread {t} per-channel scale_inv")
