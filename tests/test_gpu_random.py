"""GPU parity on seeded random cases for every entry point: random shapes
(ragged tails, odd row lengths, empty), element types, formats, magnitudes
(10^-6 .. 10^6 with zero blocks) and buffer offsets (which switch between
the vector kernels, the shifted ones and the element-wise ones), each
bit-exact against the CPU oracle (NaN by class)."""
import numpy as np
import pytest
import torch

import dequantize_amax_reduce_amd as fq
import oracle
from gpu_util import G, TORCH_HP, assert_f32_equal, assert_fp8_equal, assert_hp_equal, dev, host

pytestmark = pytest.mark.gpu
DTYPES = ("f32", "bf16", "f16")
FMTS = ("e4m3fn", "e5m2")
NCASE = 100


def _values(rng, shape, dtype):
    n = int(np.prod(shape))
    x = (rng.standard_normal(n) * 10.0 ** rng.uniform(-6, 6)).astype(np.float32)
    if n and rng.random() < 0.3:
        k = int(rng.integers(0, n))
        x[k:k + int(rng.integers(1, 300))] = 0.0
    if dtype == "bf16":
        from dequantize_amax_reduce_amd import workloads as W
        return W.to_bf16_bits(x).reshape(shape)
    if dtype == "f16":
        return np.clip(x, -6e4, 6e4).astype(np.float16).view(np.uint16).reshape(shape)
    return x.reshape(shape)


def _placed(h, dtype, off):
    """device copy of host array h (dtype 'f32'/'bf16'/'f16'/'u8') starting `off` elements into a buffer"""
    flat = np.concatenate([np.zeros(off, h.dtype), h.reshape(-1)])
    t = dev(flat, None if dtype in ("f32", "u8") else dtype)[off:]
    return t.view(h.shape)


def _empty(shape, tdtype, off):
    n = int(np.prod(shape))
    return G.empty(n + off, dtype=tdtype, device="cuda:0")[off:].view(shape)


def _case(rng):
    return (DTYPES[int(rng.integers(0, 3))], FMTS[int(rng.integers(0, 2))], DTYPES[int(rng.integers(0, 3))],
            int(rng.choice([0, 0, 1, 3, 8])), int(rng.choice([0, 0, 1, 4])))


def test_random_group128():
    rng = np.random.Generator(np.random.PCG64(9001))
    for i in range(NCASE):
        dtype, fmt, ydt, xo, qo = _case(rng)
        rows, cols = int(rng.integers(0, 70)), 128 * int(rng.integers(1, 40))
        x = _values(rng, (rows, cols), dtype)
        print(f"[case] group128 #{i} {rows}x{cols} {dtype}->{fmt}->{ydt} x_off={xo} q_off={qo}", flush=True)
        q = _empty((rows, cols), torch.uint8, qo)
        s = G.empty((rows, cols // 128), dtype=torch.float32, device="cuda:0")
        fq.fp8q_cast_per_group128(_placed(x, dtype, xo), q, s, fmt)
        y = _empty((rows, cols), TORCH_HP[ydt], xo)
        fq.fp8q_dequant_per_group128(q, s, y, fmt)
        torch.cuda.synchronize()
        wq, ws = oracle.cast_per_group128(x, dtype, fmt)
        assert_fp8_equal(host(q), wq, fmt, f"#{i} q")
        assert_f32_equal(host(s), ws, f"#{i} scale_inv")
        assert_hp_equal(host(y), oracle.dequant_per_group128(wq, fmt, ws, ydt), ydt, f"#{i} y")


def test_random_tensor_and_channel():
    rng = np.random.Generator(np.random.PCG64(9002))
    for i in range(NCASE):
        dtype, fmt, ydt, xo, qo = _case(rng)
        n = int(rng.integers(0, 300_000))
        x = _values(rng, (n,), dtype)
        print(f"[case] per-tensor #{i} n={n} {dtype}->{fmt}->{ydt} x_off={xo} q_off={qo}", flush=True)
        q = _empty((n,), torch.uint8, qo)
        s = G.empty(1, dtype=torch.float32, device="cuda:0")
        ws = G.empty(fq.fp8q_per_tensor_workspace_bytes() // 4, dtype=torch.int32, device="cuda:0")
        fq.fp8q_cast_per_tensor(_placed(x, dtype, xo), q, s, ws, fmt)
        y = _empty((n,), TORCH_HP[ydt], xo)
        fq.fp8q_dequant_per_tensor(q, s, y, fmt)
        torch.cuda.synchronize()
        wq, wsi = oracle.cast_per_tensor(x, dtype, fmt)
        assert_fp8_equal(host(q), wq, fmt, f"#{i} tensor q")
        assert_f32_equal(host(s), wsi, f"#{i} tensor scale_inv")
        assert_hp_equal(host(y), oracle.dequant_per_tensor(wq, fmt, wsi, ydt), ydt, f"#{i} tensor y")

        rows, cols = int(rng.integers(0, 40)), int(rng.integers(0, 20_000))
        x = _values(rng, (rows, cols), dtype)
        print(f"[case] per-channel #{i} {rows}x{cols} {dtype}->{fmt}->{ydt} x_off={xo} q_off={qo}", flush=True)
        q = _empty((rows, cols), torch.uint8, qo)
        s = G.empty(rows, dtype=torch.float32, device="cuda:0")
        fq.fp8q_cast_per_channel(_placed(x, dtype, xo), q, s, fmt)
        y = _empty((rows, cols), TORCH_HP[ydt], xo)
        fq.fp8q_dequant_per_channel(q, s, y, fmt)
        torch.cuda.synchronize()
        wq, wsi = oracle.cast_per_channel(x, dtype, fmt)
        assert_fp8_equal(host(q), wq, fmt, f"#{i} channel q")
        assert_f32_equal(host(s), wsi, f"#{i} channel scale_inv")
        if cols:
            assert_hp_equal(host(y), oracle.dequant_per_channel(wq, fmt, wsi, ydt), ydt, f"#{i} channel y")


def test_random_block_dequant():
    rng = np.random.Generator(np.random.PCG64(9003))
    for i in range(NCASE):
        _, fmt, ydt, qo, yo = _case(rng)
        M, N = int(rng.integers(1, 700)), int(rng.integers(1, 700))
        c = rng.integers(0, 256, size=(M, N)).astype(np.uint8)
        s = (10.0 ** rng.uniform(-6, 3, size=((M + 127) // 128, (N + 127) // 128))).astype(np.float32)
        print(f"[case] block #{i} {M}x{N} {fmt}->{ydt} q_off={qo} y_off={yo}", flush=True)
        y = _empty((M, N), TORCH_HP[ydt], yo)
        fq.fp8q_weight_dequant_block128(_placed(c, "u8", qo), dev(s), y, fmt)
        torch.cuda.synchronize()
        assert_hp_equal(host(y), oracle.weight_dequant_block128(c, fmt, s, ydt), ydt, f"#{i} block y")


def test_random_reduce_step():
    rng = np.random.Generator(np.random.PCG64(9004))
    for i in range(NCASE):
        _, fmt, ydt, qo, _ = _case(rng)
        Wn, n = int(rng.integers(1, 10)), int(rng.integers(0, 50_000))
        c = rng.integers(0, 256, size=(Wn, n)).astype(np.uint8)
        s = (10.0 ** rng.uniform(-6, 0, size=Wn)).astype(np.float32)
        avg, requant = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
        print(f"[case] reduce #{i} W={Wn} n={n} {fmt}->{ydt} avg={avg} requant={requant} q_off={qo}", flush=True)
        qd = _placed(c, "u8", qo)
        y = G.empty(n, dtype=TORCH_HP[ydt], device="cuda:0")
        if requant:
            qo_t = G.empty(n, dtype=torch.uint8, device="cuda:0")
            so = G.empty(1, dtype=torch.float32, device="cuda:0")
            ws = G.empty(fq.fp8q_per_tensor_workspace_bytes() // 4, dtype=torch.int32, device="cuda:0")
            fq.fp8q_dequant_sum_requant(qd, dev(s), y, qo_t, so, ws, fmt, avg)
        else:
            fq.fp8q_dequant_sum(qd, dev(s), y, fmt, avg)
        torch.cuda.synchronize()
        if requant:
            wy, wq, wso = oracle.dequant_sum_requant(c, fmt, s, ydt, avg)
            assert_hp_equal(host(y), wy, ydt, f"#{i} sum")
            assert_fp8_equal(host(qo_t), wq, fmt, f"#{i} requant q")
            assert_f32_equal(host(so), wso, f"#{i} requant scale_inv")
        else:
            assert_hp_equal(host(y), oracle.dequant_sum(c, fmt, s, ydt, avg), ydt, f"#{i} sum")


def test_random_packed_pipeline_fsdp():
    rng = np.random.Generator(np.random.PCG64(9005))
    for i in range(NCASE):
        dtype, fmt, ydt, xo, _ = _case(rng)
        Wn = int(rng.integers(1, 6))
        n = int(rng.integers(0, 20_000))
        n = n - n % 4 if Wn > 1 else n
        xs = [_values(rng, (n,), dtype) for _ in range(Wn)]
        print(f"[case] packed #{i} W={Wn} n={n} {dtype}->{fmt}->{ydt}", flush=True)
        comb = G.empty(Wn * (4 + n), dtype=torch.uint8, device="cuda:0")
        ws = G.empty(fq.fp8q_per_tensor_workspace_bytes() // 4, dtype=torch.int32, device="cuda:0")
        for r, x in enumerate(xs):
            fq.fp8q_cast_to_packed(_placed(x, dtype, xo), comb[r * (4 + n):(r + 1) * (4 + n)], ws, fmt)
        y = G.empty((Wn, n), dtype=TORCH_HP[ydt], device="cuda:0")
        fq.fp8q_dequant_packed(comb, Wn, n, y, fmt)
        torch.cuda.synchronize()
        want = np.concatenate([oracle.cast_to_packed(x, dtype, fmt) for x in xs])
        got = host(comb)
        assert np.array_equal(got, want) or _same_but_nan(got, want, fmt, Wn, n), f"#{i} packed bytes"
        assert_hp_equal(host(y), oracle.dequant_packed(want, fmt, Wn, n, ydt), ydt, f"#{i} packed y")

        x = xs[0]
        print(f"[case] pipeline/fsdp #{i} n={n} {dtype}->{ydt} x_off={xo}", flush=True)
        q = G.empty(n, dtype=torch.uint8, device="cuda:0")
        si = G.empty(1, dtype=torch.float32, device="cuda:0")
        word = G.empty(1, dtype=torch.int32, device="cuda:0")
        xd = _placed(x, dtype, xo)
        fq.fp8q_cast_to_fp8_pipeline(xd, q, si, word, ws)
        yp = G.empty(n, dtype=TORCH_HP[ydt], device="cuda:0")
        fq.fp8q_cast_from_fp8_pipeline(q, word, si, yp)
        torch.cuda.synchronize()
        wq, wsi, wf = oracle.cast_to_fp8_pipeline(x, dtype)
        assert {0: "e4m3fn", 1: "e5m2"}[int(host(word)[0])] == wf
        assert_fp8_equal(host(q), wq, wf, f"#{i} pipeline q")
        assert_f32_equal(host(si), wsi, f"#{i} pipeline scale_inv")
        assert_hp_equal(host(yp), oracle.cast_from_fp8_pipeline(wq, wf, wsi[0], ydt), ydt, f"#{i} pipeline y")

        a = np.float32(10.0 ** rng.uniform(-8, 8)) if rng.random() < 0.8 else np.float32(0.0)
        qf = G.empty(n, dtype=torch.uint8, device="cuda:0")
        sc = G.empty(1, dtype=torch.float32, device="cuda:0")
        fq.fp8q_cast_with_amax(xd, dev(np.array([a], np.float32)), qf, sc, fmt)
        yf = G.empty(n, dtype=TORCH_HP[ydt], device="cuda:0")
        fq.fp8q_dequant_div_scale(qf, sc, yf, fmt)
        torch.cuda.synchronize()
        wq, wsc = oracle.cast_with_amax(x, dtype, fmt, a)
        assert_fp8_equal(host(qf), wq, fmt, f"#{i} fsdp q")
        assert_f32_equal(host(sc), wsc, f"#{i} fsdp scale")
        assert_hp_equal(host(yf), oracle.dequant_div_scale(wq, fmt, wsc[0], ydt), ydt, f"#{i} fsdp y")


def _same_but_nan(got, want, fmt, Wn, n):
    """packed bytes equal except NaN codes, which are compared by class"""
    from gpu_util import FP8_NAN_CLASS
    for r in range(Wn):
        a, b = got[r * (4 + n):(r + 1) * (4 + n)], want[r * (4 + n):(r + 1) * (4 + n)]
        if not np.array_equal(a[:4], b[:4]):
            return False
        nan = FP8_NAN_CLASS[fmt](a[4:]) & FP8_NAN_CLASS[fmt](b[4:])
        if np.any((a[4:] != b[4:]) & ~nan):
            return False
    return True
