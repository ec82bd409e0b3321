"""GPU parity of the shifted stream: every entry point that streams a flat
tensor, on views that start part-way into a lane vector -- every offset of
the high-precision side from a 16-byte boundary (in elements) against every
offset of the fp8 side from an 8-byte boundary -- on element counts that end
mid-vector and span several chunks, bit-exact against the CPU oracle.  Two
larger counts per element type take the 4- and 8-sub-step chunks."""
import numpy as np
import pytest
import torch

import dequantize_amax_reduce_amd as fq
import oracle
from dequantize_amax_reduce_amd import workloads as W
from gpu_util import G, TORCH_HP, assert_f32_equal, assert_fp8_equal, assert_hp_equal, dev, host

pytestmark = pytest.mark.gpu
DTYPES = ("bf16", "f32", "f16")
FMTS = ("e4m3fn", "e5m2")
ESZ = {"f32": 4, "bf16": 2, "f16": 2}


def _values(n, dtype, seed, decades=3):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = (rng.standard_normal(n) * 10.0 ** rng.uniform(-decades, decades, size=n)).astype(np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return W.to_bf16_bits(x)
    return np.clip(x, -6e4, 6e4).astype(np.float16).view(np.uint16)


def _placed(h, dtype, off):
    """device copy of host array h starting `off` elements into a guarded buffer"""
    flat = np.concatenate([np.zeros(off, h.dtype), h.reshape(-1)])
    return dev(flat, None if dtype in ("f32", "u8") else dtype)[off:].view(h.shape)


def _empty(shape, tdtype, off):
    n = int(np.prod(shape))
    return G.empty(n + off, dtype=tdtype, device="cuda:0")[off:].view(shape)


def _offsets(dtype):
    return [(xo, qo) for xo in range(16 // ESZ[dtype]) for qo in range(8)]


WS = None


def _ws():
    global WS
    if WS is None:
        WS = G.empty(fq.fp8q_per_tensor_workspace_bytes() // 4, dtype=torch.int32, device="cuda:0")
    return WS


@pytest.mark.parametrize("dtype", DTYPES)
def test_tensor_cast_and_dequant_every_offset(dtype):
    """Per-tensor cast (both passes) and its dequant; the dequant's output
    offset runs through every value too, independently of the input's."""
    for n, seed in ((37, 1), (3 * 4096 + 1234, 2)):
        x = _values(n, dtype, seed)
        ref = {f: oracle.cast_per_tensor(x, dtype, f) for f in FMTS}
        for i, (xo, qo) in enumerate(_offsets(dtype)):
            fmt = FMTS[i % 2]
            yo = (xo + 3 * qo) % (16 // ESZ[dtype])
            print(f"[case] per-tensor {dtype} {fmt} n={n} x+{xo} q+{qo} y+{yo}", flush=True)
            q = _empty((n,), torch.uint8, qo)
            s = G.empty(1, dtype=torch.float32, device="cuda:0")
            fq.fp8q_cast_per_tensor(_placed(x, dtype, xo), q, s, _ws(), fmt)
            y = _empty((n,), TORCH_HP[dtype], yo)
            fq.fp8q_dequant_per_tensor(q, s, y, fmt)
            torch.cuda.synchronize()
            wq, wsi = ref[fmt]
            assert_fp8_equal(host(q), wq, fmt, f"q {dtype} n={n} x+{xo} q+{qo}")
            assert_f32_equal(host(s), wsi, f"scale_inv {dtype} n={n} x+{xo} q+{qo}")
            assert_hp_equal(host(y), oracle.dequant_per_tensor(wq, fmt, wsi, dtype), dtype,
                            f"y {dtype} n={n} q+{qo} y+{yo}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_amax_every_offset(dtype):
    for n, seed in ((5, 3), (2 * 4096 + 777, 4)):
        x = _values(n, dtype, seed)
        x[n // 2] = {"f32": np.float32(-12345.0), "bf16": 0xC640, "f16": 0xF000}[dtype]   # -12288 / -8192 planted
        want = oracle.amax(x, dtype)
        want_g = oracle.amax_guarded(x, dtype)
        for xo in range(16 // ESZ[dtype]):
            print(f"[case] amax {dtype} n={n} x+{xo}", flush=True)
            a = G.empty(1, dtype=torch.float32, device="cuda:0")
            ag = G.empty(1, dtype=torch.float32, device="cuda:0")
            xd = _placed(x, dtype, xo)
            fq.fp8q_amax(xd, a)
            fq.fp8q_amax_guarded(xd, ag)
            torch.cuda.synchronize()
            assert_f32_equal(host(a), np.array([want], np.float32), f"amax {dtype} n={n} x+{xo}")
            assert_f32_equal(host(ag), np.array([want_g], np.float32), f"guarded amax {dtype} n={n} x+{xo}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_fsdp_hook_every_offset(dtype):
    """Cast with a given amax (some values saturate) and the dequant by division."""
    n = 2 * 4096 + 999
    x = _values(n, dtype, 5)
    a = np.float32(oracle.amax(x, dtype) * np.float32(0.5))   # half the true amax: the top values saturate
    for i, (xo, qo) in enumerate(_offsets(dtype)):
        fmt = FMTS[i % 2]
        yo = (2 * xo + qo) % (16 // ESZ[dtype])
        print(f"[case] fsdp hook {dtype} {fmt} x+{xo} q+{qo} y+{yo}", flush=True)
        q = _empty((n,), torch.uint8, qo)
        sc = G.empty(1, dtype=torch.float32, device="cuda:0")
        fq.fp8q_cast_with_amax(_placed(x, dtype, xo), dev(np.array([a], np.float32)), q, sc, fmt)
        y = _empty((n,), TORCH_HP[dtype], yo)
        fq.fp8q_dequant_div_scale(q, sc, y, fmt)
        torch.cuda.synchronize()
        wq, wsc = oracle.cast_with_amax(x, dtype, fmt, a)
        assert_fp8_equal(host(q), wq, fmt, f"fsdp q {dtype} x+{xo} q+{qo}")
        assert_f32_equal(host(sc), wsc, f"fsdp scale {dtype} x+{xo} q+{qo}")
        assert_hp_equal(host(y), oracle.dequant_div_scale(wq, fmt, wsc[0], dtype), dtype, f"fsdp y {dtype} y+{yo}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_pipeline_every_offset(dtype):
    n = 4096 + 4095
    for big in (False, True):   # amax below / above 448: e4m3fn / e5m2 chosen on the device
        x = _values(n, dtype, 6 + big, decades=1)   # |x| < 448 unless planted
        if big and dtype != "f32":
            x[17] = 0x4480 if dtype == "bf16" else 0x6000   # 1024.0 in bf16 / 512.0 in fp16
        elif big:
            x[17] = np.float32(1000.0)
        wq, wsi, wf = oracle.cast_to_fp8_pipeline(x, dtype)
        for xo, qo in _offsets(dtype):
            yo = (xo + qo) % (16 // ESZ[dtype])
            print(f"[case] pipeline {dtype} big={big} x+{xo} q+{qo} y+{yo}", flush=True)
            q = _empty((n,), torch.uint8, qo)
            si = G.empty(1, dtype=torch.float32, device="cuda:0")
            word = G.empty(1, dtype=torch.int32, device="cuda:0")
            fq.fp8q_cast_to_fp8_pipeline(_placed(x, dtype, xo), q, si, word, _ws())
            y = _empty((n,), TORCH_HP[dtype], yo)
            fq.fp8q_cast_from_fp8_pipeline(q, word, si, y)
            torch.cuda.synchronize()
            assert {0: "e4m3fn", 1: "e5m2"}[int(host(word)[0])] == wf
            assert_fp8_equal(host(q), wq, wf, f"pipeline q {dtype} x+{xo} q+{qo}")
            assert_f32_equal(host(si), wsi, f"pipeline scale_inv {dtype}")
            assert_hp_equal(host(y), oracle.cast_from_fp8_pipeline(wq, wf, wsi[0], dtype), dtype,
                            f"pipeline y {dtype} q+{qo} y+{yo}")


@pytest.mark.parametrize("ydt", DTYPES)
def test_group_and_channel_dequant_every_offset(ydt):
    """Per-128-group dequant and the per-channel dequant (rows whose length is
    a multiple of the lane width, streamed flat) from every code offset into
    every output offset."""
    rng = np.random.Generator(np.random.PCG64(8))
    rows, cols = 33, 384
    c = rng.integers(0, 256, size=(rows, cols)).astype(np.uint8)
    sg = (10.0 ** rng.uniform(-4, 1, size=(rows, cols // 128))).astype(np.float32)
    rows2, cols2 = 17, 1000
    c2 = rng.integers(0, 256, size=(rows2, cols2)).astype(np.uint8)
    sr = (10.0 ** rng.uniform(-4, 1, size=rows2)).astype(np.float32)
    for i, (yo, qo) in enumerate(_offsets(ydt)):
        fmt = FMTS[i % 2]
        print(f"[case] group/channel dequant -> {ydt} {fmt} q+{qo} y+{yo}", flush=True)
        y = _empty((rows, cols), TORCH_HP[ydt], yo)
        fq.fp8q_dequant_per_group128(_placed(c, "u8", qo), dev(sg), y, fmt)
        y2 = _empty((rows2, cols2), TORCH_HP[ydt], yo)
        fq.fp8q_dequant_per_channel(_placed(c2, "u8", qo), dev(sr), y2, fmt)
        torch.cuda.synchronize()
        assert_hp_equal(host(y), oracle.dequant_per_group128(c, fmt, sg, ydt), ydt, f"group y q+{qo} y+{yo}")
        assert_hp_equal(host(y2), oracle.dequant_per_channel(c2, fmt, sr, ydt), ydt, f"channel y q+{qo} y+{yo}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_tensor_cast_and_dequant_fat_chunks_shifted(dtype):
    """Counts in the 4- and 8-sub-step windows, x two elements and q three
    bytes in, the dequant's output one element in."""
    sizes = (12_000_003, 20_000_001) if dtype == "bf16" else (6_000_001, 12_000_001)
    for n in sizes:
        x = _values(n, dtype, n % 97)
        print(f"[case] per-tensor shifted {dtype} n={n}", flush=True)
        q = _empty((n,), torch.uint8, 3)
        s = G.empty(1, dtype=torch.float32, device="cuda:0")
        fq.fp8q_cast_per_tensor(_placed(x, dtype, 2), q, s, _ws(), "e4m3fn")
        y = _empty((n,), TORCH_HP[dtype], 1)
        fq.fp8q_dequant_per_tensor(q, s, y, "e4m3fn")
        torch.cuda.synchronize()
        wq, wsi = oracle.cast_per_tensor(x, dtype, "e4m3fn")
        assert_fp8_equal(host(q), wq, "e4m3fn", f"q {dtype} n={n}")
        assert_f32_equal(host(s), wsi, f"scale_inv {dtype} n={n}")
        assert_hp_equal(host(y), oracle.dequant_per_tensor(wq, "e4m3fn", wsi, dtype), dtype, f"y {dtype} n={n}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_channel_cast_every_offset(dtype):
    """The per-channel cast of views: each row a shifted stream (rows of 1000,
    7168 and 16000 elements take chunks of 2, 4 and 8 sub-steps; 1004-element
    16-bit rows are not whole lane vectors and take the element-wise kernel)."""
    shapes = ((17, 1000, 21), (9, 7168, 22), (5, 16000, 23), (6, 1004, 24))
    for rows, cols, seed in shapes:
        x = _values(rows * cols, dtype, seed).reshape(rows, cols)
        ref = {f: oracle.cast_per_channel(x, dtype, f) for f in FMTS}
        offs = _offsets(dtype) if cols == 1000 else [(1, 3), (2, 6), (16 // ESZ[dtype] - 1, 7)]
        for i, (xo, qo) in enumerate(offs):
            fmt = FMTS[i % 2]
            print(f"[case] per-channel cast {dtype} {fmt} {rows}x{cols} x+{xo} q+{qo}", flush=True)
            q = _empty((rows, cols), torch.uint8, qo)
            s = G.empty(rows, dtype=torch.float32, device="cuda:0")
            fq.fp8q_cast_per_channel(_placed(x, dtype, xo), q, s, fmt)
            torch.cuda.synchronize()
            wq, ws = ref[fmt]
            assert_fp8_equal(host(q), wq, fmt, f"channel q {dtype} {rows}x{cols} x+{xo} q+{qo}")
            assert_f32_equal(host(s), ws, f"channel scale_inv {dtype} {rows}x{cols} x+{xo} q+{qo}")
