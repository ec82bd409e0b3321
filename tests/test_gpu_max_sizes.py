"""GPU: the largest shapes, past every 32-bit boundary, checked against the
CPU oracle on sampled elements (each sampled element's result depends only on
its own group, tile or the tensor's amax, so the oracle computes it from the
sampled inputs alone).  Inputs are generated on the device with seeded torch
generators; only the samples travel to the host.

- per-128-group cast and dequant of bf16 [300000, 7168] (2.15e9 elements, > 2^31),
  then the cast again from views two elements into the same buffers
- per-tensor cast and dequant of 2^32 + 37 bf16 elements with the maximum
  planted beyond 2^32, then again from views part-way into their buffers
- 128x128 block dequant of e4m3fn [4793491, 7168] (>= 2^32 lane vectors: the
  row-strip kernel), 34 GB of codes and 69 GB of bf16 output
"""
import numpy as np
import pytest
import torch

import dequantize_amax_reduce_amd as fq
import oracle
from gpu_util import G, assert_f32_equal, assert_fp8_equal, assert_hp_equal, host

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def _bits(t):
    return host(t)


def _need(gib):
    free, _ = torch.cuda.mem_get_info()
    if free < gib * (1 << 30):
        pytest.skip(f"needs {gib} GiB of free device memory, {free >> 30} GiB free")


def _free(*ts):
    del ts
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_group128_beyond_2_31_elements():
    R, C = 300_000, 7168
    _need(24)
    print(f"[case] group128 [{R}, {C}] ({R * C} elements)", flush=True)
    x = torch.randn((R, C), generator=_gen(81), device=DEV, dtype=torch.float32).to(torch.bfloat16)
    q = G.empty((R, C), dtype=torch.uint8, device=DEV)
    s = G.empty((R, C // 128), dtype=torch.float32, device=DEV)
    y = G.empty((R, C), dtype=torch.bfloat16, device=DEV)
    fq.fp8q_cast_per_group128(x, q, s, "e4m3fn")
    fq.fp8q_dequant_per_group128(q, s, y)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(82))
    rows = np.unique(np.concatenate([[0, 1, R - 2, R - 1], rng.integers(0, R, 60),
                                     rng.integers((1 << 31) // C, R, 8)]))
    ri = torch.from_numpy(rows).to(DEV)
    xs, qs, ss, ys = _bits(x[ri]), _bits(q[ri]), _bits(s[ri]), _bits(y[ri])
    wq, ws = oracle.cast_per_group128(xs, "bf16", "e4m3fn")
    assert_fp8_equal(qs, wq, "e4m3fn", "sampled rows q")
    assert_f32_equal(ss, ws, "sampled rows scale_inv")
    assert_hp_equal(ys, oracle.dequant_per_group128(wq, "e4m3fn", ws, "bf16"), "bf16", "sampled rows y")
    # again from views two elements into the same buffers (one row fewer): the
    # shifted kernel, whose vector and byte offsets pass 2^32 here
    del y
    R1 = R - 1
    print(f"[case] group128 shifted [{R1}, {C}], x and q two elements in", flush=True)
    xv = x.view(-1)[2:2 + R1 * C].view(R1, C)
    qv = q.view(-1)[2:2 + R1 * C].view(R1, C)
    sv = s.view(-1)[:R1 * (C // 128)].view(R1, C // 128)
    fq.fp8q_cast_per_group128(xv, qv, sv, "e4m3fn")
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, R1 - 2, R1 - 1], rng.integers(0, R1, 60),
                                     rng.integers((1 << 31) // C, R1, 8)]))
    ri = torch.from_numpy(rows).to(DEV)
    xs, qs, ss = _bits(xv[ri]), _bits(qv[ri]), _bits(sv[ri])
    wq, ws = oracle.cast_per_group128(xs, "bf16", "e4m3fn")
    assert_fp8_equal(qs, wq, "e4m3fn", "shifted sampled rows q")
    assert_f32_equal(ss, ws, "shifted sampled rows scale_inv")
    _free(x, q, s, xv, qv, sv)


def test_per_tensor_beyond_2_32_elements():
    n = (1 << 32) + 37
    peak = (1 << 32) + 5
    _need(40)
    print(f"[case] per-tensor bf16 n={n}, maximum at {peak}", flush=True)
    x = torch.randn(n, generator=_gen(83), device=DEV, dtype=torch.bfloat16)
    x[peak] = -300.0                      # |x| of N(0, 1) stays far below 300 over 2^32 draws
    q = G.empty(n, dtype=torch.uint8, device=DEV)
    si = G.empty(1, dtype=torch.float32, device=DEV)
    ws = G.empty(fq.fp8q_per_tensor_workspace_bytes() // 4, dtype=torch.int32, device=DEV)
    amax = G.empty(1, dtype=torch.float32, device=DEV)
    fq.fp8q_amax(x, amax)
    fq.fp8q_cast_per_tensor(x, q, si, ws, "e5m2")
    torch.cuda.synchronize()
    assert float(host(amax)[0]) == 300.0
    rng = np.random.Generator(np.random.PCG64(84))
    idx = np.unique(np.concatenate([[0, 1, peak, n - 37, n - 5, n - 1], rng.integers(0, n, 4000),
                                    rng.integers(1 << 32, n, 30)]))
    ti = torch.from_numpy(idx).to(DEV)
    xs, qs = _bits(x[ti]), _bits(q[ti])
    assert int(qs[np.nonzero(idx == peak)[0][0]]) == 0xFB          # -57344, the e5m2 maximum
    # the oracle sees the sampled values, whose maximum is the planted one
    wq, wsi = oracle.cast_per_tensor(xs, "bf16", "e5m2")
    assert_f32_equal(host(si), wsi, "scale_inv")
    assert_fp8_equal(qs, wq, "e5m2", "sampled q")
    # again from a view two elements into x, into codes one byte into their
    # buffer: the shifted amax pass and cast pass, past 2^32 elements
    nv = n - 2
    xv = x[2:]
    q2 = G.empty(n, dtype=torch.uint8, device=DEV)
    qv = q2[1:1 + nv]
    si2 = G.empty(1, dtype=torch.float32, device=DEV)
    amax2 = G.empty(1, dtype=torch.float32, device=DEV)
    print(f"[case] per-tensor bf16 shifted n={nv}", flush=True)
    fq.fp8q_amax(xv, amax2)
    fq.fp8q_cast_per_tensor(xv, qv, si2, ws, "e5m2")
    torch.cuda.synchronize()
    assert float(host(amax2)[0]) == 300.0
    idv = np.unique(np.concatenate([[0, 1, peak - 2, nv - 37, nv - 5, nv - 1], rng.integers(0, nv, 4000),
                                    rng.integers((1 << 32) - 2, nv, 30)]))
    tv = torch.from_numpy(idv).to(DEV)
    wqv, wsiv = oracle.cast_per_tensor(_bits(xv[tv]), "bf16", "e5m2")
    assert_f32_equal(host(si2), wsiv, "shifted scale_inv")
    assert_fp8_equal(_bits(qv[tv]), wqv, "e5m2", "shifted sampled q")
    del x, xv
    torch.cuda.empty_cache()
    y = G.empty(n, dtype=torch.bfloat16, device=DEV)
    fq.fp8q_dequant_per_tensor(q, si, y, "e5m2")
    torch.cuda.synchronize()
    assert_hp_equal(_bits(y[ti]), oracle.dequant_per_tensor(wq, "e5m2", wsi, "bf16"), "bf16", "sampled y")
    # the shifted dequant: those codes into an output one element into its buffer
    yv = y[1:1 + nv]
    fq.fp8q_dequant_per_tensor(qv, si2, yv, "e5m2")
    torch.cuda.synchronize()
    assert_hp_equal(_bits(yv[tv]), oracle.dequant_per_tensor(wqv, "e5m2", wsiv, "bf16"), "bf16", "shifted sampled y")
    _free(q, q2, y, ws, amax, amax2, si, si2)


def test_block_dequant_row_strip_path():
    M, N = 4_793_491, 7168                 # M * N / 8 >= 2^32 lane vectors; M % 128 = 19
    assert M * N // 8 >= 1 << 32
    _need(120)
    print(f"[case] block dequant [{M}, {N}] ({M * N} codes)", flush=True)
    c = torch.randint(0, 254, (M, N), generator=_gen(85), device=DEV, dtype=torch.uint8)
    for r0 in range(0, M, 1 << 18):        # no NaN code (0x7F, 0xFF); bounded temporaries
        blk = c[r0:r0 + (1 << 18)]
        blk += (blk >= 0x7F).to(torch.uint8)
    torch.cuda.empty_cache()
    mb, nb = (M + 127) // 128, (N + 127) // 128
    rng = np.random.Generator(np.random.PCG64(86))
    sh = (10.0 ** rng.uniform(-4.0, -1.0, size=(mb, nb))).astype(np.float32)
    s = torch.from_numpy(sh).to(DEV)
    y = G.empty((M, N), dtype=torch.bfloat16, device=DEV)
    fq.fp8q_weight_dequant_block128(c, s, y, "e4m3fn")
    torch.cuda.synchronize()
    ii = np.concatenate([[0, 0, M - 1, M - 1, M - 19, 127, 128], rng.integers(0, M, 3000)])
    jj = np.concatenate([[0, N - 1, 0, N - 1, 4095, 127, 128], rng.integers(0, N, 3000)])
    flat = torch.from_numpy(ii * N + jj).to(DEV)
    cs = _bits(c.reshape(-1)[flat])
    ys = _bits(y.reshape(-1)[flat])
    want = oracle.dequant_per_channel(cs.reshape(-1, 1), "e4m3fn", sh[ii // 128, jj // 128], "bf16").reshape(-1)
    assert_hp_equal(ys, want, "bf16", "sampled block dequant")
    _free(c, s, y)


@pytest.mark.parametrize("ydt", ["bf16", "f32"])
def test_block_dequant_single_row_beyond_2_32_columns(ydt):
    """One row of 2^32 + 1024 codes: few enough lane vectors for the flat
    kernel, but the column of an element past 2^32 no longer fits 32 bits,
    so its 128-column block must be found without forming col * VE.  The
    scale index is pid_m * ceil(N/128) + pid_n (CSDN notes, weight_dequant_kernel)."""
    M, N = 1, (1 << 32) + 1024
    esz = 2 if ydt == "bf16" else 4
    _need(4 + 4 * esz + 2)
    print(f"[case] block dequant [{M}, {N}] -> {ydt}", flush=True)
    c = torch.randint(0, 254, (M, N), generator=_gen(87), device=DEV, dtype=torch.uint8)
    flat = c.view(-1)
    for i0 in range(0, N, 1 << 30):        # no NaN code (0x7F, 0xFF); bounded temporaries
        blk = flat[i0:i0 + (1 << 30)]
        blk += (blk >= 0x7F).to(torch.uint8)
    torch.cuda.empty_cache()
    nb = (N + 127) // 128
    rng = np.random.Generator(np.random.PCG64(88))
    sh = (10.0 ** rng.uniform(-4.0, -1.0, size=(1, nb))).astype(np.float32)
    s = torch.from_numpy(sh).to(DEV)
    y = G.empty((M, N), dtype=torch.bfloat16 if ydt == "bf16" else torch.float32, device=DEV)
    fq.fp8q_weight_dequant_block128(c, s, y, "e4m3fn")
    torch.cuda.synchronize()
    jj = np.unique(np.concatenate([np.arange(0, 300), np.arange((1 << 32) - 300, (1 << 32) + 300),
                                   np.arange(N - 300, N), rng.integers(0, N, 4000),
                                   rng.integers(1 << 32, N, 500)]))
    ti = torch.from_numpy(jj).to(DEV)
    cs = _bits(flat[ti])
    ys = _bits(y.view(-1)[ti])
    want = oracle.dequant_per_channel(cs.reshape(-1, 1), "e4m3fn", sh[0, jj // 128], ydt).reshape(-1)
    assert_hp_equal(ys, want, ydt, "sampled single-row block dequant")
    _free(c, s, y)
