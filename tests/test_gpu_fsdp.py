"""GPU parity: the FSDP parameter hook's single-GPU parts (guarded local amax,
cast with the all-reduced amax, dequant by division by the scale) against the
CPU oracle, bit-exact.  The cross-rank MAX all-reduce is simulated on one GPU
by a max over the shards' guarded amax values."""
import numpy as np
import pytest
import torch

import dequantize_amax_reduce_amd as fq
import oracle
from dequantize_amax_reduce_amd import workloads as W
from gpu_util import G, assert_f32_equal, assert_fp8_equal, assert_hp_equal, dev, empty_hp, host

pytestmark = pytest.mark.gpu


def _shards(dtype, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for k, n in enumerate((1000, 4097, 64, 300)):
        x = (rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 2)).astype(np.float32)
        if k == 2:
            x[:] = 0.0                               # a rank whose shard is all zeros contributes 1
        out.append(W.to_bf16_bits(x) if dtype == "bf16" else
                   (x.astype(np.float16).view(np.uint16) if dtype == "f16" else x))
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("fmt", ["e5m2", "e4m3fn"])
def test_fsdp_hook_parts(fmt, dtype):
    shards = _shards(dtype, seed=len(dtype) * 3 + len(fmt))
    locs = []
    for sh in shards:
        a = G.empty(1, dtype=torch.float32, device="cuda:0")
        print(f"[case] amax_guarded {dtype} n={sh.size}", flush=True)
        fq.fp8q_amax_guarded(dev(sh, dtype), a)
        locs.append(a)
    torch.cuda.synchronize()
    for sh, a in zip(shards, locs):
        assert host(a)[0].view(np.uint32) == np.float32(oracle.amax_guarded(sh, dtype)).view(np.uint32)
    gmax = torch.stack(locs).max().reshape(1)            # stands in for all_reduce(MAX)
    g = np.float32(max(oracle.amax_guarded(sh, dtype) for sh in shards))
    assert host(gmax)[0] == g
    for sh in shards:
        q = G.empty(sh.size, dtype=torch.uint8, device="cuda:0")
        sc = G.empty(1, dtype=torch.float32, device="cuda:0")
        print(f"[case] cast_with_amax {fmt} {dtype} n={sh.size}", flush=True)
        fq.fp8q_cast_with_amax(dev(sh, dtype), gmax, q, sc, fmt)
        torch.cuda.synchronize()
        wq, wsc = oracle.cast_with_amax(sh, dtype, fmt, g)
        assert_fp8_equal(host(q), wq, fmt, "cast_with_amax q")
        assert_f32_equal(host(sc), wsc, "cast_with_amax scale")
        for ydt in ("bf16", "f32", "f16"):
            y = empty_hp(sh.size, ydt)
            fq.fp8q_dequant_div_scale(q, sc, y, fmt)
            torch.cuda.synchronize()
            assert_hp_equal(host(y), oracle.dequant_div_scale(wq, fmt, wsc[0], ydt), ydt, f"div dequant {ydt}")


@pytest.mark.parametrize("dtype,n", [("bf16", 9_000_005), ("f32", 12_000_003), ("f16", 30_000_001)])
def test_fsdp_hook_fat_chunks(dtype, n):
    """Shard sizes whose one-pass cast and division dequant take 4 or 8
    sub-steps per chunk, with ragged tails."""
    rng = np.random.Generator(np.random.PCG64(n))
    x = (rng.standard_normal(n) * 7.0).astype(np.float32)
    xh = W.to_bf16_bits(x) if dtype == "bf16" else (x.astype(np.float16).view(np.uint16) if dtype == "f16" else x)
    a = G.empty(1, dtype=torch.float32, device="cuda:0")
    fq.fp8q_amax_guarded(dev(xh, dtype), a)
    torch.cuda.synchronize()
    g = np.float32(oracle.amax_guarded(xh, dtype))
    assert host(a)[0] == g
    q = G.empty(n, dtype=torch.uint8, device="cuda:0")
    sc = G.empty(1, dtype=torch.float32, device="cuda:0")
    print(f"[case] cast_with_amax fat chunks {dtype} n={n}", flush=True)
    fq.fp8q_cast_with_amax(dev(xh, dtype), a, q, sc, "e5m2")
    torch.cuda.synchronize()
    wq, wsc = oracle.cast_with_amax(xh, dtype, "e5m2", g)
    assert_fp8_equal(host(q), wq, "e5m2", "fat cast_with_amax q")
    assert_f32_equal(host(sc), wsc, "fat cast_with_amax scale")
    y = empty_hp(n, "bf16")
    fq.fp8q_dequant_div_scale(q, sc, y, "e5m2")
    torch.cuda.synchronize()
    assert_hp_equal(host(y), oracle.dequant_div_scale(wq, "e5m2", wsc[0], "bf16"), "bf16", "fat div dequant")


def test_cast_with_too_small_amax_saturates():
    """An amax below the shard's own max: products leave the fp8 range and
    saturate (the hardware convert alone would give NaN/inf)."""
    rng = np.random.Generator(np.random.PCG64(3))
    x = (rng.standard_normal(5000) * 100).astype(np.float32)
    for fmt in ("e4m3fn", "e5m2"):
        for a in (np.float32(1.0), np.float32(0.0), np.float32(1e-38)):
            q = G.empty(x.size, dtype=torch.uint8, device="cuda:0")
            sc = G.empty(1, dtype=torch.float32, device="cuda:0")
            fq.fp8q_cast_with_amax(dev(x), dev(np.array([a], np.float32)), q, sc, fmt)
            torch.cuda.synchronize()
            wq, wsc = oracle.cast_with_amax(x, "f32", fmt, a)
            assert_fp8_equal(host(q), wq, fmt, f"saturating cast amax={a}")
            assert_f32_equal(host(sc), wsc)


def test_guarded_amax_special():
    z = G.zeros(100, dtype=torch.bfloat16, device="cuda:0")
    a = G.empty(1, dtype=torch.float32, device="cuda:0")
    fq.fp8q_amax_guarded(z, a)
    torch.cuda.synchronize()
    assert host(a)[0] == 1.0
    x = G.ones(100, dtype=torch.float32, device="cuda:0")
    x[7] = float("nan")
    fq.fp8q_amax_guarded(x, a)
    torch.cuda.synchronize()
    assert host(a)[0] == 1.0                          # torch.where(NaN > 0, NaN, 1) = 1
    fq.fp8q_amax_guarded(G.empty(0, dtype=torch.float32, device="cuda:0"), a)
    torch.cuda.synchronize()
    assert host(a)[0] == 1.0


def test_fsdp_full_size_shard():
    """One 2^28-element bf16 shard (the gradient-like payload) cast with its own
    guarded amax to e5m2 and dequantized by division back to bf16."""
    x = W.gradient_payload()
    xd = dev(x, "bf16")
    a = G.empty(1, dtype=torch.float32, device="cuda:0")
    q = G.empty(x.size, dtype=torch.uint8, device="cuda:0")
    sc = G.empty(1, dtype=torch.float32, device="cuda:0")
    y = G.empty(x.size, dtype=torch.bfloat16, device="cuda:0")
    print("[case] fsdp full-size shard", flush=True)
    fq.fp8q_amax_guarded(xd, a)
    fq.fp8q_cast_with_amax(xd, a, q, sc, "e5m2")
    fq.fp8q_dequant_div_scale(q, sc, y, "e5m2")
    torch.cuda.synchronize()
    del xd
    g = oracle.amax_guarded(x, "bf16")
    wq, wsc = oracle.cast_with_amax(x, "bf16", "e5m2", g)
    assert_fp8_equal(host(q), wq, "e5m2", "full-size shard q")
    assert_f32_equal(host(sc), wsc)
    assert_hp_equal(host(y), oracle.dequant_div_scale(wq, "e5m2", wsc[0], "bf16"), "bf16", "full-size div dequant")
