"""GPU parity: the pipeline p2p cast with the fp8 format chosen on the device
(fp8q_cast_to_fp8_pipeline) and its dequant (fp8q_cast_from_fp8_pipeline),
bit-exact against the CPU oracle: the format word, the codes, scale_inv and
the dequantized values, on both sides of the 448 threshold and on the
degenerate amax values."""
import numpy as np
import pytest
import torch

import dequantize_amax_reduce_amd as fq
import oracle
from dequantize_amax_reduce_amd import workloads as W
from gpu_util import G, assert_f32_equal, assert_fp8_equal, assert_hp_equal, dev, empty_hp, host

pytestmark = pytest.mark.gpu
FMT_WORD = {0: "e4m3fn", 1: "e5m2"}


def _ws():
    return G.empty(fq.fp8q_per_tensor_workspace_bytes() // 4, dtype=torch.int32, device="cuda:0")


def _to_dtype(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return W.to_bf16_bits(x32)
    if dtype == "f16":
        return x32.astype(np.float16).view(np.uint16)
    return x32.astype(np.float32)


def _check_pipeline(xh: np.ndarray, dtype: str, what: str, offset: int = 0, ydtypes=("bf16", "f32", "f16")):
    """Run the device pipeline cast (x placed `offset` elements into its
    buffer, to reach the element-wise path) and the dequant to each ydtype."""
    n = xh.size
    print(f"[case] pipeline {what} {dtype} n={n} offset={offset}", flush=True)
    buf = dev(np.concatenate([np.zeros(offset, xh.dtype), xh.reshape(-1)]), dtype)
    x = buf[offset:]
    qbuf = G.empty(n + offset, dtype=torch.uint8, device="cuda:0")
    q = qbuf[offset:]
    si = G.empty(1, dtype=torch.float32, device="cuda:0")
    word = G.full((1,), -5, dtype=torch.int32, device="cuda:0")
    fq.fp8q_cast_to_fp8_pipeline(x, q, si, word, _ws())
    torch.cuda.synchronize()
    wq, wsi, wfmt = oracle.cast_to_fp8_pipeline(xh.reshape(-1), dtype)
    assert FMT_WORD[int(host(word)[0])] == wfmt, (what, dtype)
    assert_fp8_equal(host(q), wq, wfmt, f"{what} q")
    assert_f32_equal(host(si), wsi, f"{what} scale_inv")
    for ydt in ydtypes:
        ybuf = empty_hp(n + offset, ydt)
        y = ybuf[offset:]
        fq.fp8q_cast_from_fp8_pipeline(q, word, si, y)
        torch.cuda.synchronize()
        assert_hp_equal(host(y), oracle.cast_from_fp8_pipeline(wq, wfmt, wsi[0], ydt), ydt, f"{what} -> {ydt}")
    return wfmt


@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
def test_pipeline_sizes_and_formats(dtype):
    rng = np.random.Generator(np.random.PCG64(61))
    seen = set()
    for n in (1, 7, 255, 4097, 3 * 2048 * 8 + 5, 200_003):
        for e in (-3.0, 0.0, 2.0, 2.9, 4.0):
            x = (rng.standard_normal(n) * 10.0 ** e).astype(np.float32)
            seen.add(_check_pipeline(_to_dtype(x, dtype), dtype, f"N(0,1e{e:g})", ydtypes=("bf16", "f32")))
    assert seen == {"e4m3fn", "e5m2"}


@pytest.mark.parametrize("dtype,n", [("bf16", 9_000_007), ("f32", 12_000_001), ("f16", 30_000_003)])
def test_pipeline_fat_chunks(dtype, n):
    """Sizes whose amax and cast passes both take 4 or 8 sub-steps per chunk,
    with ragged tails."""
    rng = np.random.Generator(np.random.PCG64(n))
    for e in (0.0, 3.0):
        x = (rng.standard_normal(n) * 10.0 ** e).astype(np.float32)
        _check_pipeline(_to_dtype(x, dtype), dtype, f"fat chunks N(0,1e{e:g})", ydtypes=("bf16",))


@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
def test_pipeline_unaligned(dtype):
    rng = np.random.Generator(np.random.PCG64(62))
    for off in (1, 3):
        for e in (0.0, 3.0):
            x = (rng.standard_normal(5000) * 10.0 ** e).astype(np.float32)
            _check_pipeline(_to_dtype(x, dtype), dtype, "unaligned", offset=off)


@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
def test_pipeline_degenerate(dtype):
    """amax exactly 448, just above it, zero, NaN, +-inf, and (fp32 only) an amax
    so small that the scale overflows to inf."""
    above = {"f32": np.nextafter(np.float32(448), np.float32(np.inf)), "bf16": np.float32(450.0),
             "f16": np.float32(448.25)}[dtype]
    rng = np.random.Generator(np.random.PCG64(63))
    base = (rng.standard_normal(3000) * 50).astype(np.float32)
    base = np.clip(base, -440, 440)
    cases = {}
    x = base.copy(); x[17] = -448.0; cases["amax448"] = x
    x = base.copy(); x[2999] = above; cases["above448"] = x
    cases["zeros"] = np.zeros(3000, np.float32)
    x = base.copy(); x[5] = np.nan; cases["nan"] = x
    x = base.copy(); x[1234] = -np.inf; cases["inf"] = x
    if dtype == "f32":
        cases["tiny"] = np.array([1e-40, 0.0, -1e-40, 3e-41] * 700, np.float32)
    for name, x in cases.items():
        fmt = _check_pipeline(_to_dtype(x, dtype), dtype, name)
        assert fmt == ("e5m2" if name in ("above448", "inf") else "e4m3fn"), (name, fmt)


def test_pipeline_empty():
    x = G.empty(0, dtype=torch.bfloat16, device="cuda:0")
    q = G.empty(0, dtype=torch.uint8, device="cuda:0")
    si = G.full((1,), 7.0, dtype=torch.float32, device="cuda:0")
    word = G.full((1,), 9, dtype=torch.int32, device="cuda:0")
    fq.fp8q_cast_to_fp8_pipeline(x, q, si, word, _ws())
    torch.cuda.synchronize()
    assert host(si)[0] == 1.0 and int(host(word)[0]) == 0


def test_pipeline_bad_format_word_gives_nan():
    rng = np.random.Generator(np.random.PCG64(64))
    q = dev(W.fp8_codes_finite(10_000, "e4m3fn", seed=65))
    si = dev(np.array([0.5], np.float32))
    for bad in (2, -1, 0x7FFFFFFF):
        word = G.full((1,), bad, dtype=torch.int32, device="cuda:0")
        for ydt in ("bf16", "f32", "f16"):
            y = empty_hp(q.numel(), ydt)
            fq.fp8q_cast_from_fp8_pipeline(q, word, si, y)
            torch.cuda.synchronize()
            assert torch.isnan(y.float()).all(), (bad, ydt)
    del rng


def test_pipeline_dict_helpers():
    """The page-level helpers: the dict round trip through the device word."""
    xh, _ = W.activation_outlier_channels(rows=64, cols=7168, seed=66)
    x = dev(xh, "bf16")
    inp = {"hidden_states": x}
    fq.cast_to_fp8_pipeline(inp)
    assert inp["hidden_states"].dtype == torch.uint8 and inp["dtype"] == torch.bfloat16
    fq.cast_from_fp8_pipeline(inp)
    torch.cuda.synchronize()
    wq, wsi, wfmt = oracle.cast_to_fp8_pipeline(xh, "bf16")
    assert_hp_equal(host(inp["hidden_states"]), oracle.cast_from_fp8_pipeline(wq, wfmt, wsi[0], "bf16"), "bf16")
    assert set(inp) == {"hidden_states"}
    assert fq.cast_to_fp8_pipeline(None) is None
    t = torch.ones(1)
    fq.cast_to_fp8_pipeline(t)
    assert t.item() == 1.0


def test_pipeline_full_size_activation():
    """The activation workload, bf16 [16384, 7168] (outlier channels x50, so
    e4m3fn), and the row-scaled fp32 [4096, 4096] tensor (amax ~1e3, so e5m2)."""
    xh, _ = W.activation_outlier_channels()
    assert _check_pipeline(xh, "bf16", "activation 16384x7168", ydtypes=("bf16",)) == "e4m3fn"
    del xh
    x32, _, _ = W.tensor_rows_scaled()
    assert _check_pipeline(x32, "f32", "rows-scaled 4096x4096", ydtypes=("f32",)) == "e5m2"
