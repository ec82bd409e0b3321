"""GPU parity: global amax, per-tensor and per-channel cast, their dequants,
through the C ABI, against the CPU oracle, bit-exact (NaN by class).

Workloads: rows scaled by 10**U(-3, 3) with 1 % zero rows (fp32 and bf16
roundings of the same values, both fp8 formats, plus empty tensors), and the
gradient-like 1-D payload bf16 [2^28] ~ N(0, 1e-3^2) with e5m2 per-tensor
amax -> cast -> dequant to fp32 at full size."""
import numpy as np
import pytest
import torch

import dequantize_amax_reduce_amd as fq
import oracle
from dequantize_amax_reduce_amd import workloads as W
from gpu_util import G, assert_f32_equal, assert_fp8_equal, assert_hp_equal, dev, empty_hp, host

pytestmark = pytest.mark.gpu
FMTS = ("e4m3fn", "e5m2")
FP8_MAX = {"e4m3fn": 448.0, "e5m2": 57344.0}


def _tensor_cast(xh, dtype, fmt, x_offset=0):
    n = xh.size
    flat = dev(np.concatenate([np.zeros(x_offset, xh.dtype), xh.reshape(-1)]), dtype)
    x = flat[x_offset:]
    q = G.empty(n, dtype=torch.uint8, device="cuda:0")
    s = G.empty(1, dtype=torch.float32, device="cuda:0")
    ws = G.empty(fq.fp8q_per_tensor_workspace_bytes() // 4, dtype=torch.int32, device="cuda:0")
    print(f"[case] per-tensor cast {dtype} {fmt} n={n} x_off={x_offset}", flush=True)
    fq.fp8q_cast_per_tensor(x, q, s, ws, fmt)
    torch.cuda.synchronize()
    return host(q).reshape(xh.shape), host(s)


def _channel_cast(xh, dtype, fmt):
    rows, cols = xh.shape
    q = G.empty((rows, cols), dtype=torch.uint8, device="cuda:0")
    s = G.empty(rows, dtype=torch.float32, device="cuda:0")
    print(f"[case] per-channel cast {dtype} {fmt} {rows}x{cols}", flush=True)
    fq.fp8q_cast_per_channel(dev(xh, dtype), q, s, fmt)
    torch.cuda.synchronize()
    return host(q), host(s)


def _check_tensor(xh, dtype, fmt, **kw):
    q, s = _tensor_cast(xh, dtype, fmt, **kw)
    wq, ws = oracle.cast_per_tensor(xh, dtype, fmt)
    assert_fp8_equal(q, wq, fmt, f"per-tensor q {dtype} {fmt}")
    assert_f32_equal(s, ws, f"per-tensor scale_inv {dtype} {fmt}")
    return q, s


def _check_channel(xh, dtype, fmt):
    q, s = _channel_cast(xh, dtype, fmt)
    wq, ws = oracle.cast_per_channel(xh, dtype, fmt)
    assert_fp8_equal(q, wq, fmt, f"per-channel q {dtype} {fmt}")
    assert_f32_equal(s, ws, f"per-channel scale_inv {dtype} {fmt}")
    return q, s


def _dequant(q, s, fmt, ydtype, per_channel):
    y = empty_hp(q.shape, ydtype)
    print(f"[case] dequant per_channel={per_channel} {fmt}->{ydtype} {q.shape}", flush=True)
    if per_channel:
        fq.fp8q_dequant_per_channel(dev(q), dev(s), y, fmt)
    else:
        fq.fp8q_dequant_per_tensor(dev(q), dev(s), y, fmt)
    torch.cuda.synchronize()
    return host(y)


def _rows_scaled(rows, cols, seed):
    xf, xb, _ = W.tensor_rows_scaled(rows=rows, cols=cols, seed=seed)
    return {"f32": xf, "bf16": xb}


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tensor_channel_config_full_size(dtype, fmt):
    """[4096, 4096] per-tensor and per-channel casts and their dequants back
    to the input type."""
    x = _rows_scaled(4096, 4096, seed=2)[dtype]
    q, s = _check_tensor(x, dtype, fmt)
    assert_hp_equal(_dequant(q, s, fmt, dtype, False), oracle.dequant_per_tensor(q, fmt, s, dtype), dtype,
                    "per-tensor round trip")
    q, s = _check_channel(x, dtype, fmt)
    assert_hp_equal(_dequant(q, s, fmt, dtype, True), oracle.dequant_per_channel(q, fmt, s, dtype), dtype,
                    "per-channel round trip")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 15), (7, 16), (33, 4096), (5, 4112), (4, 8192),
                                       (3, 16384), (2, 16400), (2, 40000), (2, 40001), (37, 65536)])
def test_channel_shapes(rows, cols, fmt, dtype):
    x = _rows_scaled(rows, cols, seed=rows + cols)["f32"]
    if dtype == "bf16":
        x = W.to_bf16_bits(x)
    elif dtype == "f16":
        x = np.clip(x, -6e4, 6e4).astype(np.float16).view(np.uint16)
    _check_channel(x, dtype, fmt)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("n", [1, 15, 16, 17, 1000, 65536 + 7, 3 * 2 ** 20 + 5])
def test_tensor_sizes(n, dtype):
    rng = np.random.Generator(np.random.PCG64(n))
    x = (rng.standard_normal(n, dtype=np.float32) * np.float32(3.0))
    if dtype == "bf16":
        x = W.to_bf16_bits(x)
    elif dtype == "f16":
        x = x.astype(np.float16).view(np.uint16)
    for fmt in FMTS:
        _check_tensor(x, dtype, fmt)
    _check_tensor(x, dtype, "e4m3fn", x_offset=1)           # unaligned x -> element-wise kernel


@pytest.mark.parametrize("dtype,n", [("bf16", 9_000_003), ("f32", 13_000_001), ("bf16", 30_000_007),
                                     ("f16", 20_000_001)])
def test_tensor_sizes_fat_chunks(dtype, n):
    """Sizes whose flat kernels take K = 4 or 8 sub-steps per chunk (the
    launch picks them when the K = 2 grid would span two to four dispatch
    rounds), with ragged tails: cast, then dequant to bf16 and fp32."""
    rng = np.random.Generator(np.random.PCG64(n))
    x = rng.standard_normal(n, dtype=np.float32) * np.float32(5.0)
    if dtype == "bf16":
        x = W.to_bf16_bits(x)
    elif dtype == "f16":
        x = x.astype(np.float16).view(np.uint16)
    for fmt in FMTS:
        q, s = _check_tensor(x, dtype, fmt)
        for ydt in ("bf16", "f32"):
            assert_hp_equal(_dequant(q, s, fmt, ydt, False), oracle.dequant_per_tensor(q, fmt, s, ydt), ydt,
                            f"per-tensor dequant n={n} {fmt}->{ydt}")


@pytest.mark.parametrize("rows,cols", [(3001, 4000), (2049, 7000), (1, 8_400_000), (4097, 2048), (7, 4096)])
def test_channel_fat_chunks_and_row_pairs(rows, cols):
    """Per-channel cast with two rows per workgroup trip (16-bit rows of up to
    4096 elements, odd row counts leave a half trip) and the flat per-channel
    dequant at sizes where it takes K = 4 or 8, with row lengths that are not
    powers of two (the lane's row comes from an invariant-divisor division)."""
    xf = _rows_scaled(rows, cols, seed=rows * 3 + cols)["f32"]
    for dtype in ("bf16", "f16", "f32"):
        x = {"f32": xf, "bf16": W.to_bf16_bits(xf),
             "f16": np.clip(xf, -6e4, 6e4).astype(np.float16).view(np.uint16)}[dtype]
        q, s = _check_channel(x, dtype, "e4m3fn")
    for ydt in ("bf16", "f32"):
        assert_hp_equal(_dequant(q, s, "e4m3fn", ydt, True), oracle.dequant_per_channel(q, "e4m3fn", s, ydt), ydt,
                        f"per-channel dequant [{rows}, {cols}] -> {ydt}")


def _every_amax_values(dtype, fmt):
    """The amax bit patterns of test_gpu_group128.test_group_cast_every_amax:
    every positive finite bf16 / fp16 value, or 2^18 binary32 values over every
    exponent (half of them just below a power of two times fp8_max)."""
    if dtype == "bf16":
        return np.arange(1, 0x7F80, dtype=np.uint16)
    if dtype == "f16":
        return np.arange(1, 0x7C00, dtype=np.uint16)
    rng = np.random.Generator(np.random.PCG64(43))
    spread = rng.integers(1, 0x7F800000, size=1 << 17, dtype=np.uint32)
    k = rng.integers(-120, 100, size=1 << 17)
    near = (np.ldexp(np.float64(FP8_MAX[fmt]), k).astype(np.float32).view(np.uint32) -
            rng.integers(0, 3, size=1 << 17).astype(np.uint32))
    return np.concatenate([spread, near]).astype(np.uint32)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("fmt", FMTS)
def test_channel_and_tensor_cast_every_amax(dtype, fmt):
    """The per-channel and per-tensor casts skip the clamp whenever amax > 0 and
    the scale is finite, so they rely, like the group cast, on amax *
    RN(fp8_max / amax) encoding to the maximum code when that product is one
    binary32 ulp above fp8_max.  Per-channel: one row per amax value (the value,
    its negation, the value below it, 125 smaller ones).  Per-tensor: 64 of
    those rows, one call each, chosen where the product rounds above fp8_max."""
    from test_gpu_group128 import _every_amax_groups
    amax = _every_amax_values(dtype, fmt)
    x = _every_amax_groups(amax, dtype, seed=44)
    q, s = _check_channel(x, dtype, fmt)
    code_max = 0x7E if fmt == "e4m3fn" else 0x7B
    assert np.all(q[:, 0] == code_max) and np.all(q[:, 1] == (code_max | 0x80))
    # rows whose product amax * fl32(fp8_max / amax) exceeds fp8_max in exact arithmetic
    if dtype == "f32":
        a = amax.view(np.float32)
    elif dtype == "bf16":
        a = (amax.astype(np.uint32) << 16).view(np.float32)
    else:
        a = amax.view(np.float16).astype(np.float32)
    with np.errstate(over="ignore", divide="ignore"):
        scale = (np.float32(FP8_MAX[fmt]) / a).astype(np.float32)
    over = np.nonzero(np.isfinite(scale) & (a.astype(np.float64) * scale.astype(np.float64) > FP8_MAX[fmt]))[0]
    assert over.size > 0
    rng = np.random.Generator(np.random.PCG64(45))
    for r in rng.choice(over, size=min(64, over.size), replace=False):
        qt, _ = _check_tensor(x[r:r + 1], dtype, fmt)
        assert qt.reshape(-1)[0] == code_max and qt.reshape(-1)[1] == (code_max | 0x80)


def test_amax_entry_point():
    for dtype, n in [("bf16", 1 << 20), ("f32", 12345), ("f16", 77)]:
        rng = np.random.Generator(np.random.PCG64(n))
        x = rng.standard_normal(n, dtype=np.float32)
        xh = W.to_bf16_bits(x) if dtype == "bf16" else (x.astype(np.float16).view(np.uint16) if dtype == "f16" else x)
        a = G.full((1,), -1.0, dtype=torch.float32, device="cuda:0")
        fq.fp8q_amax(dev(xh, dtype), a)
        torch.cuda.synchronize()
        assert host(a)[0].view(np.uint32) == np.float32(oracle.amax(xh, dtype)).view(np.uint32)
    x = np.ones(1000, np.float32)
    x[500] = np.nan
    a = G.zeros(1, dtype=torch.float32, device="cuda:0")
    fq.fp8q_amax(dev(x), a)
    torch.cuda.synchronize()
    assert np.isnan(host(a)[0])
    fq.fp8q_amax(G.empty(0, dtype=torch.float32, device="cuda:0"), a)
    torch.cuda.synchronize()
    assert host(a)[0] == 0.0


def test_edge_tensors():
    """all-zero, negative zeros, NaN, +-inf, tiny amax (scale = +inf: saturating
    path), denormal-only and huge values, per tensor and per channel."""
    f = np.float32
    cases = {
        "zeros": np.zeros(64, f),
        "neg_zeros": -np.zeros(64, f),
        "nan": np.array([1.0, np.nan, -2.0] + [0.5] * 61, f),
        "inf": np.array([1.0, np.inf, -2.0] + [0.5] * 61, f),
        "tiny_amax": np.array([1e-38, -5e-39, 1e-45, 0.0] * 16, f),      # 448/1e-38 overflows -> inf scale
        "denormal": np.array([1e-41, -3e-42] * 32, f),
        "huge": np.array([3e38, -1e38] * 32, f),
        "one_at_max": np.array([448.0, -448.0, 1.0, 2.0 ** -9] * 16, f),
    }
    for name, x in cases.items():
        for fmt in FMTS:
            _check_tensor(x, "f32", fmt)
            _check_tensor(W.to_bf16_bits(x), "bf16", fmt)
            _check_channel(x.reshape(4, 16), "f32", fmt)
            _check_channel(W.to_bf16_bits(x).reshape(4, 16), "bf16", fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_hardware_convert_through_abi(fmt):
    """With amax == fp8_max the per-tensor scale is exactly 1, so q = fp8(x):
    a structured sweep of every binary32 exponent field and the top mantissa
    bits (with several sticky patterns), both signs, within +-fp8_max."""
    import exact
    v = exact.structured_f32_sweep()
    v = v[np.isfinite(v) & (np.abs(v) <= FP8_MAX[fmt])]
    v = np.concatenate([[np.float32(FP8_MAX[fmt])], v, exact.fp8_midpoints(fmt)]).astype(np.float32)
    q, s = _check_tensor(v, "f32", fmt)
    assert s[0] == 1.0


@pytest.mark.parametrize("ydtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("fmt", FMTS)
def test_dequant_all_codes(fmt, ydtype):
    codes = np.tile(np.arange(256, dtype=np.uint8), 37)
    for sv in (1.0, 2.0 ** -140, 1.7e38, 0.1234567, 3.0e-8):
        s = np.array([sv], np.float32)
        assert_hp_equal(_dequant(codes, s, fmt, ydtype, False), oracle.dequant_per_tensor(codes, fmt, s, ydtype),
                        ydtype, f"per-tensor dequant s={sv}")
    q2 = codes.reshape(37, 256)
    s2 = (10.0 ** np.linspace(-30, 30, 37)).astype(np.float32)
    assert_hp_equal(_dequant(q2, s2, fmt, ydtype, True), oracle.dequant_per_channel(q2, fmt, s2, ydtype), ydtype,
                    "per-channel dequant")


def test_gradient_payload_full_size():
    """bf16 [2^28] ~ N(0, 1e-3^2): global amax -> e5m2 cast -> dequant to fp32."""
    x = W.gradient_payload()
    xd = dev(x, "bf16")
    a = G.zeros(1, dtype=torch.float32, device="cuda:0")
    print("[case] gradient payload amax", flush=True)
    fq.fp8q_amax(xd, a)
    q = G.empty(x.size, dtype=torch.uint8, device="cuda:0")
    s = G.empty(1, dtype=torch.float32, device="cuda:0")
    ws = G.empty(fq.fp8q_per_tensor_workspace_bytes() // 4, dtype=torch.int32, device="cuda:0")
    print("[case] gradient payload cast", flush=True)
    fq.fp8q_cast_per_tensor(xd, q, s, ws, "e5m2")
    y = G.empty(x.size, dtype=torch.float32, device="cuda:0")
    print("[case] gradient payload dequant", flush=True)
    fq.fp8q_dequant_per_tensor(q, s, y, "e5m2")
    torch.cuda.synchronize()
    del xd
    wa = oracle.amax(x, "bf16")
    assert host(a)[0].view(np.uint32) == np.float32(wa).view(np.uint32)
    wq, ws_ = oracle.cast_per_tensor(x, "bf16", "e5m2")
    qh = host(q)
    assert_fp8_equal(qh, wq, "e5m2", "gradient payload q")
    assert_f32_equal(host(s), ws_, "gradient payload scale_inv")
    del q
    assert_f32_equal(host(y), oracle.dequant_per_tensor(wq, "e5m2", ws_, "f32"), "gradient payload dequant")


def test_empty_tensors():
    for fmt in FMTS:
        x = G.empty(0, dtype=torch.float32, device="cuda:0")
        q = G.empty(0, dtype=torch.uint8, device="cuda:0")
        s = G.full((1,), -7.0, dtype=torch.float32, device="cuda:0")
        ws = G.empty(fq.fp8q_per_tensor_workspace_bytes() // 4, dtype=torch.int32, device="cuda:0")
        fq.fp8q_cast_per_tensor(x, q, s, ws, fmt)
        torch.cuda.synchronize()
        assert host(s)[0] == 1.0                           # cast_to_fp8's empty branch
        x2 = G.empty((4096, 0), dtype=torch.bfloat16, device="cuda:0")
        q2 = G.empty((4096, 0), dtype=torch.uint8, device="cuda:0")
        s2 = G.full((4096,), -7.0, dtype=torch.float32, device="cuda:0")
        fq.fp8q_cast_per_channel(x2, q2, s2, fmt)
        torch.cuda.synchronize()
        assert np.all(host(s2) == 1.0)
        x3 = G.empty((0, 4096), dtype=torch.bfloat16, device="cuda:0")
        fq.fp8q_cast_per_channel(x3, G.empty((0, 4096), dtype=torch.uint8, device="cuda:0"),
                                 G.empty(0, dtype=torch.float32, device="cuda:0"), fmt)
        torch.cuda.synchronize()
