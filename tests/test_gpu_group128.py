"""GPU parity: per-128-group cast and its inverse, through the C ABI, against
the CPU oracle, bit-exact (NaN by class).

Workloads follow the seeded recipes in dequantize_amax_reduce_amd.workloads:
the small per-group cast (bf16 [128, 512], zero rows, +-200 outliers) and the
LLM activation quantize (bf16 [16384, 7168], 0.1 % of channels x50) at full
size, in the same launch configuration the benchmark times."""
import numpy as np
import pytest
import torch

import dequantize_amax_reduce_amd as fq
import oracle
from dequantize_amax_reduce_amd import workloads as W
from gpu_util import G, assert_f32_equal, assert_fp8_equal, assert_hp_equal, dev, empty_hp, host

pytestmark = pytest.mark.gpu
FMTS = ("e4m3fn", "e5m2")


def _gpu_group_cast(x_host, dtype, fmt, x_offset=0, q_offset=0, fn=None):
    """Run fp8q_cast_per_group128 (or `fn`, an entry point with the same
    arguments); offsets (in elements / bytes) make the device pointers
    misaligned to exercise the shifted kernel."""
    rows, cols = x_host.shape
    flat = dev(np.concatenate([np.zeros(x_offset, x_host.dtype), x_host.reshape(-1)]), dtype)
    x = flat[x_offset:].view(rows, cols)
    qbuf = G.empty(rows * cols + q_offset, dtype=torch.uint8, device="cuda:0")
    q = qbuf[q_offset:].view(rows, cols)
    s = G.empty((rows, cols // 128), dtype=torch.float32, device="cuda:0")
    fn = fn or fq.fp8q_cast_per_group128
    print(f"[case] {fn.__name__} {dtype} {fmt} {rows}x{cols} x_off={x_offset} q_off={q_offset}", flush=True)
    fn(x, q, s, fmt)
    torch.cuda.synchronize()
    return host(q), host(s)


def _check_cast(x_host, dtype, fmt, **kw):
    q, s = _gpu_group_cast(x_host, dtype, fmt, **kw)
    wq, ws = oracle.cast_per_group128(x_host, dtype, fmt)
    assert_fp8_equal(q, wq, fmt, f"q {dtype} {fmt}")
    assert_f32_equal(s, ws, f"scale_inv {dtype} {fmt}")
    return wq, ws


def _inputs(dtype, rows, cols, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    x *= (10.0 ** rng.uniform(-3, 3, size=(rows, cols // 128, 1))).astype(np.float32).repeat(128, axis=2) \
        .reshape(rows, cols)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return W.to_bf16_bits(x)
    return x.astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("fmt", FMTS)
def test_small_group_cast_config(fmt):
    x, zero_rows = W.group_cast_small()
    wq, ws = _check_cast(x, "bf16", fmt)
    # the three zeroed rows hit the 1e-4 clamp in every group
    assert np.all(ws[zero_rows] == ws[zero_rows[0], 0])


@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rows,cols", [(1, 128), (3, 256), (17, 640), (257, 1152), (1000, 7168)])
def test_group_cast_shapes(dtype, fmt, rows, cols):
    _check_cast(_inputs(dtype, rows, cols, seed=rows * 7 + cols), dtype, fmt)


# x not 16-byte aligned or q not 4-byte aligned: the shifted kernel (aligned
# 16-byte loads re-formed by a cross-lane shuffle and a byte shift, aligned
# stores of words that straddle two lanes' codes)
@pytest.mark.parametrize("x_offset,q_offset", [(1, 0), (0, 3), (3, 5), (2, 0), (2, 2), (4, 6), (2, 1)])
@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
def test_group_cast_unaligned(dtype, x_offset, q_offset):
    for fmt in FMTS:
        _check_cast(_inputs(dtype, 33, 384, seed=5), dtype, fmt, x_offset=x_offset, q_offset=q_offset)
        _check_cast(_inputs(dtype, 70, 1152, seed=6), dtype, fmt, x_offset=x_offset, q_offset=q_offset)


@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
def test_group_cast_every_misalignment(dtype):
    """Every offset of x from a 16-byte boundary (in elements) against every
    offset of q from an 8-byte boundary, on one group and on 99 groups (whole
    chunks, then a ragged one), the formats alternating: each combination
    but the aligned one takes the shifted kernel, whose first and last
    vectors straddle the ends of x and q."""
    esz = 4 if dtype == "f32" else 2
    for rows, cols, seed in ((1, 128, 12), (33, 384, 11)):
        x_host = _inputs(dtype, rows, cols, seed=seed)
        ref = {fmt: oracle.cast_per_group128(x_host, dtype, fmt) for fmt in FMTS}
        for xo in range(16 // esz):
            for qo in range(8):
                fmt = FMTS[(xo + qo) % 2]
                q, s = _gpu_group_cast(x_host, dtype, fmt, x_offset=xo, q_offset=qo)
                assert_fp8_equal(q, ref[fmt][0], fmt, f"q {dtype} {fmt} {rows}x{cols} x+{xo} q+{qo}")
                assert_f32_equal(s, ref[fmt][1], f"scale_inv {dtype} {fmt} {rows}x{cols} x+{xo} q+{qo}")


def test_group_cast_edge_values():
    """zeros of both signs, values just under/over the clamp, denormals, the
    bf16 extremes, inf and NaN groups, one group per row."""
    f = np.float32
    groups = [
        np.zeros(128, f),
        -np.zeros(128, f),
        np.full(128, 1e-4, f),
        np.full(128, 9.9e-5, f),
        np.linspace(-1e-38, 1e-38, 128).astype(f),                 # fp32 subnormal-range inputs
        np.linspace(-3.3e38, 3.3e38, 128).astype(f),
        np.concatenate([[np.inf], np.ones(127, f)]).astype(f),
        np.concatenate([[np.nan], np.ones(127, f)]).astype(f),
        np.concatenate([[-np.inf], -np.zeros(127, f)]).astype(f),
        (np.arange(128, dtype=f) - 64) * f(3.0),
        np.array([448.0 * (1 + 2 ** -23)] + [1.0] * 127, f),
    ]
    x = np.stack(groups)
    for fmt in FMTS:
        _check_cast(x, "f32", fmt)
        _check_cast(W.to_bf16_bits(x), "bf16", fmt)


def _every_amax_groups(amax_bits: np.ndarray, dtype: str, seed: int) -> np.ndarray:
    """One 128-group per amax value: the value itself, its negation, the
    largest value below it, and 125 values of smaller magnitude with random
    signs.  Every element's product with the group's scale is at most
    amax * (fp8_max / amax) rounded, the largest product the non-saturating
    kernels ever see."""
    rng = np.random.Generator(np.random.PCG64(seed))
    g = amax_bits.size
    if dtype == "f32":
        a = amax_bits.view(np.float32).astype(np.float64)
    elif dtype == "bf16":
        a = (amax_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:
        a = amax_bits.view(np.float16).astype(np.float64)
    mags = a[:, None] * rng.uniform(0.0, 1.0, size=(g, 125))
    vals = mags * np.where(rng.integers(0, 2, size=(g, 125)) == 1, 1.0, -1.0)
    f32 = vals.astype(np.float32)                       # |rounded| <= amax: rounding is monotone
    if dtype == "f32":
        body = f32.view(np.uint32)
        below = np.maximum(amax_bits.astype(np.int64) - 1, 0).astype(np.uint32)
        neg = amax_bits | np.uint32(0x80000000)
        out = np.concatenate([amax_bits[:, None], neg[:, None], below[:, None], body], axis=1)
        return out.view(np.float32)
    body = W.to_bf16_bits(f32) if dtype == "bf16" else f32.astype(np.float16).view(np.uint16)
    below = np.maximum(amax_bits.astype(np.int64) - 1, 0).astype(np.uint16)
    neg = amax_bits | np.uint16(0x8000)
    return np.concatenate([amax_bits[:, None], neg[:, None], below[:, None], body], axis=1)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("fmt", FMTS)
def test_group_cast_every_amax(dtype, fmt):
    """The non-saturating group kernels rely on amax * RN(fp8_max / amax)
    encoding to the format's maximum code even when that product is one
    binary32 ulp above fp8_max.  Every positive finite bf16 and fp16 value,
    and 2^18 binary32 values spread over every exponent (half of them the
    largest below a power of two times 448 or 57344), appears once as a
    group's amax; each group must match the oracle bit-exactly."""
    if dtype == "bf16":
        amax = np.arange(1, 0x7F80, dtype=np.uint16)                 # 0x0001 .. 0x7F7F
    elif dtype == "f16":
        amax = np.arange(1, 0x7C00, dtype=np.uint16)                 # 0x0001 .. 0x7BFF
    else:
        rng = np.random.Generator(np.random.PCG64(41))
        spread = rng.integers(1, 0x7F800000, size=1 << 17, dtype=np.uint32)
        fmax = 448.0 if fmt == "e4m3fn" else 57344.0
        k = rng.integers(-120, 100, size=1 << 17)
        near = (np.ldexp(np.float64(fmax), k).astype(np.float32).view(np.uint32) -
                rng.integers(0, 3, size=1 << 17).astype(np.uint32))
        amax = np.concatenate([spread, near]).astype(np.uint32)
    x = _every_amax_groups(amax, dtype, seed=42)
    wq, _ = _check_cast(x, dtype, fmt)
    code_max = 0x7E if fmt == "e4m3fn" else 0x7B
    clamp = np.float32(1e-4)
    if dtype == "f32":
        a = amax.view(np.float32)
    elif dtype == "bf16":
        a = (amax.astype(np.uint32) << 16).view(np.float32)
    else:
        a = amax.view(np.float16).astype(np.float32)
    big = a >= clamp                                  # unclamped groups: the amax element maps to +-max
    assert np.all(wq[big, 0] == code_max) and np.all(wq[big, 1] == (code_max | 0x80))


@pytest.mark.parametrize("ydtype", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("fmt", FMTS)
def test_group_dequant(fmt, ydtype):
    rows, cols = 67, 896
    rng = np.random.Generator(np.random.PCG64(9))
    q = W.fp8_codes_finite((rows, cols), fmt, seed=10)
    s = (10.0 ** rng.uniform(-8, 3, size=(rows, cols // 128))).astype(np.float32)
    y = empty_hp((rows, cols), ydtype)
    print(f"[case] group128 dequant {fmt} -> {ydtype}", flush=True)
    fq.fp8q_dequant_per_group128(dev(q), dev(s), y, fmt)
    torch.cuda.synchronize()
    assert_hp_equal(host(y), oracle.dequant_per_group128(q, fmt, s, ydtype), ydtype, f"dequant {fmt} {ydtype}")


def test_small_config_round_trip():
    """cast then dequant back to bf16 and fp32, both bit-exact with the oracle."""
    x, _ = W.group_cast_small()
    for fmt in FMTS:
        q, s = _gpu_group_cast(x, "bf16", fmt)
        for ydt in ("bf16", "f32"):
            y = empty_hp(x.shape, ydt)
            fq.fp8q_dequant_per_group128(dev(q), dev(s), y, fmt)
            torch.cuda.synchronize()
            assert_hp_equal(host(y), oracle.dequant_per_group128(q, fmt, s, ydt), ydt, f"round trip {fmt} {ydt}")


def test_activation_config_full_size():
    """bf16 [16384, 7168] -> e4m3fn + float32 [16384, 56], whole output
    compared with the oracle, then the per-group dequant back to bf16."""
    x, ch = W.activation_outlier_channels()
    q, s = _check_cast(x, "bf16", "e4m3fn")
    assert s.shape == (16384, 56)
    y = empty_hp(x.shape, "bf16")
    print("[case] activation config dequant", flush=True)
    fq.fp8q_dequant_per_group128(dev(q), dev(s), y, "e4m3fn")
    torch.cuda.synchronize()
    assert_hp_equal(host(y), oracle.dequant_per_group128(q, "e4m3fn", s, "bf16"), "bf16", "activation dequant")


def test_activation_config_full_size_shifted():
    """The same workload with x and q two elements into their buffers (the
    shifted kernel, as the benchmark times it), whole output against the
    oracle."""
    x, ch = W.activation_outlier_channels()
    _check_cast(x, "bf16", "e4m3fn", x_offset=2, q_offset=2)


@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("fmt", FMTS)
def test_group_cast_wave64_variant(dtype, fmt):
    """fp8q_cast_per_group128_wave64 (one wavefront per group, two elements
    per lane) against the oracle, from aligned buffers and from views two
    elements in, on one group and on ragged counts of its 8-group wave trips."""
    for rows, cols, seed in ((1, 128, 21), (33, 384, 22), (70, 1152, 23)):
        x_host = _inputs(dtype, rows, cols, seed=seed)
        wq, ws = oracle.cast_per_group128(x_host, dtype, fmt)
        for xo, qo in ((0, 0), (2, 2), (2, 6)):
            q, s = _gpu_group_cast(x_host, dtype, fmt, x_offset=xo, q_offset=qo, fn=fq.fp8q_cast_per_group128_wave64)
            assert_fp8_equal(q, wq, fmt, f"wave64 q {dtype} {fmt} {rows}x{cols} x+{xo} q+{qo}")
            assert_f32_equal(s, ws, f"wave64 scale_inv {dtype} {fmt} {rows}x{cols} x+{xo} q+{qo}")


def test_activation_config_full_size_wave64():
    """The activation workload through the one-wavefront-per-group variant,
    as the benchmark times it (aligned buffers), whole output against the
    oracle."""
    x, ch = W.activation_outlier_channels()
    q, s = _gpu_group_cast(x, "bf16", "e4m3fn", fn=fq.fp8q_cast_per_group128_wave64)
    wq, ws = oracle.cast_per_group128(x, "bf16", "e4m3fn")
    assert_fp8_equal(q, wq, "e4m3fn", "wave64 activation q")
    assert_f32_equal(s, ws, "wave64 activation scale_inv")


def test_group_cast_empty():
    for shape in [(0, 128), (5, 0), (0, 0)]:
        x = G.empty(shape, dtype=torch.bfloat16, device="cuda:0")
        q = G.empty(shape, dtype=torch.uint8, device="cuda:0")
        s = G.empty((shape[0], shape[1] // 128), dtype=torch.float32, device="cuda:0")
        fq.fp8q_cast_per_group128(x, q, s)
        torch.cuda.synchronize()
