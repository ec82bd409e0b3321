"""Pins of the CPU oracle against facts fixed outside it.

Each ``pin_*`` function takes an ``oracle.OracleLib`` and raises
AssertionError when the oracle disagrees with:

* closed forms of the OCP fp8 formats and the values the pages print
  (448 as the e4m3fn maximum on the "5 Utils" page);
* library conversions (torch's float8 / bfloat16 casts on the CPU, numpy's
  binary16 cast) and a vectorised nearest-value search;
* exact rational arithmetic on tiny inputs (``exact.py``);
* invariants of the method (the amax element maps to +-fp8_max, zero
  groups/rows give fixed constants, power-of-two scaling is exact).

``test_oracle_pins.py`` runs them on the real oracle and
``test_oracle_mutants.py`` runs them on deliberately broken copies of the
oracle source to show that each plausible mistake fails at least one pin.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import torch

import exact as X

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
FORMATS = ("e4m3fn", "e5m2")
TORCH_FP8 = {"e4m3fn": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def _bits32(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def _bf16_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _widen(x, dtype):
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return _bf16_to_f32(x)
    return np.asarray(x, dtype=np.uint16).view(np.float16).astype(np.float32)


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# codecs
# ---------------------------------------------------------------------------

def pin_decode_closed_forms(L):
    g = _golden("fp8_format_constants.json")
    for fmt in FORMATS:
        for entry in g[fmt]["codes"]:
            code, want = int(entry["code"], 16), entry["value"]
            got = float(L.fp8_decode(np.array([code], np.uint8), fmt)[0])
            if want == "nan":
                assert np.isnan(got), (fmt, hex(code), got)
            else:
                w = float(want)
                assert got == w and np.signbit(got) == np.signbit(w), (fmt, hex(code), got, want)
        assert L.fp8_max(fmt) == float(g[fmt]["max"]), fmt


def pin_decode_all_codes_vs_torch(L):
    codes = np.arange(256, dtype=np.uint8)
    for fmt in FORMATS:
        ref = torch.from_numpy(codes).view(TORCH_FP8[fmt]).float().numpy()
        got = L.fp8_decode(codes, fmt)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan), fmt
        assert np.array_equal(_bits32(got)[~nan], _bits32(ref)[~nan]), fmt
        # and against the exact bit-field definition
        for c in range(256):
            v = X.fp8_value(c, fmt)
            if v == "nan":
                assert np.isnan(got[c])
            elif isinstance(v, str):
                assert np.isinf(got[c]) and (got[c] > 0) == (v == "inf")
            else:
                assert Fraction(float(got[c])) == v and (np.signbit(got[c]) == bool(c & 0x80)), (fmt, c)


def pin_encode_roundtrip_all_codes(L):
    for fmt in FORMATS:
        codes = np.arange(256, dtype=np.uint8)
        vals = L.fp8_decode(codes, fmt)
        back = L.fp8_encode(vals, fmt)
        finite = np.isfinite(vals)
        assert np.array_equal(back[finite], codes[finite]), fmt
        assert np.all((back[np.isnan(vals)] & 0x7F) == 0x7F), fmt          # NaN -> S.1111111
        maxc = X.FMT[fmt][3]
        inf = np.isinf(vals)
        assert np.all((back[inf] & 0x7F) == maxc), fmt                   # inf saturates


def _encode_sweep_inputs(fmt):
    return np.concatenate([X.structured_f32_sweep(), X.random_f32_bits(1 << 18, seed=11),
                           X.fp8_midpoints(fmt)])


def pin_encode_nearest_search(L):
    for fmt in FORMATS:
        v = _encode_sweep_inputs(fmt)
        got = L.fp8_encode(v, fmt)
        ref = X.nearest_fp8_codes(v, fmt)
        nan = np.isnan(v)
        assert np.all((got[nan] & 0x7F) == 0x7F), fmt
        bad = np.nonzero(got[~nan] != ref[~nan])[0]
        assert bad.size == 0, (fmt, bad.size, v[~nan][bad[:5]], got[~nan][bad[:5]], ref[~nan][bad[:5]])


def pin_encode_vs_torch_in_range(L):
    """torch's CPU cast is RNE but not saturating: where it yields NaN/inf for a
    finite binary32 input the oracle yields +-max; everywhere else they agree."""
    for fmt in FORMATS:
        v = _encode_sweep_inputs(fmt)
        v = v[np.isfinite(v)]
        ref = torch.from_numpy(v).to(TORCH_FP8[fmt]).view(torch.uint8).numpy()
        got = L.fp8_encode(v, fmt)
        maxc = X.FMT[fmt][3]
        overflow = (ref & 0x7F) > maxc
        assert np.array_equal(got[~overflow], ref[~overflow]), fmt
        assert np.all((got[overflow] & 0x7F) == maxc), fmt
        assert np.array_equal(got[overflow] & 0x80, ref[overflow] & 0x80), fmt


def pin_encode_monotone(L):
    for fmt in FORMATS:
        v = np.sort(np.abs(X.random_f32_bits(1 << 16, seed=12)))
        v = v[np.isfinite(v)]
        c = L.fp8_encode(v, fmt).astype(np.int32)
        assert np.all(np.diff(c) >= 0), fmt


def pin_bf16_vs_torch(L):
    v = np.concatenate([X.structured_f32_sweep(low_patterns=(0, 1, 0x7FFF, 0x8000 >> 1)),
                        X.random_f32_bits(1 << 18, seed=13)])
    v = np.concatenate([v, np.array([3.0e38, 3.4028235e38, 1.0 + 2 ** -8, 1.0 + 2 ** -8 + 2 ** -23],
                                    dtype=np.float32)])
    got = L.bf16_from_f32(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(v)
    assert np.all((got[nan] & 0x7F80) == 0x7F80) and np.all((got[nan] & 0x7F) != 0)
    assert np.array_equal(got[~nan], ref[~nan])


def pin_f16_vs_numpy(L):
    v = np.concatenate([X.structured_f32_sweep(), X.random_f32_bits(1 << 18, seed=14)])
    got = L.f16_from_f32(v)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    nan = np.isnan(v)
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all((got[nan] & 0x3FF) != 0)
    assert np.array_equal(got[~nan], ref[~nan])


# ---------------------------------------------------------------------------
# whole operations: exact rational references on tiny inputs
# ---------------------------------------------------------------------------

def _tiny_inputs(dtype, shape, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal(shape).astype(np.float32)
    x *= (2.0 ** rng.integers(-12, 12, size=shape)).astype(np.float32)   # wide dynamic range
    x.reshape(-1)[:: 37] = 0.0
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return x.astype(np.float16).view(np.uint16)


def _ydtype_round(p: Fraction, ydtype, negative: bool):
    """Round an exact binary32 product to the output type; `negative` restores
    the sign of a product that is (or rounds to) zero."""
    if ydtype == "f32":
        v = X.f32(p)
        return -v if (negative and v == 0) else v
    if ydtype == "bf16":
        b = np.uint16(_bits32(X.f32(X.rn_bf16(p)))[()] >> 16)
        return np.uint16(b | 0x8000) if (negative and b == 0) else b
    r = X.rn_f16(p)
    h = np.float16(float(r) if not isinstance(r, str) else r).view(np.uint16)
    return np.uint16(h | 0x8000) if (negative and h == 0) else h


def _exact_cast(vals_f32, fmt, amax_guard, scale_inv_rule):
    """vals_f32: binary32 values of one reduction unit (tensor, row or group)."""
    fmax = Fraction(float(X.fp8_value(X.FMT[fmt][3], fmt)))
    fr = [X.frac(v) for v in vals_f32]
    amax = max((abs(v) for v in fr), default=Fraction(0))
    if amax_guard == "zero_to_one":
        a = amax if amax > 0 else Fraction(1)
    else:  # clamp at fl32(1e-4)
        c = X.rn32(Fraction(1e-4))
        a = amax if amax >= c else c
    scale = X.rn32(fmax / a)
    if scale_inv_rule == "one_over_scale":
        sinv = X.rn32(1 / scale)
    else:
        sinv = X.rn32(a / fmax)
    q = [X.enc_fp8_exact(X.rn32(v * scale), bool(np.signbit(np.float32(fv))), fmt)
         for v, fv in zip(fr, vals_f32)]
    return np.array(q, dtype=np.uint8), X.f32(sinv)


def pin_exact_cast_per_group128(L):
    for fmt in FORMATS:
        for dtype in ("bf16", "f32", "f16"):
            x = _tiny_inputs(dtype, (3, 256), seed=21)
            x[1, :128] = 0                                  # an all-zero group
            xf = _widen(x, dtype).copy()
            if dtype == "f32":
                x[2, 128:] = xf[2, 128:] * np.float32(1e-7)  # a group below the clamp
                xf = _widen(x, dtype)
            q, si = L.cast_per_group128(x, dtype, fmt)
            for r in range(3):
                for g in range(2):
                    eq, es = _exact_cast(xf[r, 128 * g:128 * (g + 1)], fmt, "clamp", "amax_over_max")
                    assert np.array_equal(q[r, 128 * g:128 * (g + 1)], eq), (fmt, dtype, r, g)
                    assert _bits32(si[r, g]) == _bits32(es), (fmt, dtype, r, g, si[r, g], es)


def pin_exact_cast_per_channel(L):
    for fmt in FORMATS:
        for dtype in ("f32", "bf16", "f16"):
            x = _tiny_inputs(dtype, (4, 50), seed=22)
            x[2, :] = 0
            xf = _widen(x, dtype)
            q, si = L.cast_per_channel(x, dtype, fmt)
            for r in range(4):
                eq, es = _exact_cast(xf[r], fmt, "zero_to_one", "amax_over_max")
                assert np.array_equal(q[r], eq), (fmt, dtype, r)
                assert _bits32(si[r]) == _bits32(es), (fmt, dtype, r)


def pin_exact_cast_per_tensor(L):
    for fmt in FORMATS:
        for dtype in ("f32", "bf16", "f16"):
            x = _tiny_inputs(dtype, (200,), seed=23)
            q, si = L.cast_per_tensor(x, dtype, fmt)
            eq, es = _exact_cast(_widen(x, dtype), fmt, "zero_to_one", "one_over_scale")
            assert np.array_equal(q, eq), (fmt, dtype)
            assert _bits32(si[0]) == _bits32(es), (fmt, dtype, si, es)
        z = np.zeros(7, np.float32)
        q, si = L.cast_per_tensor(z, "f32", fmt)
        eq, es = _exact_cast(z, fmt, "zero_to_one", "one_over_scale")
        assert np.array_equal(q, eq) and _bits32(si[0]) == _bits32(es)


def pin_scale_inv_rules_differ(L):
    """The three granularities use different scale_inv formulas; an amax where
    1/(fmax/amax) and amax/fmax round differently must show the difference."""
    amax = np.float32(11.0)             # 1/fl32(448/11) != fl32(11/448) in binary32
    fmax = Fraction(448)
    s = X.rn32(fmax / Fraction(11))
    assert X.rn32(1 / s) != X.rn32(Fraction(11) / fmax)
    x = np.zeros((1, 128), np.float32)
    x[0, 5] = amax
    _, si_g = L.cast_per_group128(x, "f32", "e4m3fn")
    _, si_c = L.cast_per_channel(x, "f32", "e4m3fn")
    _, si_t = L.cast_per_tensor(x, "f32", "e4m3fn")
    assert Fraction(float(si_g[0, 0])) == X.rn32(Fraction(11) / fmax)
    assert Fraction(float(si_c[0])) == X.rn32(Fraction(11) / fmax)
    assert Fraction(float(si_t[0])) == X.rn32(1 / s)


def pin_exact_dequant(L):
    rng = np.random.Generator(np.random.PCG64(24))
    for fmt in FORMATS:
        maxc = X.FMT[fmt][3]
        codes = np.array([c for c in range(256) if (c & 0x7F) <= maxc], dtype=np.uint8)
        q = rng.choice(codes, size=(3, 256)).astype(np.uint8)
        si_g = (10.0 ** rng.uniform(-6, 2, size=(3, 2))).astype(np.float32)
        si_r = si_g[:, 0].copy()
        si_t = si_g[:1, 0].copy()
        for ydt in ("f32", "bf16", "f16"):
            yg = L.dequant_per_group128(q, fmt, si_g, ydt)
            yr = L.dequant_per_channel(q, fmt, si_r, ydt)
            yt = L.dequant_per_tensor(q, fmt, si_t, ydt)
            for r in range(3):
                for c in range(0, 256, 7):
                    d = X.fp8_value(int(q[r, c]), fmt)
                    neg = bool(q[r, c] & 0x80)
                    for y, s in ((yg, si_g[r, c // 128]), (yr, si_r[r]), (yt, si_t[0])):
                        want = _ydtype_round(X.rn32(d * X.frac(s)), ydt, neg)
                        got = y[r, c]
                        if ydt == "f32":
                            assert _bits32(got) == _bits32(want), (fmt, ydt, r, c, got, want)
                        else:
                            assert int(got) == int(want), (fmt, ydt, r, c, got, want)


def pin_block_dequant_index(L):
    """Distinct power-of-two scales per 128x128 tile on a ragged, non-square
    shape: every output must equal dec(q) * 2^k(tile) exactly, which fixes the
    tile index (row block, col block) and the ceil(M/128) x ceil(N/128) grid."""
    rng = np.random.Generator(np.random.PCG64(25))
    M, N = 300, 200
    nbm, nbn = 3, 2
    k = np.arange(nbm * nbn).reshape(nbm, nbn) - 3
    s = (2.0 ** k).astype(np.float32)
    for fmt in FORMATS:
        maxc = X.FMT[fmt][3]
        codes = np.array([c for c in range(256) if (c & 0x7F) <= maxc], dtype=np.uint8)
        q = rng.choice(codes, size=(M, N)).astype(np.uint8)
        d = L.fp8_decode(q, fmt).astype(np.float64)
        want = d * (2.0 ** k)[np.arange(M)[:, None] // 128, np.arange(N)[None, :] // 128]
        y = L.weight_dequant_block128(q, fmt, s, "f32")
        assert np.array_equal(y.astype(np.float64), want), fmt
        yb = L.weight_dequant_block128(q, fmt, s, "bf16")
        assert np.array_equal(_bf16_to_f32(yb).astype(np.float64), want), fmt   # fp8 values fit bf16


# ---------------------------------------------------------------------------
# invariants and special cases
# ---------------------------------------------------------------------------

def pin_amax_element_maps_to_max(L):
    from dequantize_amax_reduce_amd import workloads as W
    x, zr = W.group_cast_small()
    xf = _bf16_to_f32(x)
    for fmt in FORMATS:
        maxc = X.FMT[fmt][3]
        q, si = L.cast_per_group128(x, "bf16", fmt)
        g = np.abs(xf.reshape(-1, 128))
        qg = q.reshape(-1, 128)
        nz = g.max(axis=1) >= np.float32(1e-4)
        arg = g.argmax(axis=1)
        assert np.all((qg[np.arange(qg.shape[0]), arg][nz] & 0x7F) == maxc), fmt
        dec = np.abs(L.fp8_decode(q, fmt))
        assert np.all(dec <= L.fp8_max(fmt)), fmt
    xt, _, _ = W.tensor_rows_scaled(rows=64, cols=96, seed=2, zero_frac=0.05)
    for fmt in FORMATS:
        maxc = X.FMT[fmt][3]
        q, si = L.cast_per_channel(xt, "f32", fmt)
        a = np.abs(xt)
        rows = np.nonzero(a.max(axis=1) > 0)[0]
        assert np.all((q[rows, a[rows].argmax(axis=1)] & 0x7F) == maxc), fmt
        q, si = L.cast_per_tensor(xt, "f32", fmt)
        assert (q.reshape(-1)[a.argmax()] & 0x7F) == maxc, fmt


def zero_constants_from_math():
    """The zero/empty constants re-derived with exact rational arithmetic."""
    def h(fr):
        return "0x%08X" % int(_bits32(X.f32(fr))[()])
    c = X.rn32(Fraction(1e-4))
    out = {"clamp_1e-4": h(c)}
    for fmt in FORMATS:
        m = Fraction(int(X.fp8_value(X.FMT[fmt][3], fmt)))
        out[fmt] = {"zero_group_scale": h(X.rn32(m / c)), "zero_group_scale_inv": h(X.rn32(c / m)),
                    "zero_row_scale_inv": h(X.rn32(1 / m)),
                    "zero_tensor_scale_inv": h(X.rn32(1 / X.rn32(m))), "empty_scale_inv": 1.0}
    return out


def pin_zero_and_empty_constants(L):
    g = _golden("zero_and_empty_constants.json")
    for fmt in FORMATS:
        c = g[fmt]
        z = np.zeros((2, 256), np.uint16)                      # bf16 +0.0
        q, si = L.cast_per_group128(z, "bf16", fmt)
        assert np.all(q == 0) and np.all(_bits32(si) == int(c["zero_group_scale_inv"], 16)), fmt
        q, si = L.cast_per_channel(np.zeros((3, 5), np.float32), "f32", fmt)
        assert np.all(q == 0) and np.all(_bits32(si) == int(c["zero_row_scale_inv"], 16)), fmt
        q, si = L.cast_per_tensor(np.zeros(9, np.float32), "f32", fmt)
        assert np.all(q == 0) and _bits32(si[0]) == int(c["zero_tensor_scale_inv"], 16), fmt
        q, si = L.cast_per_tensor(np.zeros(0, np.float32), "f32", fmt)
        assert si[0] == 1.0, fmt
        q, si = L.cast_per_channel(np.zeros((4, 0), np.float32), "f32", fmt)
        assert np.all(si == 1.0), fmt
        # negative zeros keep their sign
        nz = np.full(128, 0x8000, np.uint16)
        q, _ = L.cast_per_group128(nz.reshape(1, 128), "bf16", fmt)
        assert np.all(q == 0x80), fmt


def pin_power_of_two_metamorphic(L):
    """Scaling a unit by 2^k (no overflow/underflow/clamp interaction) keeps q
    bit-identical and multiplies scale_inv by exactly 2^k."""
    from dequantize_amax_reduce_amd import workloads as W
    x, _, _ = W.tensor_rows_scaled(rows=16, cols=256, seed=7, zero_frac=0.0)
    x = x / np.abs(x).max(axis=1, keepdims=True)            # amax 1 per row: room both ways
    for fmt in FORMATS:
        for k in (-5, 3, 11):
            xs = (x * np.float32(2.0 ** k)).astype(np.float32)
            for op in ("cast_per_group128", "cast_per_channel", "cast_per_tensor"):
                q0, s0 = getattr(L, op)(x, "f32", fmt)
                q1, s1 = getattr(L, op)(xs, "f32", fmt)
                assert np.array_equal(q0, q1), (fmt, k, op)
                assert np.array_equal(s0 * np.float32(2.0 ** k), s1), (fmt, k, op)


def pin_nan_propagation(L):
    """torch's max propagates NaN: per-tensor/per-channel then take amax=NaN
    through torch.where(amax > 0, amax, 1) -> 1; per-group's clamp keeps NaN,
    so the whole group becomes NaN and so does its scale_inv."""
    for fmt in FORMATS:
        x = np.ones((2, 128), np.float32)
        x[0, 3] = np.nan
        q, si = L.cast_per_group128(x, "f32", fmt)
        assert np.isnan(si[0, 0]) and np.all((q[0] & 0x7F) == 0x7F), fmt
        assert not np.isnan(si[1, 0]) and np.all((q[1] & 0x7F) == X.FMT[fmt][3])
        q, si = L.cast_per_channel(x, "f32", fmt)
        fmax = Fraction(L.fp8_max(fmt))
        assert Fraction(float(si[0])) == X.rn32(1 / fmax), fmt          # NaN amax -> 1
        assert (q[0, 3] & 0x7F) == 0x7F, fmt
        q, si = L.cast_per_tensor(x, "f32", fmt)
        assert Fraction(float(si[0])) == X.rn32(1 / X.rn32(fmax)), fmt


def pin_roundtrip_error_bound(L):
    """|dec(q) * scale_inv - x| <= 2^-(mbits+1) |x| (half an ulp of the format,
    plus a few binary32 ulps) for every element whose scaled value is normal."""
    from dequantize_amax_reduce_amd import workloads as W
    x, _ = W.group_cast_small()
    xf = _bf16_to_f32(x).astype(np.float64)
    for fmt in FORMATS:
        mb = X.FMT[fmt][0]
        q, si = L.cast_per_group128(x, "bf16", fmt)
        y = L.fp8_decode(q, fmt).astype(np.float64) * np.repeat(si.astype(np.float64), 128, axis=1)
        minnorm = 2.0 ** (2 - 2 ** (X.FMT[fmt][1] - 1))
        scaled = np.abs(xf) / np.repeat(si.astype(np.float64), 128, axis=1)
        m = scaled >= minnorm
        rel = np.abs(y[m] - xf[m]) / np.abs(xf[m])
        assert rel.max() <= 2.0 ** -(mb + 1) * (1 + 2 ** -20), (fmt, rel.max())


def pin_page_worked_shapes(L):
    """"5 Utils" page, per_token_cast_to_fp8 shapes: n=512 gives g=4 groups,
    x_view (m, 4, 128) and scales (m, 4); input needs n % 128 == 0."""
    g = _golden("per_token_shapes.json")
    for case in g["cases"]:
        m, n = case["m"], case["n"]
        x = np.ones((m, n), np.uint16) * 0x3F80               # bf16 1.0
        q, si = L.cast_per_group128(x, "bf16", "e4m3fn")
        assert list(si.shape) == case["scales_shape"] and list(q.shape) == [m, n]
        assert np.all(q == 0x7E)                              # every 1.0 is the group amax -> 448
    try:
        L.cast_per_group128(np.ones((2, 100), np.uint16), "bf16", "e4m3fn")
    except ValueError:
        pass
    else:
        raise AssertionError("n % 128 != 0 must be rejected")


# ---------------------------------------------------------------------------
# reduce step of the compressed all-reduce / reduce-scatter
# ---------------------------------------------------------------------------

TORCH_HP = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _hp_bits(t: torch.Tensor, dtype):
    if dtype == "f32":
        return t.numpy().view(np.uint32)
    return t.view(torch.int16).numpy().view(np.uint16)


def _sum_inputs(W, n, fmt, seed):
    """W chunks made the way the collectives make them: each a per-tensor cast
    (with its own scale) of a tensor of a different magnitude."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = np.empty((W, n), np.uint8)
    si = np.empty(W, np.float32)
    fmax = float(X.fp8_value(X.FMT[fmt][3], fmt))
    for w in range(W):
        amax = np.float32(10.0 ** rng.uniform(-4, 3))
        x = (rng.standard_normal(n) * amax).astype(np.float32)
        scale = np.float32(fmax) / np.float32(np.abs(x).max())
        q[w] = torch.from_numpy(np.clip(x * scale, -fmax, fmax)).to(TORCH_FP8[fmt]).view(torch.uint8).numpy()
        si[w] = np.float32(1.0) / scale
    return q, si


def pin_dequant_sum_vs_torch(L):
    """The pages' reduce loop evaluated by torch on the CPU: summed_out =
    zeros(input_type); summed_out += (scale_inv * q.float()).to(input_type) per
    chunk in order; summed_out.div_(W) for AVG (W a power of two, where torch's
    division and a true division agree)."""
    for fmt in FORMATS:
        for dtype in ("bf16", "f32", "f16"):
            for W in (1, 2, 4, 8):
                q, si = _sum_inputs(W, 333, fmt, seed=W * 7 + len(dtype))
                for average in (False, True):
                    summed = torch.zeros(333, dtype=TORCH_HP[dtype])
                    for w in range(W):
                        term = (torch.tensor(si[w]) * torch.from_numpy(q[w]).view(TORCH_FP8[fmt]).float())
                        summed += term.to(TORCH_HP[dtype])
                    if average:
                        summed.div_(W)
                    got = L.dequant_sum(q, fmt, si, dtype, average)
                    want = _hp_bits(summed, dtype)
                    assert np.array_equal(np.asarray(got).view(want.dtype), want), (fmt, dtype, W, average)


def pin_dequant_sum_exact(L):
    """Exact rational reference on small inputs, W = 3 (not a power of two):
    each term and each partial sum rounded to the type, then the division."""
    rnd = {"f32": X.rn32, "bf16": X.rn_bf16, "f16": X.rn_f16}
    for fmt in FORMATS:
        for dtype in ("bf16", "f32", "f16"):
            q, si = _sum_inputs(3, 40, fmt, seed=5)
            for average in (False, True):
                got = L.dequant_sum(q, fmt, si, dtype, average)
                for i in range(40):
                    acc = Fraction(0)
                    for w in range(3):
                        term = rnd[dtype](X.rn32(X.fp8_value(int(q[w, i]), fmt) * X.frac(si[w])))
                        acc = rnd[dtype](X.rn32(acc + term))
                    if average:
                        acc = rnd[dtype](X.rn32(acc / 3))
                    g = got[i]
                    gv = Fraction(float(g)) if dtype == "f32" else (
                        Fraction(float(_bf16_to_f32(g))) if dtype == "bf16" else
                        Fraction(float(np.uint16(g).view(np.float16))))
                    assert gv == acc, (fmt, dtype, average, i, gv, acc)


def pin_dequant_sum_special(L):
    """IEEE facts the loop must keep: the sum starts from +0 (zeros), so chunks
    of -0 sum to +0; and the in-type accumulation is order dependent:
    1 + 2^-8 + 2^-8 in chunk order is 1 in bf16 (each addition ties to even)."""
    fmt = "e4m3fn"
    q = np.full((3, 4), 0x80, np.uint8)                          # -0 everywhere
    for dtype in ("bf16", "f32", "f16"):
        y = np.asarray(L.dequant_sum(q, fmt, np.ones(3, np.float32), dtype))
        assert np.all(y.view(np.uint32 if dtype == "f32" else np.uint16) == 0), dtype
    one, tiny = 0x38, 0x08                                       # e4m3fn: 1.0 and 2^-6
    q = np.array([[one], [tiny], [tiny]], np.uint8)
    si = np.array([1.0, 0.25, 0.25], np.float32)                  # terms 1, 2^-8, 2^-8
    y = L.dequant_sum(q, fmt, si, "bf16")
    assert int(y[0]) == 0x3F80, hex(int(y[0]))                    # 1.0, not 1.0078125
    y = L.dequant_sum(q[::-1].copy(), fmt, si[::-1].copy(), "bf16")
    assert int(y[0]) == 0x3F81, hex(int(y[0]))                    # 2^-8 + 2^-8 + 1 = 1.0078125


def pin_dequant_sum_requant_is_cast_of_sum(L):
    for fmt in FORMATS:
        q, si = _sum_inputs(4, 500, fmt, seed=9)
        y, qo, so = L.dequant_sum_requant(q, fmt, si, "bf16", True)
        wq, ws = L.cast_per_tensor(np.asarray(y), "bf16", fmt)
        assert np.array_equal(qo, wq) and so[0] == ws[0]
        assert np.array_equal(np.asarray(y), np.asarray(L.dequant_sum(q, fmt, si, "bf16", True)))


# ---------------------------------------------------------------------------
# FSDP parameter hook: cross-rank global amax, cast with it, dequant by division
# ---------------------------------------------------------------------------

def pin_fsdp_hook_vs_torch(L):
    """The hook's expressions evaluated by torch on the CPU for two simulated
    ranks: per_tensor_max = where(abs().max().float() > 0, ., 1) per rank, MAX
    over the ranks, scale = fp8_max / max (written as a true division, R8),
    (scale * inp.float()).to(fp8), then (fp8.float() / scale).to(out.dtype)."""
    rng = np.random.Generator(np.random.PCG64(41))
    for fmt in FORMATS:
        fmax = float(X.fp8_value(X.FMT[fmt][3], fmt))
        for dtype in ("bf16", "f32", "f16"):
            shards = [(rng.standard_normal(257) * 10.0 ** rng.uniform(-3, 2)).astype(np.float32) for _ in range(2)]
            shards.append(np.zeros(100, np.float32))                  # a rank holding zeros contributes 1
            hs = [torch.from_numpy(s_).to(TORCH_HP[dtype]) for s_ in shards]
            host = [_hp_bits(h, dtype) if dtype != "f32" else h.numpy() for h in hs]
            locs = [torch.where(h.abs().max().float() > 0, h.abs().max().float(), torch.tensor(1.0)) for h in hs]
            for h_, t in zip(host, locs):
                assert np.float32(L.amax_guarded(h_, dtype)) == np.float32(t.item()), (fmt, dtype)
            gmax = torch.stack(locs).max()
            scale = torch.div(torch.tensor(fmax, dtype=torch.float32), gmax)
            for h, h_ in zip(hs, host):
                want_q = (scale * h.float()).to(TORCH_FP8[fmt]).view(torch.uint8).numpy()
                q, sc = L.cast_with_amax(h_, dtype, fmt, gmax.item())
                assert np.float32(sc[0]) == np.float32(scale.item()), (fmt, dtype)
                assert np.array_equal(q, want_q), (fmt, dtype)
                for ydt in ("bf16", "f32", "f16"):
                    want_y = (torch.from_numpy(q).view(TORCH_FP8[fmt]).float() / scale).to(TORCH_HP[ydt])
                    got = np.asarray(L.dequant_div_scale(q, fmt, sc[0], ydt))
                    assert np.array_equal(got.view(np.uint8), _hp_bits(want_y, ydt).view(np.uint8)), (fmt, dtype, ydt)


def pin_dequant_div_scale_exact(L):
    """Division, not a product with 1/scale: exact rationals on every code."""
    for fmt in FORMATS:
        maxc = X.FMT[fmt][3]
        codes = np.array([c for c in range(256) if (c & 0x7F) <= maxc], dtype=np.uint8)
        for sc in (np.float32(3.0), np.float32(0.1), np.float32(448.0 / 2.7)):
            for ydt, rnd in (("f32", X.rn32), ("bf16", X.rn_bf16)):
                y = L.dequant_div_scale(codes, fmt, sc, ydt)
                for c, g in zip(codes, y):
                    want = rnd(X.rn32(X.fp8_value(int(c), fmt) / X.frac(sc)))
                    gv = Fraction(float(g)) if ydt == "f32" else Fraction(float(_bf16_to_f32(g)))
                    assert gv == want, (fmt, hex(int(c)), sc, ydt)


# ---------------------------------------------------------------------------
# pipeline p2p cast: the format chosen from the data
# ---------------------------------------------------------------------------

def pin_pipeline_vs_torch(L):
    """cast_to_fp8_pipeline / cast_from_fp8_pipeline evaluated by torch on the
    CPU: aminmax, maximum of the absolute values, the 448 threshold, the zero
    test, scale = finfo.max / amax (a true division, R8), (x.float() * scale)
    .to(fp8), fp8_scale = scale.reciprocal(); back: q.to(dtype) * fp8_scale."""
    rng = np.random.Generator(np.random.PCG64(43))
    for dtype in ("bf16", "f32", "f16"):
        cases = [rng.standard_normal(300) * 10.0 ** e for e in (-3, 0, 2, 2.7, 3.5)]
        cases += [np.zeros(64), np.array([448.0, -3.0]), np.array([-1.0, 2.0, -449.0 if dtype != "bf16" else -450.0])]
        for xv in cases:
            h = torch.from_numpy(np.asarray(xv, np.float32)).to(TORCH_HP[dtype])
            lo, hi = h.aminmax()
            amax = torch.maximum(lo.abs(), hi.abs())
            fmt = "e5m2" if amax > torch.finfo(torch.float8_e4m3fn).max else "e4m3fn"
            fmax = torch.finfo(TORCH_FP8[fmt]).max
            scale = torch.tensor(1.0) if amax == 0.0 else torch.div(torch.tensor(fmax, dtype=torch.float32), amax.float())
            want_q = (h.float() * scale).to(TORCH_FP8[fmt]).view(torch.uint8).numpy()
            want_si = scale.float().reciprocal()
            host = _hp_bits(h, dtype) if dtype != "f32" else h.numpy()
            q, si, gfmt = L.cast_to_fp8_pipeline(host, dtype)
            assert gfmt == fmt, (dtype, gfmt, fmt)
            assert np.array_equal(q, want_q), (dtype, fmt)
            assert np.float32(si[0]).view(np.uint32) == np.float32(want_si.item()).view(np.uint32), (dtype, fmt)
            for ydt in ("bf16", "f32", "f16"):
                want_y = torch.from_numpy(q).view(TORCH_FP8[fmt]).to(TORCH_HP[ydt]) * want_si
                got = np.asarray(L.cast_from_fp8_pipeline(q, fmt, si[0], ydt))
                assert np.array_equal(got.view(np.uint8), _hp_bits(want_y, ydt).view(np.uint8)), (dtype, fmt, ydt)


def pin_pipeline_format_rule(L):
    """The threshold and the degenerate amax values, from their definitions:
    amax = 448 keeps e4m3fn with scale 1; the next value up in each type
    switches to e5m2; the element at amax always lands on the format's largest
    code; zero gives scale 1; NaN keeps e4m3fn with a NaN scale (NaN codes);
    inf gives e5m2 with scale 0 (finite -> signed zero, inf -> NaN); an empty
    tensor is amax 0."""
    nxt = {"f32": np.float32(np.nextafter(np.float32(448), np.float32(np.inf))),
           "bf16": np.float32(450.0), "f16": np.float32(448.25)}
    for dtype in ("f32", "bf16", "f16"):
        enc = (lambda v: (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)) if dtype == "bf16" else (  # exact values only
            (lambda v: np.asarray(v, np.float32).astype(np.float16).view(np.uint16)) if dtype == "f16" else
            (lambda v: np.asarray(v, np.float32)))
        q, si, f = L.cast_to_fp8_pipeline(enc(np.array([448.0, -1.0, 0.5], np.float32)), dtype)
        assert f == "e4m3fn" and si[0] == 1.0 and list(q) == [0x7E, 0xB8, 0x30], (dtype, q, si, f)
        q, si, f = L.cast_to_fp8_pipeline(enc(np.array([0.25, -nxt[dtype]], np.float32)), dtype)
        want_scale = X.rn32(Fraction(57344) / X.frac(nxt[dtype]))
        assert f == "e5m2" and q[1] == 0xFB, (dtype, q, f)
        assert X.frac(si[0]) == X.rn32(1 / want_scale), dtype
        q, si, f = L.cast_to_fp8_pipeline(enc(np.zeros(5, np.float32)), dtype)
        assert f == "e4m3fn" and si[0] == 1.0 and not q.any(), dtype
        q, si, f = L.cast_to_fp8_pipeline(enc(np.array([1.0, np.nan, -2.0], np.float32)), dtype)
        assert f == "e4m3fn" and np.isnan(si[0]) and all((int(c) & 0x7F) == 0x7F for c in q), (dtype, q)
        q, si, f = L.cast_to_fp8_pipeline(enc(np.array([1.0, -np.inf, -2.0], np.float32)), dtype)
        assert f == "e5m2" and si[0] == np.inf and q[0] == 0x00 and q[2] == 0x80, (dtype, q, si)
        assert (int(q[1]) & 0x7F) > 0x7C, (dtype, q)              # -inf * 0 = NaN
        q, si, f = L.cast_to_fp8_pipeline(enc(np.zeros(0, np.float32)), dtype)
        assert f == "e4m3fn" and si[0] == 1.0 and q.size == 0
    rng = np.random.Generator(np.random.PCG64(44))
    for _ in range(20):
        x = (rng.standard_normal(257) * 10.0 ** rng.uniform(-5, 5)).astype(np.float32)
        q, si, f = L.cast_to_fp8_pipeline(x, "f32")
        i = int(np.argmax(np.abs(x)))
        assert (int(q[i]) & 0x7F) == X.FMT[f][3], (f, hex(int(q[i])))
        assert f == ("e5m2" if np.abs(x).max() > 448 else "e4m3fn")
    # amax so small that fmax / amax overflows: the scale is inf, zero -> NaN,
    # nonzero -> the largest code (saturation, R2)
    q, si, f = L.cast_to_fp8_pipeline(np.array([1e-40, 0.0, -1e-40], np.float32), "f32")
    assert f == "e4m3fn" and si[0] == 0.0 and q[0] == 0x7E and (int(q[1]) & 0x7F) == 0x7F and q[2] == 0xFE, (q, si)


def pin_pipeline_dequant_exact(L):
    """Back from either format, every code, exact rationals: the code's value
    (exact in every output type) times scale_inv, rounded to binary32, then to
    the output type; equal to the per-tensor dequant."""
    for fmt in FORMATS:
        maxc = X.FMT[fmt][3]
        codes = np.array([c for c in range(256) if (c & 0x7F) <= maxc], dtype=np.uint8)
        for si in (np.float32(1.0), np.float32(0.1), np.float32(1.0 / 448.0 * 3.3), np.float32(2.0 ** -20)):
            for ydt, rnd in (("f32", X.rn32), ("bf16", X.rn_bf16), ("f16", X.rn_f16)):
                y = L.cast_from_fp8_pipeline(codes, fmt, si, ydt)
                assert np.array_equal(np.asarray(y).view(np.uint8),
                                      np.asarray(L.dequant_per_tensor(codes, fmt, np.array([si]), ydt)).view(np.uint8))
                if ydt == "f16":
                    continue
                for c, g in zip(codes, y):
                    want = rnd(X.rn32(X.fp8_value(int(c), fmt) * X.frac(si)))
                    gv = Fraction(float(g)) if ydt == "f32" else Fraction(float(_bf16_to_f32(g)))
                    assert gv == want, (fmt, hex(int(c)), si, ydt)


# ---------------------------------------------------------------------------
# packed [scale_inv | payload] slots of the fp8 all-gather
# ---------------------------------------------------------------------------

def _page_cast_into(inp: torch.Tensor, fmt: str, out: torch.Tensor):
    """cast_to_fp8(inp, per-tensor, out=out) as the page writes it, evaluated
    by torch on the CPU (the scale as a true division, R8)."""
    fp8_type = TORCH_FP8[fmt]
    if inp.numel() == 0:
        return torch.tensor([1.0])
    m = inp.abs().max().float()
    m = torch.where(m > 0, m, 1.0)
    scale = torch.div(torch.tensor(torch.finfo(fp8_type).max, dtype=torch.float32), m)
    scale_inv = 1.0 / scale
    torch.mul(scale, inp.float(), out=out)
    return torch.unsqueeze(scale_inv, 0)


def pin_packed_slots_vs_torch(L):
    """all_gather_fp8_lagacy's buffer handling, with W simulated ranks, run by
    torch on the CPU: the combined buffer of W * (4 + n) bytes, chunked per
    rank; each rank casts into slot[4:] and stores scale_inv into slot[0:4];
    every slot is read back with slot[:4].clone().view(float) and
    cast_from_fp8(..., out=...)."""
    rng = np.random.Generator(np.random.PCG64(45))
    for fmt in FORMATS:
        for dtype in ("bf16", "f32", "f16"):
            for W, n in ((1, 37), (3, 64), (4, 1000), (2, 0)):
                xs = [torch.from_numpy((rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32))
                      .to(TORCH_HP[dtype]) for _ in range(W)]
                if W > 2:
                    xs[1].zero_()                               # a rank holding zeros
                combined = torch.zeros(W * (4 + n), dtype=torch.uint8)
                bufs = list(combined.chunk(W)) if n + 4 > 0 else []
                got_slots = np.zeros(W * (4 + n), np.uint8)
                for r in range(W):
                    cur = bufs[r]
                    sinv = _page_cast_into(xs[r].view(-1), fmt, cur[4:].view(TORCH_FP8[fmt]))
                    cur[:4].view(torch.float)[0] = sinv
                    host = _hp_bits(xs[r], dtype) if dtype != "f32" else xs[r].numpy()
                    got_slots[r * (4 + n):(r + 1) * (4 + n)] = L.cast_to_packed(host, dtype, fmt)
                assert np.array_equal(got_slots, combined.numpy()), (fmt, dtype, W, n)
                for ydt in ("bf16", "f32", "f16"):
                    want = torch.empty((W, n), dtype=TORCH_HP[ydt])
                    for r in range(W):
                        scale = bufs[r][:4].clone().view(torch.float)
                        torch.mul(scale, bufs[r][4:].view(TORCH_FP8[fmt]).float(), out=want[r])
                    got = np.asarray(L.dequant_packed(combined.numpy(), fmt, W, n, ydt))
                    assert np.array_equal(got.view(np.uint8), _hp_bits(want, ydt).view(np.uint8)), (fmt, W, n, ydt)


def pin_packed_layout_closed_form(L):
    """Byte-level layout from the definition: an all-zero rank stores
    scale_inv = fl32(1/fp8_max) as little-endian bytes at offset 0 and zero
    codes after it; a rank holding [fp8_max, -1] stores scale_inv = 1 and the
    codes of fp8_max and -1; an empty rank stores 1.0.  Reading two slots back
    puts slot w's values at y[w]."""
    for fmt, fmax, maxc, neg1 in (("e4m3fn", 448.0, 0x7E, 0xB8), ("e5m2", 57344.0, 0x7B, 0xBC)):
        s = L.cast_to_packed(np.zeros(8, np.float32), "f32", fmt)
        want_inv = X.f32(X.rn32(Fraction(1) / X.rn32(Fraction(int(fmax)))))
        assert bytes(s[:4]) == np.float32(want_inv).tobytes() and not s[4:].any(), fmt
        s2 = L.cast_to_packed(np.array([fmax, -1.0], np.float32), "f32", fmt)
        assert list(s2) == [0x00, 0x00, 0x80, 0x3F, maxc, neg1], (fmt, list(s2))
        assert list(L.cast_to_packed(np.zeros(0, np.float32), "f32", fmt)) == [0x00, 0x00, 0x80, 0x3F]
        both = np.concatenate([s2, np.array([0, 0, 0, 0x40, maxc, neg1], np.uint8)])   # second scale_inv = 2
        y = np.asarray(L.dequant_packed(both, fmt, 2, 2, "f32"))
        assert y.tolist() == [[fmax, -1.0], [2 * fmax, -2.0]], (fmt, y)


# the exact-rational cast references are the slow ones (seconds each): run last,
# so that a planted mistake caught by a cheaper pin is reported sooner
_SLOW = ("pin_exact_cast_per_group128", "pin_exact_cast_per_tensor", "pin_exact_cast_per_channel")
ALL_PINS = ([v for k, v in sorted(globals().items()) if k.startswith("pin_") and k not in _SLOW]
            + [globals()[k] for k in _SLOW])
