"""Independent references used to pin the CPU oracle.

Nothing here calls the oracle or the HIP library.  Two techniques:

* exact rational arithmetic (``fractions.Fraction``) with a textbook
  round-to-nearest-even onto a binary grid, for end-to-end checks on tiny
  inputs;
* a vectorised nearest-value search over the table of all finite fp8 values,
  for sweeps over hundreds of thousands of binary32 inputs.

Both build the fp8 value tables from the bit-field layout of the OCP 8-bit
floating point formats (E4M3: bias 7, 3 mantissa bits, only S.1111.111 is NaN;
E5M2: bias 15, 2 mantissa bits, exponent field 31 is inf/NaN), not from the
oracle's decoder.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

FMT = {
    # name: (mantissa bits, exponent bits, bias, largest finite magnitude code)
    "e4m3fn": (3, 4, 7, 0x7E),
    "e5m2": (2, 5, 15, 0x7B),
}


def fp8_value(code: int, fmt: str):
    """Exact value of an fp8 code as a Fraction, or 'nan' / 'inf' / '-inf'."""
    mb, eb, bias, maxc = FMT[fmt]
    s = -1 if code & 0x80 else 1
    E = (code >> mb) & ((1 << eb) - 1)
    m = code & ((1 << mb) - 1)
    if (code & 0x7F) > maxc:
        if fmt == "e5m2" and (code & 0x7F) == 0x7C:
            return "inf" if s > 0 else "-inf"
        return "nan"
    if E == 0:
        v = Fraction(m, 1 << mb) * Fraction(2) ** (1 - bias)
    else:
        v = (1 + Fraction(m, 1 << mb)) * Fraction(2) ** (E - bias)
    return s * v


def fp8_table(fmt: str):
    """Finite non-negative values indexed by magnitude code 0..max_code (monotone)."""
    maxc = FMT[fmt][3]
    return [fp8_value(c, fmt) for c in range(maxc + 1)]


def floor_log2(v: Fraction) -> int:
    e = v.numerator.bit_length() - v.denominator.bit_length()
    while Fraction(2) ** e > v:
        e -= 1
    while Fraction(2) ** (e + 1) <= v:
        e += 1
    return e


def round_rne(v: Fraction, precision: int, emin: int) -> Fraction:
    """Round v to the nearest number with `precision` significant bits and
    exponent >= emin (gradual underflow below 2^emin), ties to even."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    q = max(floor_log2(a), emin) - (precision - 1)
    scaled = a / Fraction(2) ** q
    k = scaled.numerator // scaled.denominator
    r = scaled - k
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and k % 2 == 1):
        k += 1
    return sign * k * Fraction(2) ** q


def rn32(v: Fraction) -> Fraction:
    """Round to binary32 (no overflow handling: callers stay in range)."""
    r = round_rne(v, 24, -126)
    assert abs(r) < Fraction(2) ** 128, "rn32 overflow in an exact reference"
    return r


def rn_bf16(v: Fraction) -> Fraction:
    r = round_rne(v, 8, -126)
    assert abs(r) < Fraction(2) ** 128
    return r


def rn_f16(v: Fraction):
    r = round_rne(v, 11, -14)
    if abs(r) >= 65536:
        return "inf" if r > 0 else "-inf"
    return r


def enc_fp8_exact(v: Fraction, negative: bool, fmt: str) -> int:
    """fp8 code of a finite value: RNE onto the fp8 grid, then saturation to
    +-max.  `negative` carries the sign (so that -0 and negative underflow keep it)."""
    mb, eb, bias, maxc = FMT[fmt]
    table = fp8_table(fmt)
    a = abs(v)
    r = round_rne(a, mb + 1, 1 - bias)
    code = maxc if r > table[maxc] else table.index(r)
    return code | (0x80 if negative else 0)


def f32(fr: Fraction) -> np.float32:
    return np.float32(float(fr))


def frac(x) -> Fraction:
    return Fraction(float(x))


# ---------------------------------------------------------------------------
# vectorised nearest-value search (numpy, float64 is exact for these values)
# ---------------------------------------------------------------------------

def nearest_fp8_codes(v: np.ndarray, fmt: str) -> np.ndarray:
    """For finite or infinite binary32 inputs: the fp8 code of the nearest
    finite fp8 value (ties to the even code), saturating to +-max; NaN inputs
    get 0xFF (caller compares NaN by class)."""
    mb, eb, bias, maxc = FMT[fmt]
    table = np.array([float(t) for t in fp8_table(fmt)], dtype=np.float64)
    v = np.asarray(v, dtype=np.float32)
    with np.errstate(invalid="ignore"):
        a = np.abs(v.astype(np.float64))
    nan = np.isnan(a)
    a_ = np.where(nan, 0.0, a)
    i = np.searchsorted(table, a_, side="right") - 1          # table[i] <= a < table[i+1]
    i = np.clip(i, 0, maxc)
    hi_i = np.minimum(i + 1, maxc)
    mid = (table[i] + table[hi_i]) / 2.0                      # exact (few significant bits)
    up = (a_ > mid) | ((a_ == mid) & (hi_i % 2 == 0))
    code = np.where((i < maxc) & up, hi_i, i)
    code = np.where(a_ >= table[maxc], maxc, code)           # saturation (incl. inf)
    code = code | np.where(np.signbit(v), 0x80, 0)
    return np.where(nan, 0xFF, code).astype(np.uint8)


def structured_f32_sweep(low_patterns=(0x0, 0x1, 0x4000, 0x7FFF), top_bits: int = 8) -> np.ndarray:
    """Every sign x every binary32 exponent field x every pattern of the top
    `top_bits` mantissa bits x a few patterns of the remaining low bits.  This
    covers every guard/sticky combination that any rounding position between
    mantissa bit 22 and bit 15 (and, via subnormal exponents, above) can see."""
    low_bits = 23 - top_bits
    s = np.arange(2, dtype=np.uint32)[:, None, None, None] << 31
    e = np.arange(256, dtype=np.uint32)[None, :, None, None] << 23
    t = np.arange(1 << top_bits, dtype=np.uint32)[None, None, :, None] << low_bits
    lo = np.array(low_patterns, dtype=np.uint32)[None, None, None, :] & ((1 << low_bits) - 1)
    u = (s | e | t | lo).reshape(-1)
    return u.view(np.float32)


def random_f32_bits(n: int, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32).view(np.float32)


def fp8_midpoints(fmt: str) -> np.ndarray:
    """Midpoints between adjacent finite fp8 values and their binary32
    neighbours (one ulp either side), both signs."""
    table = [float(t) for t in fp8_table(fmt)]
    mids = np.array([(table[i] + table[i + 1]) / 2 for i in range(len(table) - 1)], dtype=np.float32)
    above = np.nextafter(mids, np.float32(np.inf))
    below = np.nextafter(mids, np.float32(0))
    vals = np.concatenate([mids, above, below, np.array(table, dtype=np.float32)])
    return np.concatenate([vals, -vals])
